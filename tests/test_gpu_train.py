"""GPU parity of the recall-head training step (include/oda_train.h) against
the training oracle, through the C ABI.  The bars are stated in
tests/_train_harness.py."""
import dataclasses

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import conditional_sparse_attention_amd as C
    from _train_harness import (SCORE_TOL, TrainProblem, check_grad, check_labels, dev, oracle_step)


def _small_vocab_shape(**kw):
    base = dict(name="v1000", hidden=256, vocab=1000, runs=1, rows_per_run=37, first_pos=2040, differ_rate=0.5,
                seed=51, head_seed=151, embed_seed=251, lam=0.0)
    base.update(kw)
    return synth.TrainShape(**base)


def test_labels_ragged_vocab_and_rows():
    """D = 256, V = 1000 (7 full vocabulary tiles and a ragged one), 37 rows
    across the s + w boundary; one row without a reference token and one with
    an id outside the vocabulary (error bit, no reference token)."""
    sh = _small_vocab_shape()
    pos, prev, tok, nxt = synth.train_rows(sh)
    nxt = nxt.copy()
    nxt[5] = -1
    nxt[30] = sh.vocab + 7
    pr = TrainProblem(sh, nxt=nxt)
    pr.labels()
    torch.cuda.synchronize()
    assert pr.err_word() & C.ODA_ERR_TOKEN
    pr.nxt[30] = -1                      # what the library made of it
    worst = check_labels(pr, np.arange(sh.rows))
    v = pr.valid.cpu().numpy()
    assert v[5] == 0 and v[30] == 0 and v[:12].sum() == 0 and v[12:].sum() > 0
    print("worst label error / bound", round(worst, 3))


def test_labels_full_vocabulary_sampled():
    """Qwen3-1.7B hidden size and vocabulary (151,936 rows, 1,187 tiles),
    300 rows (600 hidden rows, a ragged row block); 24 sampled rows against
    the oracle, every row's validity against the position rule."""
    sh = dataclasses.replace(synth.train_shapes()["small"], runs=3, rows_per_run=100, first_pos=2000)
    pr = TrainProblem(sh)
    pr.labels()
    rows = np.random.default_rng(3).choice(sh.rows, 24, replace=False)
    worst = check_labels(pr, rows)
    v = pr.valid.cpu().numpy().astype(bool)
    assert np.array_equal(v, pr.pos >= 2052)
    print("worst label error / bound", round(worst, 3))


def _step_and_compare(pr, valid_np=None, rows=None):
    valid_t = None if valid_np is None else dev(valid_np.astype(np.uint8))
    pr.head_step(valid_t)
    torch.cuda.synchronize()
    valid = pr.valid.cpu().numpy() if valid_np is None else valid_np
    loss, q, grad = oracle_step(pr, valid, rows)
    sel = np.arange(pr.sh.rows) if rows is None else np.asarray(rows)
    q_gpu = pr.score.cpu().numpy()[sel]
    assert np.all(np.abs(q_gpu - q) <= SCORE_TOL * (1 + np.abs(q))), np.max(np.abs(q_gpu - q))
    loss_gpu = float(pr.loss.item())
    assert loss_gpu == pytest.approx(loss, rel=1e-4, abs=1e-7)
    ratios = check_grad(pr.grad.cpu().numpy().astype(np.float64), grad, pr.sh.hidden)
    worst = max(ratios.values())
    print("grad error / bound per tensor:", {k: round(v, 3) for k, v in ratios.items()})
    assert worst <= 1.0, ratios
    return worst


def test_head_step_small_batch():
    """Two runs of 20 rows across the boundary, lambda = 0.001: labels, then
    forward, loss and the whole gradient against the oracle."""
    pr = TrainProblem(synth.train_shapes()["small"])
    pr.labels()
    check_labels(pr, np.arange(pr.sh.rows))
    _step_and_compare(pr)


def test_head_step_sequence_starts_and_hidden_4096():
    """D = 4096 (the 8B shape's towers), rows at sequence starts (previous
    state zero), every row valid by construction of its position."""
    sh = _small_vocab_shape(hidden=4096, rows_per_run=29, first_pos=3000, seed=52, head_seed=152, embed_seed=252)
    pos, prev, tok, nxt = synth.train_rows(sh)
    prev = prev.copy()
    prev[[0, 7, 19]] = -1
    pr = TrainProblem(sh, prev=prev)
    pr.labels()
    _step_and_compare(pr)


def test_head_step_without_valid_rows():
    """No valid row: loss 0 and an all-zero gradient, scores still computed."""
    sh = _small_vocab_shape(rows_per_run=9, first_pos=100)
    pr = TrainProblem(sh)
    pr.labels()
    assert int(pr.valid.sum().item()) == 0
    pr.grad.fill_(7.0)
    _step_and_compare(pr)
    assert float(pr.loss.item()) == 0.0
    assert torch.count_nonzero(pr.grad).item() == 0


def test_head_step_is_deterministic_and_checks_rows():
    """Two runs give identical bits; a previous-row index outside the batch
    raises ODA_ERR_ROW and reads a zero previous state."""
    pr = TrainProblem(synth.train_shapes()["small"])
    pr.labels()
    pr.head_step()
    a = [pr.grad.clone(), pr.score.clone(), pr.loss.clone()]
    pr.head_step()
    for x, y in zip(a, [pr.grad, pr.score, pr.loss]):
        assert torch.equal(x, y)
    assert pr.err_word() == 0
    prev = pr.prev.copy()
    prev[3] = 10_000
    pr2 = TrainProblem(pr.sh, prev=prev)
    pr2.labels()
    pr2.head_step()
    torch.cuda.synchronize()
    assert pr2.err_word() & C.ODA_ERR_ROW
    prev[3] = -1
    pr3 = TrainProblem(pr.sh, prev=prev)
    pr3.labels()
    pr3.head_step()
    assert torch.equal(pr2.score, pr3.score)


def test_full_size_step_sampled():
    """The benchmarked micro-batch (4 x 2048 rows, D = 2048, V = 151,936) in
    the same launch configuration: labels of sampled rows against the oracle,
    then the head step with the valid set cut down to 16 sampled rows, whose
    gradient and scores the oracle recomputes."""
    sh = synth.train_shapes()["qwen3-1.7b-8k"]
    pr = TrainProblem(sh)
    pr.labels()
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(np.flatnonzero(pr.pos >= 2052), 16, replace=False))
    check_labels(pr, rows)
    v = pr.valid.cpu().numpy().astype(bool)
    assert np.array_equal(v, pr.pos >= 2052)
    valid = np.zeros(sh.rows, dtype=np.uint8)
    valid[rows] = 1
    _step_and_compare(pr, valid, rows)


def test_single_row_and_single_token_vocabulary():
    """Degenerate sizes: one row, and a one-row vocabulary (every log-probability
    is 0, so the gain is exactly 0 and the label is -log(1 + lambda))."""
    sh = _small_vocab_shape(vocab=1, rows_per_run=1, first_pos=5000, lam=0.25, seed=53, head_seed=153, embed_seed=253)
    pr = TrainProblem(sh, nxt=np.zeros(1, np.int32), tok=np.zeros(1, np.int32))
    pr.labels()
    torch.cuda.synchronize()
    assert float(pr.gain.item()) == 0.0
    assert float(pr.label.item()) == pytest.approx(-np.log1p(0.25), abs=1e-6)
    assert int(pr.valid.item()) == 1
    _step_and_compare(pr)


def test_single_row_full_head():
    """One row through the full-size head and the full vocabulary."""
    sh = dataclasses.replace(synth.train_shapes()["small"], runs=1, rows_per_run=1, first_pos=2100)
    pr = TrainProblem(sh)
    pr.labels()
    check_labels(pr, [0])
    _step_and_compare(pr)
