"""Pins of the training-step oracle (On-Demand Attention notes, §2.1 equation
for the gain g; §2.2 equations for d, y, the Huber loss and the paragraph on
paired supervision).

* Labels: log-probabilities against closed forms of one-hot LM heads, the
  softmax normalisation, the sign and antisymmetry of g, and the valid-set
  rule at the s + w boundary.
* Previous-state selection: hand cases.
* The head's backward pass against central finite differences of the
  forward, for every parameter of a small head, with rows in both Huber
  regimes and rows outside the valid set; the output-bias gradient against
  its closed form; a perfect fit and an empty valid set.
* The batched forward against the decode step's per-row recall score.
"""
import math

import numpy as np
import pytest

import synth
from oracle import benefit_label, recall_score, unpack_head
from oracle import train as T
from oracle.oda_oracle import bf16_to_f64, f64_to_bf16

D, TW, FF = 16, 8, 12


def _one_hot_head(V, Dm):
    """E with E[k] = unit vector k for k < Dm and zero rows after (bf16 bits)."""
    E = np.zeros((V, Dm))
    E[np.arange(min(V, Dm)), np.arange(min(V, Dm))] = 1.0
    return f64_to_bf16(E)


def test_log_prob_one_hot_closed_form():
    V, Dm, c = 40, 8, 3.0
    E = bf16_to_f64(_one_hot_head(V, Dm))
    h = np.zeros(Dm)
    h[5] = c
    Z = math.exp(c) + V - 1
    assert T.log_prob(E, h, 5) == pytest.approx(c - math.log(Z), abs=1e-13)
    assert T.log_prob(E, h, 7) == pytest.approx(-math.log(Z), abs=1e-13)
    assert T.log_prob(E, h, 30) == pytest.approx(-math.log(Z), abs=1e-13)
    # a zero hidden state gives the uniform distribution
    assert T.log_prob(E, np.zeros(Dm), 11) == pytest.approx(-math.log(V), abs=1e-13)


def test_log_prob_normalised_and_shift_invariant():
    rng = np.random.default_rng(3)
    E = rng.normal(size=(50, 6))
    h = rng.normal(size=6) * 4
    p = np.exp([T.log_prob(E, h, x) for x in range(50)])
    assert p.sum() == pytest.approx(1.0, abs=1e-12)
    # logits large enough to overflow a naive exp stay finite
    assert math.isfinite(T.log_prob(E, h * 300, 0))


def test_gain_sign_and_antisymmetry():
    V, Dm = 40, 8
    Eb = _one_hot_head(V, Dm)
    E = bf16_to_f64(Eb)
    hf = np.zeros(Dm)
    hf[2] = 3.0
    hl = np.zeros(Dm)
    g = T.gain(E, hf, hl, 2)
    assert g == pytest.approx(3.0 - math.log(math.exp(3.0) + V - 1) + math.log(V), abs=1e-13)
    assert g > 0                                  # the full state puts more mass on the reference
    assert T.gain(E, hl, hf, 2) == pytest.approx(-g, abs=1e-14)
    assert T.gain(E, hf, hf, 2) == 0.0            # identical candidates: no benefit


def test_labels_valid_set_and_label_values():
    V, Dm = 40, 8
    Eb = _one_hot_head(V, Dm)
    rng = np.random.default_rng(5)
    hl = f64_to_bf16(rng.normal(size=(5, Dm)))
    hf = f64_to_bf16(rng.normal(size=(5, Dm)))
    pos = np.array([2050, 2051, 2052, 9000, 9001])
    nxt = np.array([1, 2, 3, 4, -1])
    lam = 0.25
    g, y, valid = T.labels(Eb, hl, hf, nxt, pos, lam)
    # t = pos + 1 must exceed s + w = 2052: pos 2052 is the first valid position
    assert valid.tolist() == [False, False, True, True, False]
    E = bf16_to_f64(Eb)
    for i in range(4):
        hF = bf16_to_f64(hf[i])
        hL = bf16_to_f64(hl[i])
        assert g[i] == pytest.approx(T.log_prob(E, hF, nxt[i]) - T.log_prob(E, hL, nxt[i]), abs=1e-13)
        assert y[i] == pytest.approx(benefit_label(g[i], lam), abs=1e-15)
    assert g[4] == 0.0 and y[4] == 0.0


def test_prev_hidden_hand_cases():
    hl = np.arange(12, dtype=np.float64).reshape(4, 3)
    hf = -hl - 1
    g = np.array([0.5, 0.1, math.nan, -2.0])
    lam = 0.1
    prev = np.array([-1, 0, 1, 2])
    out = T.prev_hidden(hl, hf, prev, g, lam)
    assert np.array_equal(out[0], np.zeros(3))        # sequence start
    assert np.array_equal(out[1], hf[0])              # d = 0.4 > 0: full
    assert np.array_equal(out[2], hl[1])              # d = 0: not above zero, local
    assert np.array_equal(out[3], hf[2])              # non-finite: full


def _tiny_problem(seed=11, n=14):
    rng = np.random.default_rng(seed)
    blob = synth.head_blob(D, seed, perturb=True, tower=TW, ffn=FF).astype(np.float64)
    Hp = rng.normal(size=(n, D))
    Hp[0] = 0.0                                       # a sequence start: zero previous state
    Em = rng.normal(size=(n, D)) * 0.5
    HL = rng.normal(size=(n, D)) * 2.0
    P = T.unpack(blob, D, TW, FF)
    q, _ = T.head_forward(P, Hp, Em, HL)
    # labels that put residuals in both Huber regimes, away from the kink
    off = np.array([0.3, -0.6, 2.5, -3.0, 0.05, 1.7, -1.4, 0.8, -0.2, 4.0, -0.9, 0.45, 1.2, -2.2])[:n]
    y = q - off
    valid = np.ones(n, dtype=bool)
    valid[[3, 8]] = False
    return blob, Hp, Em, HL, y, valid


def test_backward_matches_finite_differences():
    blob, Hp, Em, HL, y, valid = _tiny_problem()
    P = T.unpack(blob, D, TW, FF)
    q, cache = T.head_forward(P, Hp, Em, HL)
    r = q - y
    assert np.min(np.abs(np.abs(r) - 1.0)) > 1e-3
    _, dq = T.loss_and_dq(q, y, valid)
    grad = T.pack(T.head_backward(P, cache, dq), D, TW, FF)
    assert grad.size == blob.size
    h = 1e-5
    fd = np.empty_like(grad)
    for i in range(blob.size):
        bp, bm = blob.copy(), blob.copy()
        bp[i] += h
        bm[i] -= h
        fd[i] = (T.loss_of(bp, D, Hp, Em, HL, y, valid, TW, FF) -
                 T.loss_of(bm, D, Hp, Em, HL, y, valid, TW, FF)) / (2 * h)
    scale = np.max(np.abs(fd))
    err = np.abs(grad - fd)
    assert np.max(err) <= 1e-6 * scale, (np.argmax(err), np.max(err), scale)
    # every tensor receives a gradient
    at = 0
    for name, shape in T.head_layout(D, TW, FF):
        k = int(np.prod(shape))
        assert np.any(grad[at:at + k] != 0.0), name
        at += k


def test_output_bias_gradient_closed_form():
    blob, Hp, Em, HL, y, valid = _tiny_problem(seed=12)
    P = T.unpack(blob, D, TW, FF)
    q, cache = T.head_forward(P, Hp, Em, HL)
    _, dq = T.loss_and_dq(q, y, valid)
    G = T.head_backward(P, cache, dq)
    r = (q - y)[valid]
    want = np.mean(np.clip(r, -1.0, 1.0))             # d Huber_1 / dr = clip(r, -1, 1)
    assert G["c_o"][0] == pytest.approx(want, abs=1e-14)


def test_loss_values_and_degenerate_batches():
    blob, Hp, Em, HL, y, valid = _tiny_problem(seed=13)
    P = T.unpack(blob, D, TW, FF)
    q, cache = T.head_forward(P, Hp, Em, HL)
    loss, _ = T.loss_and_dq(q, y, valid)
    r = (q - y)[valid]
    want = np.mean([0.5 * x * x if abs(x) <= 1 else abs(x) - 0.5 for x in r])
    assert loss == pytest.approx(want, abs=1e-14)
    # perfect labels: zero loss, zero gradient
    loss0, dq0 = T.loss_and_dq(q, q.copy(), valid)
    assert loss0 == 0.0
    g0 = T.pack(T.head_backward(P, cache, dq0), D, TW, FF)
    assert np.all(g0 == 0.0)
    # no valid rows: zero loss, zero gradient
    lossn, dqn = T.loss_and_dq(q, y, np.zeros_like(valid))
    assert lossn == 0.0 and np.all(dqn == 0.0)


def test_batched_forward_matches_decode_score():
    blob, Hp, Em, HL, _, _ = _tiny_problem(seed=14)
    P = T.unpack(blob, D, TW, FF)
    q, _ = T.head_forward(P, Hp, Em, HL)
    Pd = unpack_head(blob.astype(np.float32), D, TW, FF)
    for i in range(len(q)):
        assert q[i] == pytest.approx(recall_score(Pd, Hp[i], Em[i], HL[i]), rel=1e-12, abs=1e-12)


def test_train_step_wires_labels_prev_and_embedding():
    """head_train_step gathers E[x_t], picks h_prev by the previous row's gain
    and differentiates the mean Huber loss: equal to the finite differences
    of the loss built from those pieces by hand."""
    rng = np.random.default_rng(21)
    V, n = 30, 6
    Eb = f64_to_bf16(rng.normal(size=(V, D)))
    hl = f64_to_bf16(rng.normal(size=(n, D)))
    hf = f64_to_bf16(rng.normal(size=(n, D)))
    tok = rng.integers(0, V, size=n)
    nxt = rng.integers(0, V, size=n)
    pos = np.arange(2050, 2050 + n)
    prev = np.array([-1, 0, 1, 2, 3, 4])
    lam = 0.05
    g, y, valid = T.labels(Eb, hl, hf, nxt, pos, lam)
    blob = synth.head_blob(D, 22, perturb=True, tower=TW, ffn=FF)
    loss, q, grad = T.head_train_step(blob, D, Eb, hl, hf, tok, prev, g, y, valid, lam, TW, FF)
    E = bf16_to_f64(Eb)
    HL = bf16_to_f64(hl)
    HF = bf16_to_f64(hf)
    Hp = np.zeros((n, D))
    for i in range(1, n):
        Hp[i] = HF[i - 1] if g[i - 1] - lam > 0 else HL[i - 1]
    b64 = blob.astype(np.float64)
    assert loss == pytest.approx(T.loss_of(b64, D, Hp, E[tok], HL, y, valid, TW, FF), abs=1e-14)
    for i in np.random.default_rng(0).choice(blob.size, 60, replace=False):
        bp, bm = b64.copy(), b64.copy()
        bp[i] += 1e-5
        bm[i] -= 1e-5
        fd = (T.loss_of(bp, D, Hp, E[tok], HL, y, valid, TW, FF) -
              T.loss_of(bm, D, Hp, E[tok], HL, y, valid, TW, FF)) / 2e-5
        assert grad[i] == pytest.approx(fd, abs=1e-7 * max(1.0, abs(fd)))
