"""Device-side error paths, forced from the host, through the C ABI.

The kernels never fault on bad positions or block tables: a sequence whose
position is past its cache capacity is skipped by every kernel (its outputs,
position and hidden state stay as they were) and raises ODA_ERR_CAPACITY; a
block-table entry outside [0, num_blocks) is read as block 0, its rows are
masked out of the softmax, and ODA_ERR_BLOCK is raised.  The other sequences
of the batch are computed exactly as without the fault, and the next step,
with the fault removed, is correct in every sequence (no ticket, queue or
partial is left behind).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import decode_attention, full_index_set, local_index_set

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import conditional_sparse_attention_amd as C
    from _harness import Problem, assert_close_bf16, from_dev_u16, replay_step, to_dev_u16

SENTINEL = 0x7FC1


def small_wl(t0, *, layout="contig", layers=2, seed=31):
    t0 = np.asarray(t0, dtype=np.int64)
    return synth.Workload(f"err-{layout}", layers, 16, 8, 128, len(t0), t0, 2, seed=seed, head_seed=seed + 100,
                          layout=layout, t_cap_slack=40)


def run_forced_full(pr, inp, pos):
    """Step with every sequence forced to the full branch; both outputs start
    as the sentinel.  Returns (oL, oF, h_prev before, h_prev after, pos after)."""
    L, B, Hq, d = pr.wl.layers, pr.wl.batch, pr.wl.hq, pr.wl.head_dim
    pr.upload_step(inp)
    pr.set_force(np.ones(B, np.int8))
    pr.bufs.pos.copy_(torch.from_numpy(pos.astype(np.int32)))
    sentinel = to_dev_u16(np.full((L, B, Hq, d), SENTINEL, dtype=np.uint16))
    pr.bufs.oL.copy_(sentinel)
    pr.bufs.oF.copy_(sentinel)
    h_before = from_dev_u16(pr.bufs.h_prev)
    pr.plan.run()
    torch.cuda.synchronize()
    return (from_dev_u16(pr.bufs.oL), from_dev_u16(pr.bufs.oF), h_before, from_dev_u16(pr.bufs.h_prev),
            pr.bufs.pos.cpu().numpy())


def check_healthy(pr, inp, oL, oF, pos, bs, what):
    """Local and full outputs of the sequences in bs against the oracle."""
    Kh, Vh = pr.host[synth.TAG_K], pr.host[synth.TAG_V]
    for l in range(pr.wl.layers):
        for b in bs:
            p = int(pos[b])
            ref = decode_attention(inp["qL"][l, b], Kh[l, b, :, :p], Vh[l, b, :, :p], inp["kL"][l, b],
                                   inp["vL"][l, b], local_index_set(p + 1, pr.wl.sink, pr.wl.window))
            assert_close_bf16(oL[l, b], ref, f"{what}: local l={l} b={b}")
            ref = decode_attention(inp["qF"][l, b], Kh[l, b, :, :p], Vh[l, b, :, :p], inp["kF"][l, b],
                                   inp["vF"][l, b], full_index_set(p + 1))
            assert_close_bf16(oF[l, b], ref, f"{what}: full l={l} b={b}")


def commit_host(pr, inp, pos, bs):
    """The full branch's staged rows into the host copy of the cache."""
    for b in bs:
        p = int(pos[b])
        for l in range(pr.wl.layers):
            pr.host[synth.TAG_K][l, b, :, p] = inp["kF"][l, b]
            pr.host[synth.TAG_V][l, b, :, p] = inp["vF"][l, b]


def clear_error_word(pr):
    pr.ws[:4].zero_()
    torch.cuda.synchronize()


def test_position_past_capacity_is_skipped_and_reported():
    wl = small_wl([100, 3000, 2052])
    pr = Problem(wl, head_perturb=True)
    t_cap = wl.t_cap
    inp = pr.step_inputs(0)
    pos = wl.t0.copy()
    pos[1] = t_cap  # t = t_cap + 1: one past the capacity
    oL, oF, h_before, h_after, pos_after = run_forced_full(pr, inp, pos)
    err = pr.ws_error_word()
    assert err & C.ODA_ERR_CAPACITY and not err & C.ODA_ERR_BLOCK, err
    # the faulty sequence: nothing written, nothing committed
    assert np.all(oL[:, 1] == SENTINEL) and np.all(oF[:, 1] == SENTINEL)
    assert pos_after[1] == pos[1]
    assert np.array_equal(h_after[1], h_before[1])
    # the others: exact outputs and commits
    check_healthy(pr, inp, oL, oF, pos, [0, 2], "capacity step")
    assert pos_after[0] == pos[0] + 1 and pos_after[2] == pos[2] + 1
    for b in (0, 2):
        assert np.array_equal(h_after[b], oF[wl.layers - 1, b].reshape(-1))
        for l in range(wl.layers):
            ks, vs = pr.cache_slot(l, b, int(pos[b]))
            assert np.array_equal(ks, inp["kF"][l, b]) and np.array_equal(vs, inp["vF"][l, b])
    # next step with the position back in range: every sequence correct
    commit_host(pr, inp, pos, [0, 2])
    pr.bufs.pos.copy_(torch.from_numpy(np.array([pos[0] + 1, wl.t0[1], pos[2] + 1], dtype=np.int32)))
    clear_error_word(pr)
    replay_step(pr, 1, theta=0.0, force=np.array([1, 1, 0], np.int8))


def test_block_table_entry_out_of_range_is_masked_and_reported():
    wl = small_wl([100, 3000, 2052], layout="paged")
    pr = Problem(wl, head_perturb=True)
    bs_ = wl.block_size
    inp = pr.step_inputs(0)
    pos = wl.t0.copy()
    # sequence 1: a block inside its local window (positions 2976..2991) points past the pool
    bad = 2990 // bs_
    good = int(pr.tables_np[1, bad])
    pr.tables[1, bad] = pr.num_blocks
    torch.cuda.synchronize()
    oL, oF, h_before, h_after, pos_after = run_forced_full(pr, inp, pos)
    err = pr.ws_error_word()
    assert err & C.ODA_ERR_BLOCK and not err & C.ODA_ERR_CAPACITY, err
    check_healthy(pr, inp, oL, oF, pos, [0, 2], "block step")
    # the faulty sequence's outputs were written (its masked rows left out) and are finite
    for o in (oL[:, 1], oF[:, 1]):
        assert not np.any(o == SENTINEL)
        assert np.all(np.isfinite((o.astype(np.uint32) << 16).view(np.float32)))
    # its slot 3000 lies in an intact block, so its commit went through
    assert np.array_equal(pos_after, pos + 1)
    for b in range(wl.batch):
        for l in range(wl.layers):
            ks, vs = pr.cache_slot(l, b, int(pos[b]))
            assert np.array_equal(ks, inp["kF"][l, b]) and np.array_equal(vs, inp["vF"][l, b])
    # next step with the table repaired: every sequence correct
    pr.tables[1, bad] = good
    commit_host(pr, inp, pos, range(wl.batch))
    clear_error_word(pr)
    replay_step(pr, 1, theta=0.0, force=np.array([1, 0, 1], np.int8))
