"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bars (float tolerances are those the workload definition states):
  index sets, flags outside |q - theta| < 1e-3, work list, commit: bit-exact;
  bf16 attention outputs: |gpu - oracle| <= 1e-2 + 1e-2 |oracle|;
  recall scores: |gpu - oracle| <= 1e-4 (1 + |oracle|).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import branch_rule, local_index_set, recall_score, unpack_head

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import conditional_sparse_attention_amd as C
    from _harness import Problem, replay_step, to_dev_u16, from_dev_u16


def small_wl(t0, *, layers=2, hq=16, hkv=8, steps=3, layout="contig", seed=11, needles=()):
    t0 = np.asarray(t0, dtype=np.int64)
    return synth.Workload(f"small-{hq}-{hkv}-{layout}", layers, hq, hkv, 128, len(t0), t0, steps, seed=seed,
                          head_seed=seed + 100, layout=layout, needles=needles, t_cap_slack=40)


def test_local_ranges_bitexact():
    pos = np.array([0, 1, 2, 3, 4, 5, 100, 2046, 2047, 2048, 2049, 2050, 2051, 2052, 2053, 2054, 4095,
                    4096, 65535, 131071, 131072, 200000, 7, 9, 11, 13, 2100, 3000, 1 << 20, 17, 19, 23],
                   dtype=np.int32)
    dims = C.make_dims(1, len(pos), 16, 8, t_cap=1 << 21)
    ranges = torch.zeros((len(pos), 4), dtype=torch.int32, device="cuda")
    C.oda_local_ranges(dims, torch.from_numpy(pos).cuda(), ranges)
    r = ranges.cpu().numpy()
    for b, p in enumerate(pos):
        got = np.concatenate([np.arange(r[b, 0], r[b, 1]), np.arange(r[b, 2], r[b, 3])])
        assert np.array_equal(got, local_index_set(int(p) + 1)), (p, r[b])


@pytest.mark.parametrize("layout", ["contig", "paged"])
@pytest.mark.parametrize("hq,hkv", [(16, 8), (32, 8), (8, 8)])
def test_ragged_batch_forced_and_head(layout, hq, hkv):
    """Ragged lengths spanning t = 1, the sink/window boundary (2052/2053),
    several full-branch splits and a ragged tail; step 0 forces every
    sequence to the full branch, step 1 forces local, step 2 lets the head
    decide."""
    wl = small_wl([0, 4, 2051, 2052, 2999, 4600], hq=hq, hkv=hkv, layout=layout)
    pr = Problem(wl, head_perturb=True)
    B = wl.batch
    replay_step(pr, 0, theta=0.0, force=np.ones(B, np.int8))
    replay_step(pr, 1, theta=0.0, force=np.zeros(B, np.int8))
    replay_step(pr, 2, theta=0.0)


def test_full_branch_units_past_one_round():
    """17 flagged sequences x 16 KV heads make more units than one round of
    the full kernel's persistent grid, even at one split each: the units past
    the first round come from the kernel's device-side queue, largest first.
    Two layers and two all-flagged steps check that the queue starts from
    zero at every launch (ragged lengths across t = 2052 / 2053)."""
    wl = small_wl([2600, 2100, 300, 2052, 2053, 1500, 900, 2400, 64, 1999, 2222, 777, 1234, 2500, 1800, 1,
                   2049], hq=16, hkv=16)
    pr = Problem(wl, head_perturb=True)
    B = wl.batch
    for j in range(2):
        replay_step(pr, j, theta=0.0, force=np.ones(B, np.int8))
    units = sum(n for (_, n, s) in pr.worklist() if s == 0) * wl.hkv
    assert units > 256, units


def test_single_key_output_is_value_exactly():
    """t = 1: the index set holds only the current token, so o = v_cur
    exactly (bit-exact after the bf16 round trip)."""
    wl = small_wl([0, 0, 0], layers=1, steps=1)
    pr = Problem(wl)
    inp = pr.step_inputs(0)
    pr.upload_step(inp)
    pr.set_force(np.ones(wl.batch, np.int8))
    pr.plan.run()
    torch.cuda.synchronize()
    oL = from_dev_u16(pr.bufs.oL)[0]
    oF = from_dev_u16(pr.bufs.oF)[0]
    for h in range(wl.hq):
        g = h // (wl.hq // wl.hkv)
        assert np.array_equal(oL[:, h], inp["vL"][0][:, g])
        assert np.array_equal(oF[:, h], inp["vF"][0][:, g])


def test_config1_replay_all_steps():
    """Workload 1 (one layer, 16/8 heads, batch 1, 4096 context, three
    needles, 64 steps, random Xavier head, theta = 0) replayed step by step."""
    wl = synth.workloads()[1]
    pr = Problem(wl)
    nflag = 0
    for j in range(wl.steps):
        rec = replay_step(pr, j, theta=0.0)
        nflag += int(rec["flag"].sum())
    print(f"config 1: {nflag} of {wl.steps} steps took the full branch")


def test_nonfinite_scores_force_full():
    """A non-finite score sends the sequence to the full branch: NaN and +Inf
    planted in the embedding of two sequences make their scores non-finite."""
    wl = small_wl([100, 3000, 5000], layers=1, steps=1)
    pr = Problem(wl)
    inp = pr.step_inputs(0)
    inp["emb"] = inp["emb"].copy()
    inp["emb"][0, 7] = 0x7FC0   # NaN
    inp["emb"][2, 9] = 0x7F80   # +Inf
    pr.upload_step(inp)
    pr.set_force(np.full(wl.batch, -1, np.int8))
    pr.plan.set_theta(1e30)
    pr.plan.run()
    torch.cuda.synchronize()
    score = pr.bufs.score.cpu().numpy()
    flag = pr.bufs.flag.cpu().numpy()
    assert not np.isfinite(score[0]) and not np.isfinite(score[2]) and np.isfinite(score[1])
    assert flag.tolist() == [1, 0, 1]


def test_two_runs_bit_identical():
    """Determinism (and a race check): the same step from the same state
    twice gives identical outputs, scores, flags and commits."""
    wl = small_wl([10, 2100, 5000], layers=2, steps=1)
    outs = []
    for _ in range(2):
        pr = Problem(wl, head_perturb=True)
        inp = pr.step_inputs(0)
        pr.upload_step(inp)
        pr.set_force(np.array([1, -1, 1], np.int8))
        pr.plan.run()
        torch.cuda.synchronize()
        outs.append([from_dev_u16(pr.bufs.oL), from_dev_u16(pr.bufs.oF), pr.bufs.score.cpu().numpy(),
                     pr.bufs.flag.cpu().numpy(), from_dev_u16(pr.bufs.h_prev), pr.K.cpu().numpy()])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_device_generator_matches_host():
    """Device G (synth/csrc/fill.hip) reproduces host G bit for bit."""
    import synth.device as sd
    wl = small_wl([37, 1000, 2500], layers=2, needles=(5, 900))
    pr = Problem(wl, host_cache=True)
    K2 = torch.zeros_like(pr.K)
    V2 = torch.zeros_like(pr.V)
    sd.fill_cache(K2, wl, synth.TAG_K, pr.t0_dev)
    sd.fill_cache(V2, wl, synth.TAG_V, pr.t0_dev)
    assert torch.equal(K2, pr.K) and torch.equal(V2, pr.V)
    bufs = {k: torch.zeros_like(getattr(pr.bufs, k)) for k in ("qL", "qF", "kL", "vL", "kF", "vF")}
    bufs["e"] = torch.zeros_like(pr.bufs.emb)
    for j in (0, 3, 8):
        pos = pr.t0_dev + j
        sd.fill_step(bufs, wl, pos, pr.t0_dev)
        inp = pr.step_inputs(j)
        for k in ("qL", "qF", "kL", "vL", "kF", "vF"):
            assert np.array_equal(from_dev_u16(bufs[k]), inp[k]), (j, k)
        assert np.array_equal(from_dev_u16(bufs["e"]), inp["emb"])


def test_device_generator_paged_matches_contig():
    import synth.device as sd
    wl = small_wl([37, 1000, 2500], layers=2, layout="paged", needles=(5, 900))
    pr = Problem(wl, host_cache=True)
    K2 = torch.zeros_like(pr.K)
    sd.fill_cache(K2, wl, synth.TAG_K, pr.t0_dev, tables=pr.tables, num_blocks=pr.num_blocks)
    assert torch.equal(K2, pr.K)


def test_worklist_entry_point_bitexact():
    """oda_worklist (compaction from caller flags) writes the same list as
    the oracle's work list, with the split counts of the policy, for ragged
    positions (long, and short enough for the finer splits), mixed flags,
    one flag and none, at 2, 4 and 8 KV heads."""
    from _harness import decode_items, want_worklist
    rng = np.random.default_rng(5)
    cases = []
    for B in (1, 7, 32):
        for top in (200000, 9000):
            cases.append((B, rng.integers(0, top, size=B), rng.integers(0, 2, size=B)))
        one = np.zeros(B, np.int64)
        one[B // 2] = 1
        cases.append((B, rng.integers(0, 5000, size=B), one))
    cases.append((5, rng.integers(0, 5000, size=5), np.zeros(5, np.int64)))
    for hq, hkv in ((16, 8), (16, 4), (4, 2)):
        for B, pos, flags in cases:
            pos = pos.astype(np.int32)
            flags = flags.astype(np.uint8)
            dims = C.make_dims(2, B, hq, hkv, t_cap=1 << 18)
            ws = torch.zeros(C.oda_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
            C.oda_workspace_init(dims, ws)
            C.oda_worklist(dims, torch.from_numpy(flags).cuda(), torch.from_numpy(pos).cuda(), ws)
            torch.cuda.synchronize()
            off = C.oda_workspace_worklist_offset(dims)
            w = ws[off:].view(torch.int32).cpu().numpy()
            assert decode_items(w[1:1 + w[0]]) == want_worklist(flags, pos.astype(np.int64) + 1, hkv), (hkv, B)


@pytest.mark.parametrize("B,hq", [(1, 16), (4, 16), (5, 8), (6, 32), (7, 16), (8, 16), (9, 8), (16, 32), (17, 16),
                                  (32, 8), (32, 32), (24, 16)])
def test_recall_head_batch_sizes(B, hq):
    """oda_recall_score alone, on both sides of the switch from the
    bandwidth-shaped GEMV (up to 6 sequences: batch widths 1, 2, 4 and 8) to
    the fp32 MFMA GEMMs (7 and up: one 16-wide column group through 16, two
    from 17), at D = 1024, 2048 and 4096, with a perturbed head so every bias
    and gain term counts.
    Scores to 1e-4 (1 + |q|); flags bit-exact outside the tie band; the work
    list bit-exact against the oracle's for the GPU's flags."""
    from _harness import SCORE_TOL, TIE_BAND, decode_items, want_worklist
    D = hq * 128
    seed = 40 + B
    blob = synth.head_blob(D, seed, perturb=True)
    P = unpack_head(blob, D)
    idx = np.arange(B * D)
    xs = [synth.bf16_at(seed, tag, idx).reshape(B, D) for tag in (synth.TAG_H0, synth.TAG_E, synth.TAG_QL)]
    pos = synth.word32_at(seed, synth.TAG_LEN, np.arange(B)).astype(np.int64) % 150000
    pos = pos.astype(np.int32)
    force = np.full(B, -1, np.int8)
    force[::5] = 1
    dims = C.make_dims(1, B, hq, 8, t_cap=1 << 18)
    ws = torch.zeros(C.oda_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    C.oda_workspace_init(dims, ws)
    dev = [to_dev_u16(x) for x in xs]
    w = torch.from_numpy(blob).cuda()
    score = torch.zeros(B, dtype=torch.float32, device="cuda")
    flag = torch.zeros(B, dtype=torch.uint8, device="cuda")
    qs = np.array([recall_score(P, xs[0][b], xs[1][b], xs[2][b]) for b in range(B)])
    theta = float(np.median(qs))
    for rep in range(2):  # the second call reuses the zeroed tickets of the first
        C.oda_recall_score(dims, w, dev[0], dev[1], dev[2], theta, torch.from_numpy(force).cuda(),
                           torch.from_numpy(pos).cuda(), score, flag, ws)
        torch.cuda.synchronize()
        got = score.cpu().numpy().astype(np.float64)
        err = np.abs(got - qs)
        assert np.all(err <= SCORE_TOL * (1 + np.abs(qs))), (rep, float(np.max(err / (1 + np.abs(qs)))))
        f = flag.cpu().numpy()
        for b in range(B):
            want = branch_rule(qs[b], theta, int(force[b]))
            if force[b] >= 0 or abs(qs[b] - theta) >= TIE_BAND:
                assert f[b] == want, (b, qs[b], theta)
        off = C.oda_workspace_worklist_offset(dims)
        wl_ = ws[off:].view(torch.int32).cpu().numpy()
        assert decode_items(wl_[1:1 + wl_[0]]) == want_worklist(f, pos.astype(np.int64) + 1, 8)
