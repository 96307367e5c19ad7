"""GPU parity of the recurrent-state transaction of a hybrid backbone
(include/oda_hybrid.h) against the hybrid oracle, through the C ABI.

Bars: recurrent states are fp32 on both sides of a float64 comparison, an
element within STATE_TOL (1 + |ref|) with STATE_TOL = 2e-6 (one step's
arithmetic carries about 1e-7 relative, a few steps compound it; measured
worst 1.8e-7); outputs
are bf16, within one bf16 ulp (2^-7 |ref|) plus 1e-5; convolution states
hold bf16 inputs and must match bit for bit; slot indices bit for bit; the
pre-step slot is never written.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

STATE_TOL = 2e-6
OUT_RTOL = 2.0 ** -7

if torch.cuda.is_available():
    import conditional_sparse_attention_amd as C
    from _harness import Problem, replay_step
    from conditional_sparse_attention_amd.hybrid import GdnBuffers, HybridPlan
    from oracle import hybrid as HY
    from oracle.oda_oracle import bf16_to_f64


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


class GdnProblem:
    """The pool with a seeded pre-step state in each sequence's committed
    slot (the other slots hold a marker value), and the oracle's copy."""

    def __init__(self, sh, slots):
        self.sh = sh
        self.gd = C.make_gdn_dims(sh.layers, sh.batch, sh.heads, sh.d, sh.conv_width)
        self.g = GdnBuffers.allocate(self.gd)
        self.rec, self.conv = self.g.views(self.gd)
        self.rec.fill_(7.0)
        self.conv.fill_(0x40E0)                        # bf16 7.0
        self.g.slot.copy_(torch.tensor(slots, dtype=torch.uint8))
        self.states = []
        for b in range(sh.batch):
            S_l, c_l = [], []
            for l in range(sh.layers):
                S0, c0 = synth.gdn_initial_state(sh, l, b)
                self.rec[l, b, slots[b]] = _dev(S0)
                self.conv[l, b, slots[b]] = _dev(c0.view(np.int16))
                S_l.append(S0.astype(np.float64))
                c_l.append(bf16_to_f64(c0))
            self.states.append(HY.HybridState(S_l, c_l))
        self.w = [synth.gdn_conv_weights(sh, l) for l in range(sh.layers)]
        for l in range(sh.layers):
            self.g.conv_w[l] = _dev(self.w[l].view(np.int16))

    def feed(self, step):
        sh, g = self.sh, self.g
        self.inp = {0: [], 1: []}
        for l in range(sh.layers):
            for br in (0, 1):
                x = synth.gdn_x(sh, l, br, step)
                a, b = synth.gdn_gates(sh, l, br, step)
                (g.xL if br == 0 else g.xF)[l] = _dev(x.view(np.int16))
                (g.aL if br == 0 else g.aF)[l] = _dev(a)
                (g.bL if br == 0 else g.bF)[l] = _dev(b)
                self.inp[br].append((x, a, b))

    def run(self, flags):
        gd, g = self.gd, self.g
        flag = _dev(np.asarray(flags, dtype=np.uint8))
        for l in range(self.sh.layers):
            C.oda_gdn_step(gd, l, C.ODA_GDN_LOCAL, g.state, g.slot, None, g.xL[l], g.conv_w[l], g.aL[l], g.bL[l],
                           g.oL[l])
        for l in range(self.sh.layers):
            C.oda_gdn_step(gd, l, C.ODA_GDN_FULL, g.state, g.slot, flag, g.xF[l], g.conv_w[l], g.aF[l], g.bF[l],
                           g.oF[l])
        C.oda_gdn_commit(gd, g.slot, flag)
        torch.cuda.synchronize()


def _snapshot(pr, seqs):
    old_slot = pr.g.slot.cpu().numpy().copy()
    before = {b: [pr.rec[l, b, old_slot[b]].clone() for l in range(pr.sh.layers)] for b in seqs}
    return old_slot, before


def _check(pr, old_slot, before, flags, seqs):
    """The step just run against the oracle's transaction, for sequences
    `seqs`, given the flags the step took."""
    sh = pr.sh
    new_slot = pr.g.slot.cpu().numpy()
    assert np.array_equal(new_slot, (old_slot + 1 + np.asarray(flags)) % 3)
    oL = pr.g.oL.cpu().numpy().view(np.uint16)
    oF = pr.g.oF.cpu().numpy().view(np.uint16)
    worst = 0.0
    for b in seqs:
        loc = [(x[b], a[b], be[b]) for x, a, be in pr.inp[0]]
        ful = [(x[b], a[b], be[b]) for x, a, be in pr.inp[1]]
        out_l, out_f, new = HY.transaction_step(pr.states[b], loc, ful, pr.w, flags[b])
        for l in range(sh.layers):
            # the pre-step slot is untouched (the full retry restores from it)
            assert torch.equal(pr.rec[l, b, old_slot[b]], before[b][l])
            for got, want in ((oL[l, b], out_l[l]),) + (((oF[l, b], out_f[l]),) if flags[b] else ()):
                g64 = bf16_to_f64(got)
                assert np.all(np.abs(g64 - want) <= OUT_RTOL * np.abs(want) + 1e-5), (b, l)
            S = pr.rec[l, b, new_slot[b]].cpu().numpy().astype(np.float64)
            err = np.abs(S - new.S[l]) / (STATE_TOL * (1 + np.abs(new.S[l])))
            worst = max(worst, float(err.max()))
            conv = pr.conv[l, b, new_slot[b]].cpu().numpy().view(np.uint16)
            assert np.array_equal(bf16_to_f64(conv), new.conv[l]), (b, l)
        pr.states[b] = new
    assert worst <= 1.0, worst
    return worst


def _step_and_check(pr, step, flags, seqs=None):
    seqs = range(pr.sh.batch) if seqs is None else seqs
    old_slot, before = _snapshot(pr, seqs)
    pr.feed(step)
    pr.run(flags)
    return _check(pr, old_slot, before, flags, seqs)


@pytest.mark.parametrize("width", [4, 2, 3, 6])
def test_transaction_small_three_steps(width):
    """3 recurrent layers (the first shared by both branches), 5 sequences
    with committed slots 0, 1, 2, 0, 1, three steps with different flags:
    outputs, the committed state of each layer and the slot indices against
    the oracle's save / restore / commit; convolution widths 4 (the Qwen
    hybrid family's), 2, 3 and 6."""
    sh = synth.GdnShape(layers=3, batch=5, heads=4, shared_layers=1, seed=71, conv_width=width)
    pr = GdnProblem(sh, [0, 1, 2, 0, 1])
    worst = 0.0
    for step, flags in enumerate(([1, 0, 1, 1, 0], [0, 0, 0, 0, 0], [1, 1, 1, 1, 1])):
        worst = max(worst, _step_and_check(pr, step, flags))
    print("worst state error / bound", round(worst, 4))


def test_shared_layer_branches_agree_bitwise():
    """Where both branches see the same inputs (recurrent layers before the
    first attention layer) the full retry from the restored state equals the
    local trial bit for bit."""
    sh = synth.GdnShape(layers=2, batch=3, heads=2, shared_layers=2, seed=72)
    pr = GdnProblem(sh, [2, 0, 1])
    pr.feed(0)
    slot = pr.g.slot.cpu().numpy().copy()
    pr.run([1, 1, 1])
    for l in range(2):
        for b in range(3):
            assert torch.equal(pr.rec[l, b, (slot[b] + 1) % 3], pr.rec[l, b, (slot[b] + 2) % 3])
            assert torch.equal(pr.conv[l, b, (slot[b] + 1) % 3], pr.conv[l, b, (slot[b] + 2) % 3])
        assert torch.equal(pr.g.oL[l], pr.g.oF[l])


def test_full_size_sampled_sequences():
    """The benchmarked shape (18 recurrent layers, 16 heads, 8 sequences):
    two steps, the oracle following two sampled sequences through every
    layer."""
    sh = synth.GdnShape(layers=18, batch=8, heads=16, seed=73)
    pr = GdnProblem(sh, [0, 1, 2, 0, 1, 2, 0, 1])
    worst = 0.0
    for step, flags in enumerate(([1, 0, 0, 1, 0, 1, 1, 0], [0, 1, 1, 0, 0, 1, 0, 1])):
        worst = max(worst, _step_and_check(pr, step, flags, seqs=[3, 6]))
    print("worst state error / bound", round(worst, 4))


@pytest.mark.parametrize("layout", ["contig", "paged"])
def test_hybrid_step_with_the_head_deciding(layout):
    """The whole hybrid step through HybridPlan (pattern GGGA GGGA: 6
    recurrent and 2 attention layers, 3 sequences across the s + w
    boundary), with a contiguous and a paged KV cache: the attention path,
    rule, work list and KV commit against the oracle as for the
    attention-only step, and the recurrent states against the oracle's
    transaction under the flags the step took (forced full / local at steps
    0 and 1, decided by the head at steps 2 and 3)."""
    wl = synth.Workload("hybrid-small", 2, 16, 8, 128, 3, np.array([60, 2100, 2600]), 4, seed=81, head_seed=181,
                        layout=layout)
    pr = Problem(wl)
    gp = GdnProblem(synth.GdnShape(layers=6, batch=3, heads=4, seed=82), [0, 1, 2])
    hp = HybridPlan(pr.plan, gp.gd, gp.g, "GGGAGGGA")
    pr.plan.run = hp.run
    forces = [np.ones(3, np.int8), np.zeros(3, np.int8), None, None]
    seen = set()
    for j, f in enumerate(forces):
        gp.feed(j)
        old_slot, before = _snapshot(gp, range(3))
        rec = replay_step(pr, j, theta=0.0, force=f)
        flags = [int(x) for x in rec["flag"]]
        seen.update(flags)
        _check(gp, old_slot, before, flags, range(3))
    assert seen == {0, 1}


def test_one_sequence_one_head_widest_convolution():
    """Degenerate sizes: one sequence, one head, one layer, convolution width
    8 (the largest supported), committed slot 2, two steps."""
    sh = synth.GdnShape(layers=1, batch=1, heads=1, shared_layers=0, seed=74, conv_width=8)
    pr = GdnProblem(sh, [2])
    for step, flags in enumerate(([1], [0])):
        _step_and_check(pr, step, flags)


@pytest.mark.parametrize("batch,heads", [(1024, 1), (1, 64)])
def test_largest_batch_and_head_count(batch, heads):
    """The largest batch (1024 sequences) and the most heads (64) the
    library takes, one layer, two steps with complementary flags: slot
    indices of every sequence, and outputs and states of sampled sequences
    against the oracle."""
    sh = synth.GdnShape(layers=1, batch=batch, heads=heads, shared_layers=0, seed=75)
    pr = GdnProblem(sh, [b % 3 for b in range(batch)])
    seqs = [0, batch // 2, batch - 1] if batch > 1 else [0]
    flags0 = [(b * 7 + 1) % 2 for b in range(batch)]
    for step, flags in enumerate((flags0, [1 - f for f in flags0])):
        _step_and_check(pr, step, flags, seqs=seqs)
