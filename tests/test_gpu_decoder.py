"""GPU parity of the decoder step around the ODA path (include/oda_decoder.h)
against the decoder oracle, through the C ABI.  The bars are stated in
tests/_dec_harness.py."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import conditional_sparse_attention_amd as C
    import synth.device as sd
    from _dec_harness import DecProblem, layerwise_check, replay_dec_step, u16


def test_device_decoder_weights_match_host():
    """The device generator writes the host generator's decoder weights, bit
    for bit: every element of a tiny model, sampled elements of the full-size
    one."""
    sh = synth.decoder_shapes()["tiny"]
    dd = C.make_dec_dims(C.make_dims(sh.layers, 1, sh.hq, sh.hkv, t_cap=64), sh.inter, sh.vocab)
    blob = torch.zeros(C.oda_dec_layer_numel(dd), dtype=torch.int16, device="cuda")
    for l in range(sh.layers):
        sd.fill_dec_layer(blob, 21, sh, l, perturb=True)
        assert np.array_equal(u16(blob), synth.dec_layer_blob(21, sh, l, perturb=True))
    E = torch.zeros((sh.vocab, sh.hidden), dtype=torch.int16, device="cuda")
    sd.fill_dec_embed(E, 21)
    assert np.array_equal(u16(E), synth.dec_embed_bits(21, sh, np.arange(sh.vocab)))
    big = synth.decoder_shapes()["qwen3-1.7b"]
    n = big.inter * big.hidden
    W = torch.zeros(n, dtype=torch.int16, device="cuda")
    sd.fill_dec_matrix(W, 22, synth.dec_tensor_id(27, "W_down"))
    idx = np.random.default_rng(1).integers(0, n, size=200000)
    assert np.array_equal(u16(W)[idx], synth.dec_matrix_bits(22, synth.dec_tensor_id(27, "W_down"), idx))


def test_decoder_tiny_replay():
    """Tiny decoder (2 layers, 8/4 heads, D = 1024, MLP 2048, vocabulary 4096,
    perturbed gains) on ragged contexts across the sink/window boundary:
    step 0 forces every sequence full, step 1 local, then the head decides."""
    pr = DecProblem("tiny", [100, 2052, 2100, 3000], steps=5, seed=31)
    forces = [np.ones(4, np.int8), np.zeros(4, np.int8), None, None, None]
    worst = {"h": 0.0, "kv": 0.0}
    for j, f in enumerate(forces):
        rec = replay_dec_step(pr, theta=0.0, force=f)
        for k in worst:
            worst[k] = max(worst[k], rec["worst"][k])
        print(f"step {j}: flags {rec['flag'].tolist()} tokens {rec['tokens'].tolist()}")
    print("worst |err| / tolerance:", worst)


def test_decoder_step_is_deterministic_and_graph_capturable():
    """Two problems from the same seeds give identical bits, eager or replayed
    from a captured HIP graph; the graph replays three steps in a row."""
    outs = []
    for use_graph in (False, True):
        pr = DecProblem("tiny", [50, 2500], steps=4, seed=41)
        pr.bufs.force.copy_(torch.tensor([1, -1], dtype=torch.int8))
        s = torch.cuda.Stream()
        if use_graph:
            from conditional_sparse_attention_amd.decoder import DecoderPlan
            with torch.cuda.stream(s):
                plan = DecoderPlan(pr.dd, pr.kv, pr.weights, pr.bufs, pr.ws, pr.dws, theta=0.0, stream=s)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    plan.run()
                # capture records the work without running it: the state is still the start state
                for _ in range(3):
                    g.replay()
                    torch.cuda.synchronize()
        else:
            for _ in range(3):
                pr.plan.run()
        torch.cuda.synchronize()
        outs.append([u16(pr.bufs.hL), u16(pr.bufs.hF), pr.bufs.tokens.cpu().numpy(), pr.bufs.pos.cpu().numpy(),
                     u16(pr.bufs.h_prev), u16(pr.K), u16(pr.V)])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_always_full_matches_forced_full():
    """The always-full step (no local branch, no head) and an ODA step forced
    to the full branch run the same full-branch kernels on the same inputs:
    identical tokens, hidden states and commits."""
    res = []
    for mode in ("forced", "always"):
        pr = DecProblem("tiny", [300, 2600, 4000], steps=2, seed=51)
        if mode == "forced":
            pr.bufs.force.copy_(torch.ones(3, dtype=torch.int8))
            pr.plan.run()
        else:
            pr.plan.run_always_full(torch.ones(3, dtype=torch.uint8, device="cuda"))
        torch.cuda.synchronize()
        res.append([u16(pr.bufs.hF), pr.bufs.tokens.cpu().numpy(), u16(pr.bufs.h_prev), u16(pr.K), u16(pr.V)])
    for a, b in zip(*res):
        assert np.array_equal(a, b)


def test_decoder_full_size_layerwise():
    """Qwen3-1.7B-shaped decoder (28 layers, 16/8 heads, D = 2048, MLP 6144,
    vocabulary 151,936; device-generated weights, checked against the host
    generator above), one step of two sequences, the second flagged: every
    layer of both branches checked against the oracle's layer on the GPU's
    own input of that layer, then the final hidden states and the next token
    over the whole vocabulary.  (Across 28 layers one-ulp rounding
    differences compound, so the full depth is checked layer by layer.)"""
    pr = DecProblem("qwen3-1.7b", [1500, 3000], steps=1, seed=61, device_weights=True, perturb=True)
    worst = layerwise_check(pr, [0, 1])
    print("full size: worst |err| / bound", round(worst, 3))


def test_decoder_tiny_layerwise_across_the_boundary():
    """The same per-layer check on the tiny decoder, contexts on both sides
    of t = 2052 and all sequences flagged."""
    pr = DecProblem("tiny", [10, 2051, 2052, 5000], steps=1, seed=71)
    worst = layerwise_check(pr, [1, 1, 1, 1])
    print("tiny: worst |err| / bound", round(worst, 3))


def test_decoder_tiny_layerwise_paged_cache():
    """The per-layer check with a paged cache (16-row blocks at shuffled
    physical places): the local branch's attention with its QK-norm and
    RoPE folded in reads the cache through the block tables, contexts on
    both sides of t = 2052, half of the sequences flagged."""
    pr = DecProblem("tiny", [30, 2051, 2600, 4100], steps=1, seed=91, layout="paged")
    worst = layerwise_check(pr, [1, 0, 1, 0])
    print("tiny paged: worst |err| / bound", round(worst, 3))


@pytest.mark.parametrize("shape,layout", [("tiny-g1", "contig"), ("tiny-g4", "paged"), ("tiny-i3k", "contig")])
def test_decoder_tiny_layerwise_group_sizes(shape, layout):
    """The per-layer check with one and with four query heads per KV head
    (the attention kernels' other instantiations, QK-norm and RoPE folded
    into the local one), contiguous and paged caches, and with an MLP width
    of 3072 (three K slices in the down projection)."""
    pr = DecProblem(shape, [40, 2052, 3100], steps=1, seed=95, layout=layout)
    worst = layerwise_check(pr, [1, 1, 0])
    print(f"{shape} {layout}: worst |err| / bound", round(worst, 3))


def test_decoder_tiny_layerwise_wide_batch():
    """Twenty sequences (two 16-wide column groups in every GEMM) with ragged
    contexts, half of them flagged, checked layer by layer."""
    t0 = [7 + 211 * i for i in range(20)]
    pr = DecProblem("tiny", t0, steps=1, seed=81)
    worst = layerwise_check(pr, [i % 2 for i in range(20)])
    print("tiny B=20: worst |err| / bound", round(worst, 3))
