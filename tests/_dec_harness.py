"""Test harness for the decoder step around the ODA path: device buffers for
a decoder workload, and a reference replay of decode steps against the CPU
oracle (oracle/oda_decoder_oracle.py).

Replay protocol (the GPU trajectory drives, as for the attention-only
step): before each step the harness records the GPU's tokens, positions,
h_prev and cache; after it, the oracle recomputes from that state
  * the local branch of every sequence: staged K/V per layer, h^L;
  * the recall score from the GPU's h_prev, E(x_t) and h^L, and the rule;
  * the full branch of every flagged sequence: staged K/V, h^F;
  * the logits of the GPU's chosen hidden state and their argmax;
and compares (the tolerances follow from bf16 storage with fp32 accumulation):
  * h^L, h^F, staged K/V      |gpu - oracle| <= ATOL + RTOL |oracle|
  * scores                    |gpu - oracle| <= 1e-4 (1 + |oracle|)
  * flags                     bit-exact unless |q_oracle - theta| < 1e-3
  * next token                the GPU's token's logit is within TOKEN_BAND of the maximum,
                              and equal to the argmax when the top-two gap exceeds it
  * committed slots, h_prev, pos   bit-exact against the GPU's own staged values.
"""
from __future__ import annotations

import numpy as np
import torch

import synth
import synth.device as sd
from oracle import bf16_to_f64, branch_rule, full_index_set, local_index_set, recall_score, unpack_head
from oracle import decoder as D
import conditional_sparse_attention_amd as C
from conditional_sparse_attention_amd.decoder import DecoderBuffers, DecoderPlan, DecoderWeights

ATOL = RTOL = 3e-2
SCORE_TOL = 1e-4
TIE_BAND = 1e-3
TOKEN_BAND = 2e-2
DEV = "cuda"


def u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def close_report(gpu_bits, ref_bits, what):
    g = bf16_to_f64(gpu_bits)
    r = bf16_to_f64(ref_bits)
    err = np.abs(g - r)
    lim = ATOL + RTOL * np.abs(r)
    worst = float(np.max(err / lim)) if err.size else 0.0
    if np.any(err > lim):
        i = np.unravel_index(np.argmax(err - lim), err.shape)
        raise AssertionError(f"{what}: {int((err > lim).sum())} of {err.size} outside tolerance; worst at {i}: "
                             f"gpu {g[i]} oracle {r[i]}")
    return worst


class DecProblem:
    """Device state of a decoder workload (contiguous or paged cache)."""

    def __init__(self, shape_key: str, t0, *, steps: int, seed: int, perturb: bool = True,
                 device_weights: bool = False, layout: str = "contig"):
        sh = synth.decoder_shapes()[shape_key]
        self.sh = sh
        t0 = np.asarray(t0, dtype=np.int64)
        B = len(t0)
        self.wl = synth.Workload(f"dec-{shape_key}", sh.layers, sh.hq, sh.hkv, sh.head_dim, B, t0, steps, seed=seed,
                                 head_seed=seed + 100, t_cap_slack=16, layout=layout)
        wl = self.wl
        L, Hq, Hkv, d, Dm = sh.layers, sh.hq, sh.hkv, sh.head_dim, sh.hidden
        self.t0_dev = torch.from_numpy(t0.astype(np.int32)).to(DEV)
        if layout == "paged":
            tables, nb = synth.paged_block_tables(wl)
            self.attn = C.make_dims(L, B, Hq, Hkv, kv_layout=C.ODA_KV_PAGED, block_size=wl.block_size,
                                    max_blocks_per_seq=tables.shape[1], num_blocks=nb)
            self.tables = torch.from_numpy(tables).to(DEV)
            self.K = torch.zeros((L, nb, Hkv, wl.block_size, d), dtype=torch.int16, device=DEV)
            fill = dict(tables=self.tables, num_blocks=nb)
        else:
            self.attn = C.make_dims(L, B, Hq, Hkv, t_cap=wl.t_cap)
            self.tables = None
            self.K = torch.zeros((L, B, Hkv, wl.t_cap, d), dtype=torch.int16, device=DEV)
            fill = {}
        self.dd = C.make_dec_dims(self.attn, sh.inter, sh.vocab, sh.rope_theta, sh.eps)
        self.V = torch.zeros_like(self.K)
        sd.fill_cache(self.K, wl, synth.TAG_K, self.t0_dev, **fill)
        sd.fill_cache(self.V, wl, synth.TAG_V, self.t0_dev, **fill)
        self.kv = C.make_kv(self.K, self.V, self.tables)
        numel = C.oda_dec_layer_numel(self.dd)
        layers = torch.zeros((L, numel), dtype=torch.int16, device=DEV)
        embed = torch.zeros((sh.vocab, Dm), dtype=torch.int16, device=DEV)
        if device_weights:
            for l in range(L):
                sd.fill_dec_layer(layers[l], seed, sh, l, perturb=perturb)
            sd.fill_dec_embed(embed, seed)
        else:
            for l in range(L):
                layers[l].copy_(torch.from_numpy(synth.dec_layer_blob(seed, sh, l, perturb=perturb).view(np.int16)))
            embed.copy_(torch.from_numpy(synth.dec_embed_bits(seed, sh, np.arange(sh.vocab)).view(np.int16)))
        gamma_f = torch.from_numpy(synth.dec_gain_bits(seed, L, "gamma_final", Dm, perturb).view(np.int16)).to(DEV)
        self.weights = DecoderWeights(layers, embed, gamma_f)
        self.seed, self.perturb = seed, perturb
        self.head_blob = synth.head_blob(Dm, wl.head_seed, perturb=True)
        self.head_P = unpack_head(self.head_blob, Dm)
        tokens = torch.from_numpy(synth.dec_first_tokens(seed, B, sh.vocab)).to(DEV)
        h0 = torch.from_numpy(synth.h_prev0(wl).view(np.int16)).to(DEV)
        self.bufs = DecoderBuffers.allocate(self.dd, torch.from_numpy(self.head_blob).to(DEV), tokens,
                                            self.t0_dev.clone(), h0)
        self.ws = torch.zeros(C.oda_workspace_bytes(self.attn), dtype=torch.uint8, device=DEV)
        C.oda_workspace_init(self.attn, self.ws)
        self.dws = torch.zeros(C.oda_dec_workspace_bytes(self.dd), dtype=torch.uint8, device=DEV)
        C.oda_dec_workspace_init(self.dd, self.dws)
        self.plan = DecoderPlan(self.dd, self.kv, self.weights, self.bufs, self.ws, self.dws, theta=0.0)
        # host copies for the oracle: weights, and the cache rows the steps read
        self.layers_host = u16(layers)
        self.embed_host = u16(embed)
        self.gamma_f = bf16_to_f64(u16(gamma_f))
        self._P = {}
        self._cache_params = numel * L <= (1 << 26)
        torch.cuda.synchronize()

    def layer_params(self, l):
        sh = self.sh
        if l in self._P:
            return self._P[l]
        P = D.unpack_layer(self.layers_host[l], sh.hidden, sh.hq, sh.hkv, sh.head_dim, sh.inter)
        if self._cache_params:
            self._P[l] = P
        return P

    def history(self, b, pos):
        """[L] of ([Hkv][pos][d], [Hkv][pos][d]) bf16 bits of the GPU cache
        (positions 0 .. pos-1 of sequence b, through its block table when
        the cache is paged)."""
        if self.tables is None:
            Kh = u16(self.K[:, b, :, :pos])
            Vh = u16(self.V[:, b, :, :pos])
        else:
            bs = self.wl.block_size
            p = np.arange(pos)
            blk = self.tables[b].cpu().numpy()[p // bs]
            row = p % bs
            # advanced indices around a slice put the position axis first
            Kh = u16(self.K)[:, blk, :, row, :].transpose(1, 2, 0, 3)
            Vh = u16(self.V)[:, blk, :, row, :].transpose(1, 2, 0, 3)
        return [Kh[l] for l in range(self.sh.layers)], [Vh[l] for l in range(self.sh.layers)]


def replay_dec_step(pr: DecProblem, *, theta: float, force=None, check_b=None):
    """One step on the GPU, recomputed and checked by the oracle.  Returns
    the per-step record (flags, tokens, worst tolerance ratios)."""
    sh, b_ = pr.sh, pr.bufs
    B, L = pr.wl.batch, sh.layers
    pr.plan.set_theta(theta)
    f = np.full(B, -1, np.int8) if force is None else np.asarray(force, np.int8)
    b_.force.copy_(torch.from_numpy(f).to(DEV))
    pos0 = b_.pos.cpu().numpy().astype(np.int64)
    tok0 = b_.tokens.cpu().numpy().astype(np.int64)
    hprev0 = u16(b_.h_prev)
    hist = [pr.history(b, int(pos0[b])) for b in range(B)]
    pr.plan.run()
    torch.cuda.synchronize()
    assert int(pr.ws[:4].view(torch.int32).item()) == 0, "device error bits set"
    hL, hF = u16(b_.hL), u16(b_.hF)
    flag = b_.flag.cpu().numpy()
    score = b_.score.cpu().numpy().astype(np.float64)
    tok = b_.tokens.cpu().numpy()
    kL, vL, kF, vF = u16(b_.kL), u16(b_.vL), u16(b_.kF), u16(b_.vF)
    emb = u16(b_.emb)
    worst = {"h": 0.0, "kv": 0.0}
    layers = _LazyLayers(pr)
    bs = range(B) if check_b is None else check_b
    for b in bs:
        p = int(pos0[b])
        t = p + 1
        erow = pr.embed_host[tok0[b]]
        assert np.array_equal(emb[b], erow), "embedding row"
        x0 = bf16_to_f64(erow)
        Kh, Vh = hist[b]
        hL_ref, kL_ref, vL_ref, _ = D.branch_pass(x0, layers, sh.hq, sh.hkv, sh.head_dim, p, Kh, Vh,
                                                  local_index_set(t, pr.wl.sink, pr.wl.window), pr.gamma_f,
                                                  sh.rope_theta, sh.eps)
        worst["h"] = max(worst["h"], close_report(hL[b], hL_ref, f"h^L b={b}"))
        for l in range(L):
            worst["kv"] = max(worst["kv"], close_report(kL[l, b], kL_ref[l], f"kL l={l} b={b}"),
                              close_report(vL[l, b], vL_ref[l], f"vL l={l} b={b}"))
        q_ref = recall_score(pr.head_P, hprev0[b], erow, hL[b])
        assert abs(score[b] - q_ref) <= SCORE_TOL * (1 + abs(q_ref)), (b, score[b], q_ref)
        want = branch_rule(q_ref, theta, int(f[b]))
        if f[b] >= 0 or abs(q_ref - theta) >= TIE_BAND:
            assert flag[b] == want, (b, q_ref, theta, flag[b])
        if flag[b]:
            hF_ref, kF_ref, vF_ref, _ = D.branch_pass(x0, layers, sh.hq, sh.hkv, sh.head_dim, p, Kh, Vh,
                                                      full_index_set(t), pr.gamma_f, sh.rope_theta, sh.eps)
            worst["h"] = max(worst["h"], close_report(hF[b], hF_ref, f"h^F b={b}"))
            for l in range(L):
                worst["kv"] = max(worst["kv"], close_report(kF[l, b], kF_ref[l], f"kF l={l} b={b}"),
                                  close_report(vF[l, b], vF_ref[l], f"vF l={l} b={b}"))
        h_sel = hF[b] if flag[b] else hL[b]
        # next token: logits of the GPU's chosen hidden state
        lg = logits_of(pr, h_sel)
        top = np.sort(lg)[::-1]
        assert lg[tok[b]] >= top[0] - TOKEN_BAND, (b, tok[b], lg[tok[b]], top[:2])
        if top[0] - top[1] > TOKEN_BAND:
            assert tok[b] == D.argmax_first(lg), (b, tok[b], D.argmax_first(lg))
    # commit: slot, h_prev and pos from the GPU's own chosen values, bit for bit
    pos1 = b_.pos.cpu().numpy()
    hprev1 = u16(b_.h_prev)
    for b in range(B):
        p = int(pos0[b])
        assert pos1[b] == p + 1
        sel_k, sel_v = (kF, vF) if flag[b] else (kL, vL)
        assert np.array_equal(u16(pr.K[:, b, :, p]), sel_k[:, b]), f"committed K slot b={b}"
        assert np.array_equal(u16(pr.V[:, b, :, p]), sel_v[:, b]), f"committed V slot b={b}"
        assert np.array_equal(hprev1[b], hF[b] if flag[b] else hL[b]), f"h_prev b={b}"
    return {"flag": flag, "tokens": tok, "worst": worst}


class _LazyLayers:
    """Sequence of a problem's layer parameters, unpacked on access."""

    def __init__(self, pr):
        self.pr = pr

    def __len__(self):
        return self.pr.sh.layers

    def __getitem__(self, l):
        return self.pr.layer_params(l)

    def __iter__(self):
        return (self.pr.layer_params(l) for l in range(len(self)))


def logits_of(pr: DecProblem, h_bits: np.ndarray) -> np.ndarray:
    """E h over the whole vocabulary, in row chunks (float64)."""
    h = bf16_to_f64(h_bits)
    V = pr.sh.vocab
    out = np.empty(V, dtype=np.float64)
    step = 8192
    for r0 in range(0, V, step):
        r1 = min(V, r0 + step)
        out[r0:r1] = bf16_to_f64(pr.embed_host[r0:r1]) @ h
    return out


LAYER_TOL = 2.0 ** -5   # per-layer bound, in units of the compared vector's RMS (4 bf16 ulps at that scale)


def _rms_close(gpu, ref, what, rows=None):
    """|gpu - ref| <= LAYER_TOL * rms(ref) per vector (rows of the last axis)."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
    ratio = np.abs(g - r) / (LAYER_TOL * np.maximum(rms, 1e-30))
    if np.any(ratio > 1.0):
        i = np.unravel_index(np.argmax(ratio), ratio.shape)
        raise AssertionError(f"{what}: worst at {i}: gpu {g[i]} oracle {r[i]} (rms {float(rms.reshape(-1)[0]):.4g})")
    return float(ratio.max())


def layerwise_check(pr: DecProblem, flags):
    """One step run layer by layer through the C ABI, each layer checked
    against the oracle's layer applied to the GPU's own input of that layer
    (teacher forcing), so differences do not compound across layers.  Checks
    the residual stream, the staged K/V and the attention output of every
    layer of both branches (the full branch for the flagged sequences), the
    final hidden states from the GPU's residual, and the next token from the
    GPU's chosen hidden state.  Returns the worst ratio to the bound."""
    sh, b_ = pr.sh, pr.bufs
    B, L = pr.wl.batch, sh.layers
    flags = np.asarray(flags, np.uint8)
    pos0 = b_.pos.cpu().numpy().astype(np.int64)
    tok0 = b_.tokens.cpu().numpy().astype(np.int64)
    hist = [pr.history(b, int(pos0[b])) for b in range(B)]
    fdev = torch.from_numpy(flags).to(DEV)
    C.oda_dec_embed(pr.dd, pr.weights.embed, b_.tokens, b_.xL, b_.xF, b_.emb, pr.ws)
    C.oda_worklist(pr.attn, fdev, b_.pos, pr.ws)
    worst = 0.0
    branches = ((C.ODA_DEC_LOCAL, b_.xL, b_.kL, b_.vL, b_.oL, b_.hL, range(B)),
                (C.ODA_DEC_FULL, b_.xF, b_.kF, b_.vF, b_.oF, b_.hF, [b for b in range(B) if flags[b]]))
    for br, x, kk, vv, oo, hh, rows in branches:
        for l in range(L):
            xin = x.cpu().numpy().astype(np.float64)
            C.oda_dec_layer(pr.dd, l, br, pr.weights.layers[l], pr.kv, b_.pos, x, b_.q, kk[l], vv[l], oo, pr.ws,
                            pr.dws)
            torch.cuda.synchronize()
            xout = x.cpu().numpy().astype(np.float64)
            kc, vc, oc = u16(kk[l]), u16(vv[l]), u16(oo)
            P = pr.layer_params(l)
            for b in rows:
                p = int(pos0[b])
                S = local_index_set(p + 1, pr.wl.sink, pr.wl.window) if br == C.ODA_DEC_LOCAL else full_index_set(p + 1)
                Kh, Vh = hist[b]
                xr, kr, vr, orf = D.decoder_layer(xin[b], P, sh.hq, sh.hkv, sh.head_dim, p, Kh[l], Vh[l], S,
                                                  sh.rope_theta, sh.eps)
                tag = f"branch {br} layer {l} b={b}"
                worst = max(worst, _rms_close(xout[b], xr, "x " + tag),
                            _rms_close(bf16_to_f64(kc[b]), bf16_to_f64(kr), "k_cur " + tag),
                            _rms_close(bf16_to_f64(vc[b]), bf16_to_f64(vr), "v_cur " + tag),
                            _rms_close(bf16_to_f64(oc[b]), bf16_to_f64(orf), "o " + tag))
        C.oda_dec_final_norm(pr.dd, br, pr.weights.gamma_f, x, hh, pr.ws)
        torch.cuda.synchronize()
        xg = x.cpu().numpy().astype(np.float64)
        hg = u16(hh)
        for b in rows:
            worst = max(worst, _rms_close(bf16_to_f64(hg[b]), bf16_to_f64(D.final_hidden(xg[b], pr.gamma_f, sh.eps)),
                                          f"h branch {br} b={b}"))
    C.oda_dec_next_token(pr.dd, pr.weights.embed, b_.hL, b_.hF, fdev, b_.tokens, b_.max_logit, pr.dws)
    torch.cuda.synchronize()
    tok = b_.tokens.cpu().numpy()
    hL, hF = u16(b_.hL), u16(b_.hF)
    for b in range(B):
        assert np.array_equal(u16(b_.emb)[b], pr.embed_host[tok0[b]])
        lg = logits_of(pr, hF[b] if flags[b] else hL[b])
        top = np.sort(lg)[::-1]
        assert lg[tok[b]] >= top[0] - TOKEN_BAND, (b, tok[b], lg[tok[b]], top[:2])
        if top[0] - top[1] > TOKEN_BAND:
            assert tok[b] == D.argmax_first(lg), (b, tok[b], D.argmax_first(lg))
    return worst
