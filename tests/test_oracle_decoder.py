"""Pins of the decoder oracle (oracle/oda_decoder_oracle.py) against facts
that do not come from the oracle itself: the pages' parameter ratio, closed
forms of RoPE and RMSNorm, brute-force loops on tiny shapes, and the
invariants of the branch structure."""
import math

import numpy as np
import pytest

import synth
from oracle import bf16_to_f64, f64_to_bf16, attention, recall_score, unpack_head
from oracle import decoder as D

RNG = np.random.default_rng(7)


def bits(x):
    return f64_to_bf16(np.asarray(x, dtype=np.float64))



def test_bf16_rounding_is_nearest_even():
    """bf16 keeps 8 significand bits, so between 1 and 2 its spacing is
    2^-7.  An exact midpoint goes to the neighbour with an even last bit,
    anything off the midpoint to the nearer neighbour (decided on the float64
    value, not on a float32 rounding of it), and the sign is symmetric."""
    cases = {
        1.0: 0x3F80,
        1.0 + 2.0 ** -8: 0x3F80,                      # midpoint of 0x3F80 / 0x3F81 -> even
        1.0 + 3 * 2.0 ** -8: 0x3F82,                  # midpoint of 0x3F81 / 0x3F82 -> even
        1.0 + 2.0 ** -8 + 2.0 ** -30: 0x3F81,         # just above a midpoint
        1.0 + 2.0 ** -8 - 2.0 ** -30: 0x3F80,         # just below it
        -(1.0 + 3 * 2.0 ** -8): 0xBF82,
        0.0: 0x0000,
    }
    for x, bits in cases.items():
        assert int(f64_to_bf16(np.array([x]))[0]) == bits, (x, hex(bits))

def test_backbone_size_matches_pages_ratio():
    """The pages put the recall head at about 1.7% of the backbone's
    parameters (ODA notes, §3.3 closing paragraph).  A Qwen3-1.7B-shaped
    decoder (28 layers of 16/8 heads, hidden 2048, MLP 6144, vocabulary
    151,936 with a tied embedding, a final norm) gives 1.65% with the
    page's 28,325,889-parameter head."""
    sh = synth.decoder_shapes()["qwen3-1.7b"]
    per_layer = D.layer_param_count(sh.hidden, sh.hq, sh.hkv, sh.head_dim, sh.inter)
    assert per_layer == 50_336_000
    total = sh.layers * per_layer + sh.vocab * sh.hidden + sh.hidden
    ratio = 28_325_889 / total
    assert abs(ratio - 0.017) < 0.001, ratio


def test_layout_agrees_with_generator_blob():
    sh = synth.decoder_shapes()["tiny"]
    lay = D.layer_layout(sh.hidden, sh.hq, sh.hkv, sh.head_dim, sh.inter)
    assert [(n, tuple(s)) for n, s in lay] == [(n, tuple(s)) for n, s in synth.dec_layer_tensors(sh)]
    blob = synth.dec_layer_blob(3, sh, 1)
    P = D.unpack_layer(blob, sh.hidden, sh.hq, sh.hkv, sh.head_dim, sh.inter)
    assert P["W_qkv"].shape == ((sh.hq + 2 * sh.hkv) * sh.head_dim, sh.hidden)
    assert np.all(P["gamma_in"] == 1.0)


def test_rope_closed_forms():
    d, theta = 8, 10000.0
    x = RNG.standard_normal(d)
    assert np.allclose(D.rope(x, 0, theta), x, rtol=0, atol=0)
    # pair i rotates by pos * theta^(-2i/d): unit vector on pair 0 at pos 1 -> (cos 1, sin 1)
    e = np.zeros(d)
    e[0] = 1.0
    r = D.rope(e, 1, theta)
    assert np.allclose(r, [math.cos(1.0), 0, 0, 0, math.sin(1.0), 0, 0, 0], atol=1e-15)
    # pair 1 (components 1 and 5) at pos 3
    e = np.zeros(d)
    e[5] = 2.0
    a = 3 * theta ** (-2.0 / d)
    r = D.rope(e, 3, theta)
    assert np.allclose(r, [0, -2 * math.sin(a), 0, 0, 0, 2 * math.cos(a), 0, 0], atol=1e-15)
    # rotations compose and preserve each pair's length
    p1, p2 = 1234, 98765
    assert np.allclose(D.rope(D.rope(x, p1, theta), p2, theta), D.rope(x, p1 + p2, theta), atol=1e-9)
    r = D.rope(x, 77777, theta)
    assert np.allclose(r[:4] ** 2 + r[4:] ** 2, x[:4] ** 2 + x[4:] ** 2, rtol=1e-12)


def test_rms_scale_and_final_hidden_closed_forms():
    eps = 1e-6
    x = np.full(64, -3.0)
    assert math.isclose(D.rms_scale(x, eps), 1.0 / math.sqrt(9.0 + eps), rel_tol=1e-15)
    h = bf16_to_f64(D.final_hidden(x, np.full(64, 0.5), eps))
    assert np.all(h == bf16_to_f64(bits(-0.5 * 3.0 / math.sqrt(9.0 + eps))))


def test_qk_norm_rope_is_scale_free():
    v = bits(RNG.standard_normal(128) * 3.0)
    v2 = bits(bf16_to_f64(v) * 4.0)      # exact in bf16
    g = bf16_to_f64(bits(1.0 + 0.1 * RNG.standard_normal(128)))
    a = bf16_to_f64(D.qk_norm_rope(v, g, 4567, 1e6, 1e-6))
    b = bf16_to_f64(D.qk_norm_rope(v2, g, 4567, 1e6, 1e-6))
    assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.abs(a) + 1e-30)


def test_argmax_first_takes_the_smallest_index_on_ties():
    assert D.argmax_first([0.0, 3.0, 1.0, 3.0]) == 1
    assert D.argmax_first([-1.0]) == 0


def _tiny_layer(D_, hq, hkv, d, I, seed):
    rng = np.random.default_rng(seed)
    P = {"gamma_in": bf16_to_f64(bits(1 + 0.1 * rng.standard_normal(D_))),
         "W_qkv": bf16_to_f64(bits(0.3 * rng.standard_normal(((hq + 2 * hkv) * d, D_)))),
         "gamma_q": bf16_to_f64(bits(1 + 0.1 * rng.standard_normal(d))),
         "gamma_k": bf16_to_f64(bits(1 + 0.1 * rng.standard_normal(d))),
         "W_o": bf16_to_f64(bits(0.3 * rng.standard_normal((D_, hq * d)))),
         "gamma_post": bf16_to_f64(bits(1 + 0.1 * rng.standard_normal(D_))),
         "W_gate": bf16_to_f64(bits(0.3 * rng.standard_normal((I, D_)))),
         "W_up": bf16_to_f64(bits(0.3 * rng.standard_normal((I, D_)))),
         "W_down": bf16_to_f64(bits(0.3 * rng.standard_normal((D_, I))))}
    return P


def _dot(row, vec):
    s = 0.0
    for a, b in zip(row, vec):
        s += a * b
    return s


def test_layer_matches_loops_on_a_tiny_shape():
    """The whole layer recomputed with explicit loops (no matmul) on a tiny
    shape: projections, QK-norm + RoPE, attention over the history plus the
    staged row, output projection, SwiGLU MLP, both residual adds."""
    Dm, hq, hkv, d, I, pos, eps, theta = 16, 2, 1, 8, 12, 5, 1e-6, 10000.0
    P = _tiny_layer(Dm, hq, hkv, d, I, 3)
    rng = np.random.default_rng(4)
    x = rng.standard_normal(Dm)
    K = bits(rng.standard_normal((hkv, pos, d)))
    V = bits(rng.standard_normal((hkv, pos, d)))
    S = [0, 2, 3, 5]
    x_out, kc, vc, o = D.decoder_layer(x, P, hq, hkv, d, pos, K, V, S, theta, eps)

    r = 1.0 / math.sqrt(sum(v * v for v in x) / Dm + eps)
    a_in = bf16_to_f64(bits([P["gamma_in"][i] * x[i] for i in range(Dm)]))
    qkv = bf16_to_f64(bits([r * _dot(P["W_qkv"][n], a_in) for n in range(P["W_qkv"].shape[0])]))

    def qkr(v, gamma):
        rr = 1.0 / math.sqrt(sum(t * t for t in v) / d + eps)
        y = [gamma[i] * v[i] * rr for i in range(d)]
        out = [0.0] * d
        for i in range(d // 2):
            ang = pos * theta ** (-2.0 * i / d)
            out[i] = y[i] * math.cos(ang) - y[i + d // 2] * math.sin(ang)
            out[i + d // 2] = y[i + d // 2] * math.cos(ang) + y[i] * math.sin(ang)
        return bf16_to_f64(bits(out))

    q = [qkr(qkv[h * d:(h + 1) * d], P["gamma_q"]) for h in range(hq)]
    k = qkr(qkv[hq * d:(hq + 1) * d], P["gamma_k"])
    v = qkv[(hq + 1) * d:(hq + 2) * d]
    assert np.array_equal(bf16_to_f64(kc[0]), k)
    assert np.array_equal(bf16_to_f64(vc[0]), v)
    Kf, Vf = bf16_to_f64(K[0]), bf16_to_f64(V[0])
    o_ref = []
    for h in range(hq):
        keys = [Kf[i] if i < pos else k for i in S]
        vals = [Vf[i] if i < pos else v for i in S]
        sc = [_dot(q[h], kk) / math.sqrt(d) for kk in keys]
        m = max(sc)
        w = [math.exp(s - m) for s in sc]
        z = sum(w)
        o_ref.append(bf16_to_f64(bits([sum(w[j] * vals[j][i] for j in range(len(S))) / z for i in range(d)])))
    o_ref = np.concatenate(o_ref)
    assert np.allclose(bf16_to_f64(o).reshape(-1), o_ref, rtol=2.0 ** -7, atol=1e-12)
    o_used = bf16_to_f64(o).reshape(-1)
    x1 = [x[i] + _dot(P["W_o"][i], o_used) for i in range(Dm)]
    r2 = 1.0 / math.sqrt(sum(t * t for t in x1) / Dm + eps)
    a_mid = bf16_to_f64(bits([P["gamma_post"][i] * x1[i] for i in range(Dm)]))
    g = bf16_to_f64(bits([r2 * _dot(P["W_gate"][j], a_mid) for j in range(I)]))
    u = bf16_to_f64(bits([r2 * _dot(P["W_up"][j], a_mid) for j in range(I)]))
    mm = bf16_to_f64(bits([g[j] / (1.0 + math.exp(-g[j])) * u[j] for j in range(I)]))
    x2 = np.array([x1[i] + _dot(P["W_down"][i], mm) for i in range(Dm)])
    assert np.allclose(x_out, x2, rtol=1e-12, atol=1e-12)


def test_layer_with_zero_output_projections_keeps_the_residual():
    Dm, hq, hkv, d, I = 16, 2, 1, 8, 12
    P = _tiny_layer(Dm, hq, hkv, d, I, 5)
    P["W_o"][:] = 0.0
    P["W_down"][:] = 0.0
    x = np.random.default_rng(6).standard_normal(Dm)
    K = bits(np.zeros((hkv, 3, d)))
    x_out, *_ = D.decoder_layer(x, P, hq, hkv, d, 3, K, K, [0, 1, 2, 3], 1e6, 1e-6)
    assert np.array_equal(x_out, x)


def test_zero_query_attention_averages_values_inside_the_layer():
    """With the q rows of W_qkv zeroed, QK-norm of a zero vector is zero, so
    every head's attention output is the mean of v over the index set."""
    Dm, hq, hkv, d, I, pos = 16, 2, 1, 8, 12, 4
    P = _tiny_layer(Dm, hq, hkv, d, I, 8)
    P["W_qkv"][:hq * d] = 0.0
    rng = np.random.default_rng(9)
    x = rng.standard_normal(Dm)
    K = bits(rng.standard_normal((hkv, pos, d)))
    V = bits(rng.standard_normal((hkv, pos, d)))
    S = [0, 1, 2, 3, 4]
    _, kc, vc, o = D.decoder_layer(x, P, hq, hkv, d, pos, K, V, S, 1e6, 1e-6)
    vals = np.concatenate([bf16_to_f64(V[0]), bf16_to_f64(vc)], axis=0)
    for h in range(hq):
        assert np.allclose(bf16_to_f64(o[h]), bf16_to_f64(bits(vals.mean(axis=0))), rtol=0, atol=0)


def _tiny_model(seed, perturb=True):
    sh = synth.decoder_shapes()["tiny"]
    layers = [D.unpack_layer(synth.dec_layer_blob(seed, sh, l, perturb=perturb), sh.hidden, sh.hq, sh.hkv,
                             sh.head_dim, sh.inter) for l in range(sh.layers)]
    gf = bf16_to_f64(synth.dec_gain_bits(seed, sh.layers, "gamma_final", sh.hidden, perturb))
    return sh, layers, gf


def test_branches_agree_bitwise_when_the_sets_coincide():
    """For t <= s + w = 2052 the local and full index sets are the same set
    (ODA notes §2.1), so both branches produce identical bits."""
    sh, layers, gf = _tiny_model(11)
    pos = 700
    rng = np.random.default_rng(12)
    K = [bits(0.5 * rng.standard_normal((sh.hkv, pos, sh.head_dim))) for _ in range(sh.layers)]
    V = [bits(0.5 * rng.standard_normal((sh.hkv, pos, sh.head_dim))) for _ in range(sh.layers)]
    x0 = bf16_to_f64(synth.dec_embed_bits(11, sh, [17])[0])
    from oracle import local_index_set, full_index_set
    hL, kL, vL, _ = D.branch_pass(x0, layers, sh.hq, sh.hkv, sh.head_dim, pos, K, V, local_index_set(pos + 1),
                                  gf, sh.rope_theta, sh.eps)
    hF, kF, vF, _ = D.branch_pass(x0, layers, sh.hq, sh.hkv, sh.head_dim, pos, K, V, full_index_set(pos + 1),
                                  gf, sh.rope_theta, sh.eps)
    assert np.array_equal(hL, hF)
    for a, b in zip(kL + vL, kF + vF):
        assert np.array_equal(a, b)


def test_step_takes_the_chosen_branch():
    """oda_decoder_step: a forced local step returns the local branch's
    hidden state and token; a forced full step the full branch's (they differ
    once t > 2052)."""
    sh, layers, gf = _tiny_model(13)
    pos = 2100
    rng = np.random.default_rng(14)
    K = [bits(0.5 * rng.standard_normal((sh.hkv, pos, sh.head_dim))) for _ in range(sh.layers)]
    V = [bits(0.5 * rng.standard_normal((sh.hkv, pos, sh.head_dim))) for _ in range(sh.layers)]
    tok = 5
    erow = synth.dec_embed_bits(13, sh, [tok])[0]
    E = synth.dec_embed_bits(13, sh, np.arange(64))
    head_P = unpack_head(synth.head_blob(sh.hidden, 113), sh.hidden)
    h_prev = bits(rng.standard_normal(sh.hidden))
    lf = lambda h: D.logits(E, h)
    recs = [D.oda_decoder_step(tok, erow, layers, sh.hq, sh.hkv, sh.head_dim, pos, K, V, gf, sh.rope_theta,
                               sh.eps, head_P, h_prev, 0.0, force, lf) for force in (0, 1)]
    assert recs[0]["flag"] == 0 and recs[1]["flag"] == 1
    assert np.array_equal(recs[0]["h"], recs[0]["hL"])
    assert np.array_equal(recs[1]["h"], recs[1]["hF"])
    assert not np.array_equal(recs[1]["hF"], recs[1]["hL"])
    # the score is the head on (h_prev, E(x_t), h^L) whatever the branch
    assert recs[0]["score"] == recs[1]["score"] == recall_score(head_P, h_prev, erow, recs[0]["hL"])
    for r in recs:
        assert r["token"] == D.argmax_first(D.logits(E, r["h"]))


# ---------------------------------------------------------------------------
# the oracle's rounded layer against the textbook float64 layer
# ---------------------------------------------------------------------------
U_BF16 = 2.0 ** -9      # unit roundoff of round-to-nearest bf16 (8 significand bits)


def _textbook_layer(x, P, hq, hkv, d, pos, Kf, Vf, S, theta, eps, *, pert=None, mlp_norm_from=None,
                    rope_shift=0, v_rotated=False):
    """The standard pre-norm decoder layer in float64: RMSNorm before each
    projection, QK-norm, RoPE, softmax attention over S of the history plus
    the current row, residuals, SwiGLU.  With pert=None nothing is rounded.
    pert(y) is applied wherever a backbone stores an activation (the
    normalised input, the q/k/v projection, the rotated q and k, the
    attention output, the normalised MLP input, gate, up and their product).
    mlp_norm_from / rope_shift / v_rotated plant plausible mistakes (the MLP
    norm of the pre-attention stream; RoPE one position off; v rotated like
    k).  Returns (x2, k, v, o)."""
    f = pert if pert is not None else (lambda y: y)
    rms = lambda v: 1.0 / math.sqrt(float(np.mean(v * v)) + eps)
    a = f(P["gamma_in"] * x) * rms(x)
    qkv = f(P["W_qkv"] @ a)
    half = d // 2
    ang = (pos + rope_shift) * theta ** (-2.0 * np.arange(half) / d)
    c, s = np.cos(ang), np.sin(ang)

    def norm_rope(v, gamma):
        y = gamma * v * rms(v)
        return f(np.concatenate([y[:half] * c - y[half:] * s, y[half:] * c + y[:half] * s]))

    q = np.stack([norm_rope(qkv[h * d:(h + 1) * d], P["gamma_q"]) for h in range(hq)])
    k = np.stack([norm_rope(qkv[(hq + g) * d:(hq + g + 1) * d], P["gamma_k"]) for g in range(hkv)])
    v = np.stack([qkv[(hq + hkv + g) * d:(hq + hkv + g + 1) * d] for g in range(hkv)])
    if v_rotated:
        v = np.concatenate([v[:, :half] * c - v[:, half:] * s, v[:, half:] * c + v[:, :half] * s], axis=1)
    G = hq // hkv
    o = np.zeros((hq, d))
    for h in range(hq):
        g = h // G
        keys = np.stack([Kf[g][i] if i < pos else k[g] for i in S])
        vals = np.stack([Vf[g][i] if i < pos else v[g] for i in S])
        sc = keys @ q[h] / math.sqrt(d)
        p = np.exp(sc - sc.max())
        o[h] = f((p / p.sum()) @ vals)
    x1 = x + P["W_o"] @ o.reshape(-1)
    xm = x if mlp_norm_from == "x" else x1
    a2 = f(P["gamma_post"] * xm) * rms(xm)
    gt, ut = f(P["W_gate"] @ a2), f(P["W_up"] @ a2)
    m = f(gt / (1.0 + np.exp(-gt)) * ut)
    return x1 + P["W_down"] @ m, k, v, o


@pytest.mark.parametrize("seed,pos,S", [(21, 9, [0, 1, 2, 3, 7, 8, 9]), (22, 30, list(range(31))),
                                        (23, 40, [0, 1, 38, 39, 40])])
def test_rounded_layer_is_the_textbook_layer_within_the_bf16_budget(seed, pos, S):
    """The oracle's decoder layer rounds to bf16 where the backbone stores
    activations and applies each RMSNorm scale to the finished dot product.
    Without rounding that is exactly the textbook pre-norm layer.  The
    budget for one bf16 rounding per stored activation: the textbook layer
    is re-run 300 times with every stored activation multiplied by
    (1 + delta), delta uniform in [-u, u] (u = 2^-9, the bound of
    round-to-nearest), and the oracle's distance from the unrounded layer
    must lie within 1.5x the largest distance seen.  The budget is small
    against the layer's own update, and plausible misreadings (the MLP norm
    from the pre-attention stream; RoPE one position off; v rotated like k)
    lie far outside it."""
    Dm, hq, hkv, d, I, eps, theta = 64, 4, 2, 16, 96, 1e-6, 10000.0
    rng = np.random.default_rng(seed)
    w = lambda n, k: bf16_to_f64(bits(rng.standard_normal((n, k)) / math.sqrt(k)))
    gain = lambda n: bf16_to_f64(bits(1 + 0.1 * rng.standard_normal(n)))
    P = {"gamma_in": gain(Dm), "W_qkv": w((hq + 2 * hkv) * d, Dm), "gamma_q": gain(d), "gamma_k": gain(d),
         "W_o": w(Dm, hq * d), "gamma_post": gain(Dm), "W_gate": w(I, Dm), "W_up": w(I, Dm), "W_down": w(Dm, I)}
    x = rng.standard_normal(Dm)
    K = bits(rng.standard_normal((hkv, pos, d)))
    V = bits(rng.standard_normal((hkv, pos, d)))
    Kf, Vf = bf16_to_f64(K), bf16_to_f64(V)
    got = D.decoder_layer(x, P, hq, hkv, d, pos, K, V, S, theta, eps)
    got = (got[0], bf16_to_f64(got[1]), bf16_to_f64(got[2]), bf16_to_f64(got[3]))
    exact = _textbook_layer(x, P, hq, hkv, d, pos, Kf, Vf, S, theta, eps)
    prng = np.random.default_rng(seed + 1000)
    pert = lambda y: y * (1.0 + prng.uniform(-U_BF16, U_BF16, np.shape(y)))
    budget = np.zeros(4)
    for _ in range(300):
        smp = _textbook_layer(x, P, hq, hkv, d, pos, Kf, Vf, S, theta, eps, pert=pert)
        budget = np.maximum(budget, [np.max(np.abs(a - b)) for a, b in zip(smp, exact)])
    dist = np.array([np.max(np.abs(a - b)) for a, b in zip(got, exact)])
    assert np.all(dist <= 1.5 * budget), (dist, budget)
    update = np.max(np.abs(exact[0] - x))
    assert budget[0] < 0.02 * update, (budget[0], update)
    for mistake in ({"mlp_norm_from": "x"}, {"rope_shift": 1}, {"v_rotated": True}):
        wrong = _textbook_layer(x, P, hq, hkv, d, pos, Kf, Vf, S, theta, eps, **mistake)
        assert np.max(np.abs(wrong[0] - exact[0])) > 5.0 * budget[0], mistake
