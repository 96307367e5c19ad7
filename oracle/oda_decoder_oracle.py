"""CPU oracle of a dense decoder step around the ODA path.

TEST INFRASTRUCTURE ONLY, like ``oda_oracle``: only the tests, the smoke
check and the bench's CPU baseline may import it; the product path never
does, and nothing here is shared with it.

What it computes.  The pages run ODA inside a dense Qwen3 backbone kept in
BF16 ([ODA notes] §3.3, efficiency paragraph: backbone and cache in BF16, the
recall head in FP32).  Both branches recompute the whole backbone for the
step from the same pre-step state and commit the chosen branch's state
([ODA notes] §2.3).  The pages do not restate the backbone's layer; the
reading here is the standard pre-norm decoder layer of that family:

    a   = RMSNorm(x) ; q, k, v = W_qkv a
    q_h = RoPE(RMSNorm_d(q_h)), k_g = RoPE(RMSNorm_d(k_g))   (QK-norm)
    o   = attention over the branch's index set (the ODA path)
    x  += W_o o
    x  += W_down (SiLU(W_gate RMSNorm(x)) * (W_up RMSNorm(x)))

then a final RMSNorm gives the step's hidden state h and the tied LM head
gives logits E h; the next token is their argmax (greedy decoding).

Rounding points.  Every stored activation is bf16 (the pages' precision of
the backbone); each is computed here in float64 from the bf16 values it
reads and rounded to nearest-even once:
    a_in  = bf16(gamma_in * x),  r = 1 / sqrt(mean(x^2) + eps)
    qkv   = bf16(r * (W_qkv a_in))
    q', k' = bf16(RoPE(gamma * v / sqrt(mean(v^2) + eps)))   per head
    o     = bf16(attention(...))
    x     = x + W_o o                              (residual kept unrounded)
    a_mid = bf16(gamma_post * x), r2 = 1 / sqrt(mean(x^2) + eps)
    g, u  = bf16(r2 * (W_gate a_mid)), bf16(r2 * (W_up a_mid))
    m     = bf16(SiLU(g) * u)
    x     = x + W_down m
    h     = bf16(gamma_f * x * r_f)
The RMSNorm scale r multiplies the finished dot product rather than the bf16
operand; both are RMSNorm, and the rounding point is part of this
definition.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

from .oda_oracle import bf16_to_f64, branch_rule, decode_attention, f64_to_bf16, full_index_set, local_index_set


# ---------------------------------------------------------------------------
# layout of one layer's bf16 parameters (this module's own statement of it)
# ---------------------------------------------------------------------------
def layer_layout(hidden: int, hq: int, hkv: int, head_dim: int, inter: int) -> List[Tuple[str, tuple]]:
    D, d, I = hidden, head_dim, inter
    return [("gamma_in", (D,)), ("W_qkv", ((hq + 2 * hkv) * d, D)), ("gamma_q", (d,)), ("gamma_k", (d,)),
            ("W_o", (D, hq * d)), ("gamma_post", (D,)), ("W_gate", (I, D)), ("W_up", (I, D)),
            ("W_down", (D, I))]


def layer_param_count(hidden: int, hq: int, hkv: int, head_dim: int, inter: int) -> int:
    return sum(int(np.prod(s)) for _, s in layer_layout(hidden, hq, hkv, head_dim, inter))


def unpack_layer(blob_bits: np.ndarray, hidden: int, hq: int, hkv: int, head_dim: int,
                 inter: int) -> Dict[str, np.ndarray]:
    blob_bits = np.asarray(blob_bits, dtype=np.uint16)
    out, at = {}, 0
    for name, shape in layer_layout(hidden, hq, hkv, head_dim, inter):
        n = int(np.prod(shape))
        out[name] = bf16_to_f64(blob_bits[at:at + n]).reshape(shape)
        at += n
    if at != blob_bits.size:
        raise ValueError(f"layer blob has {blob_bits.size} values, layout needs {at}")
    return out


# ---------------------------------------------------------------------------
# pieces
# ---------------------------------------------------------------------------
def rms_scale(x: np.ndarray, eps: float) -> float:
    """1 / sqrt(mean(x^2) + eps) of a vector (float64)."""
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / math.sqrt(float(np.mean(x * x)) + eps)


def rope(x: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotary embedding of one head vector at 0-based position pos: pair
    (x_i, x_{i+d/2}) is rotated by pos * theta^(-2i/d)."""
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    i = np.arange(half, dtype=np.float64)
    ang = float(pos) * theta ** (-2.0 * i / x.shape[-1])
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def qk_norm_rope(v_bits: np.ndarray, gamma: np.ndarray, pos: int, theta: float, eps: float) -> np.ndarray:
    """bf16(RoPE(gamma * v / rms(v))) of one head (bits in, bits out)."""
    v = bf16_to_f64(v_bits)
    return f64_to_bf16(rope(gamma * v * rms_scale(v, eps), pos, theta))


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def argmax_first(logits: np.ndarray) -> int:
    """Index of the largest logit; the smallest such index on ties."""
    logits = np.asarray(logits, dtype=np.float64)
    return int(np.flatnonzero(logits == logits.max())[0])


# ---------------------------------------------------------------------------
# one layer, one sequence
# ---------------------------------------------------------------------------
def decoder_layer(x: np.ndarray, P: Dict[str, np.ndarray], hq: int, hkv: int, head_dim: int, pos: int,
                  K_hist: np.ndarray, V_hist: np.ndarray, S: Sequence[int], theta: float,
                  eps: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """One decoder layer of one sequence.

    x: residual stream [D] float64.  K_hist, V_hist: [Hkv][pos][d] bf16 bits,
    the committed history of this layer.  S: the branch's index set over
    [0, pos].  Returns (x_out, k_cur bits [Hkv][d], v_cur bits [Hkv][d],
    o bits [Hq][d]); k_cur / v_cur are what the commit writes if this branch
    is chosen."""
    d = head_dim
    a_in = f64_to_bf16(P["gamma_in"] * x)
    qkv = f64_to_bf16(rms_scale(x, eps) * (P["W_qkv"] @ bf16_to_f64(a_in)))
    q = np.stack([qk_norm_rope(qkv[h * d:(h + 1) * d], P["gamma_q"], pos, theta, eps) for h in range(hq)])
    k0 = hq * d
    k_cur = np.stack([qk_norm_rope(qkv[k0 + g * d:k0 + (g + 1) * d], P["gamma_k"], pos, theta, eps)
                      for g in range(hkv)])
    v0 = (hq + hkv) * d
    v_cur = np.stack([qkv[v0 + g * d:v0 + (g + 1) * d] for g in range(hkv)])
    o = f64_to_bf16(decode_attention(q, K_hist, V_hist, k_cur, v_cur, S))
    x = x + P["W_o"] @ bf16_to_f64(o.reshape(-1))
    a_mid = bf16_to_f64(f64_to_bf16(P["gamma_post"] * x))
    r2 = rms_scale(x, eps)
    g = bf16_to_f64(f64_to_bf16(r2 * (P["W_gate"] @ a_mid)))
    u = bf16_to_f64(f64_to_bf16(r2 * (P["W_up"] @ a_mid)))
    m = f64_to_bf16(silu(g) * u)
    x = x + P["W_down"] @ bf16_to_f64(m)
    return x, k_cur, v_cur, o


def final_hidden(x: np.ndarray, gamma_f: np.ndarray, eps: float) -> np.ndarray:
    """The step's hidden state h = bf16(RMSNorm(x)) (bits)."""
    return f64_to_bf16(gamma_f * x * rms_scale(x, eps))


def logits(E_rows: np.ndarray, h_bits: np.ndarray) -> np.ndarray:
    """Tied LM head: E h (float64) for the given embedding rows [R][D]."""
    return bf16_to_f64(E_rows) @ bf16_to_f64(h_bits)


def branch_pass(x0: np.ndarray, layers: Sequence[Dict[str, np.ndarray]], hq: int, hkv: int, head_dim: int,
                pos: int, K_hist: Sequence[np.ndarray], V_hist: Sequence[np.ndarray], S: Sequence[int],
                gamma_f: np.ndarray, theta: float, eps: float):
    """All layers of one branch for one sequence from the embedding x0.
    Returns (h bits [D], staged k_cur per layer, staged v_cur per layer,
    attention output bits per layer)."""
    x = np.asarray(x0, dtype=np.float64)
    ks, vs, os_ = [], [], []
    for l, P in enumerate(layers):
        x, kc, vc, o = decoder_layer(x, P, hq, hkv, head_dim, pos, K_hist[l], V_hist[l], S, theta, eps)
        ks.append(kc)
        vs.append(vc)
        os_.append(o)
    return final_hidden(x, gamma_f, eps), ks, vs, os_


def oda_decoder_step(token: int, E_row_bits: np.ndarray, layers, hq: int, hkv: int, head_dim: int, pos: int,
                     K_hist, V_hist, gamma_f, theta_rope: float, eps: float, head_P, h_prev_bits, theta: float,
                     force: int, logits_fn, sink: int = 4, window: int = 2048):
    """One ODA decode step of one sequence around the decoder [ODA notes
    §2.3]: the local branch from the pre-step state, the recall score of
    (h_prev, E(x_t), h^L), the full branch when the rule asks, then the
    chosen branch's next token, hidden state and staged K/V.

    E_row_bits: the embedding row of `token`.  logits_fn(h_bits) returns the
    logits over the vocabulary (the tied LM head).  Returns a dict."""
    from .oda_oracle import recall_score
    t = pos + 1
    x0 = bf16_to_f64(E_row_bits)
    hL, kL, vL, oL = branch_pass(x0, layers, hq, hkv, head_dim, pos, K_hist, V_hist,
                                 local_index_set(t, sink, window), gamma_f, theta_rope, eps)
    q = recall_score(head_P, h_prev_bits, E_row_bits, hL)
    flag = branch_rule(q, theta, force)
    rec = {"score": q, "flag": flag, "hL": hL, "kL": kL, "vL": vL, "oL": oL}
    if flag:
        hF, kF, vF, oF = branch_pass(x0, layers, hq, hkv, head_dim, pos, K_hist, V_hist, full_index_set(t),
                                     gamma_f, theta_rope, eps)
        rec.update({"hF": hF, "kF": kF, "vF": vF, "oF": oF})
        h = hF
    else:
        h = hL
    rec["h"] = h
    lg = logits_fn(h)
    rec["logits"] = lg
    rec["token"] = argmax_first(lg)
    return rec
