"""CPU oracle of the On-Demand Attention (ODA) decode step.

TEST INFRASTRUCTURE ONLY.  This is a plain, slow, obviously correct float64
restatement of what one ODA decode step computes.  Only the test suite, the
smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the product path (the HIP library and its Python
binding) never calls, links or imports anything here, and shares no code
with it.

Source of every definition: the page "On-Demand Attention：让语言模型按需读取
完整历史" (notes on arXiv 2609.20734, checked against the full paper), cited
below as [ODA notes] with its section and equation.  Cross-checks come from
"On-Demand Attention：模型知道自己什么时候需要回头看" (zhichai.net), cited as
[ODA explainer].

Conventions
-----------
* The pages count positions from 1; here position index i (0-based) is the
  page's position i+1, and ``pos`` = committed length, so the current token
  is index ``pos`` and the page's t equals ``pos + 1``.
* bf16 values arrive as raw uint16 bits and are widened to float64 exactly.
* No tiling, no online rescaling, no fusion: each function computes its
  definition directly, using numpy matmul / sum as library primitives.

Parity status of each function is stated in its docstring.  Every function
here is pinned by a test in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

SINK = 4          # s  [ODA notes §2.1, definition of S^L]
WINDOW = 2048     # w  [ODA notes §2.1]; the window counts the current token
THETA_DEFAULT = 0.0   # [ODA notes §2.3] full recompute when the score exceeds zero
HEAD_TOWER = 1024     # [ODA notes §2.2] towers map each input to 1024 dims
HEAD_FFN = 2048       # gated FFN hidden width (reading: see head_layout)
HEAD_EPS = 1e-6       # RMSNorm epsilon (reading)


# ---------------------------------------------------------------------------
# numeric helpers
# ---------------------------------------------------------------------------
def bf16_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(x) -> np.ndarray:
    """Round float64 to bf16 bits, nearest-even (via an exact float32 step is
    not exact, so round directly from the float64 value)."""
    x = np.asarray(x, dtype=np.float64)
    f32 = x.astype(np.float32)
    u = f32.view(np.uint32).astype(np.uint64)
    # candidates: truncation toward zero and one bf16 ulp away from zero
    lo = (u >> np.uint64(16)).astype(np.uint64)
    hi = lo + np.uint64(1)
    lo_v = bf16_to_f64(lo.astype(np.uint16))
    hi_v = bf16_to_f64(hi.astype(np.uint16))
    d_lo = np.abs(x - lo_v)
    d_hi = np.abs(x - hi_v)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((lo & np.uint64(1)) == np.uint64(1)))
    out = np.where(pick_hi, hi, lo).astype(np.uint16)
    return np.where(np.isfinite(x), out, f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------------------
# index sets  [ODA notes §2.1, equation for S^F and S^L]
# ---------------------------------------------------------------------------
def full_index_set(t: int) -> np.ndarray:
    """S^F_t = {1..t}, returned as ascending 0-based indices.

    Pinned: closed-form sizes and the sets' first difference (tests)."""
    return np.arange(t, dtype=np.int64)


def local_index_set(t: int, s: int = SINK, w: int = WINDOW) -> np.ndarray:
    """S^L_t = {1..min(s,t)} ∪ {max(1, t-w+1)..t}, as ascending 0-based indices.

    Written as the literal set union of the page's two 1-based ranges; the
    window therefore includes the current position t.  Pinned: the page says
    the sets first differ at position 2053 for s=4, w=2048 (tests)."""
    if t < 1:
        raise ValueError("t must be >= 1")
    sink = set(range(1, min(s, t) + 1))
    window = set(range(max(1, t - w + 1), t + 1))
    return np.array(sorted(sink | window), dtype=np.int64) - 1


# ---------------------------------------------------------------------------
# attention  [ODA notes §2.1, equation for o_t]
# ---------------------------------------------------------------------------
def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, S: Sequence[int]) -> np.ndarray:
    """o = softmax(q K[S]^T / sqrt(d_k)) V[S] for one query head, float64.

    q: [d]; K, V: [n][d] (the tilde cache: committed history followed by the
    current token's key/value); S: indices into the rows of K, V.
    Two passes: scores, then max-shifted exponentials and their normalised
    weighted sum.  Pinned against torch's float64 scaled-dot-product attention
    and closed-form special cases (tests)."""
    q = np.asarray(q, dtype=np.float64)
    S = np.asarray(S, dtype=np.int64)
    Ks = np.asarray(K, dtype=np.float64)[S]
    Vs = np.asarray(V, dtype=np.float64)[S]
    d_k = q.shape[-1]
    x = (Ks @ q) / math.sqrt(d_k)
    m = np.max(x)
    wts = np.exp(x - m)
    Z = np.sum(wts)
    return (wts @ Vs) / Z


def log_sum_exp_scores(q: np.ndarray, K: np.ndarray, S: Sequence[int]) -> float:
    """log sum_i exp(q.K[i]/sqrt(d_k)) over S (natural log), float64."""
    q = np.asarray(q, dtype=np.float64)
    Ks = np.asarray(K, dtype=np.float64)[np.asarray(S, dtype=np.int64)]
    x = (Ks @ q) / math.sqrt(q.shape[-1])
    m = np.max(x)
    return float(m + np.log(np.sum(np.exp(x - m))))


def kv_group(h: int, hq: int, hkv: int) -> int:
    """Grouped-query mapping: consecutive query heads share one KV head.
    The page omits head indices; this is the standard GQA reading."""
    return h // (hq // hkv)


def tilde(history: np.ndarray, current: np.ndarray) -> np.ndarray:
    """K~_t: the committed rows [0, pos) followed by the current token's row."""
    return np.concatenate([np.asarray(history), np.asarray(current)[None, :]], axis=0)


def decode_attention(q: np.ndarray, K_hist: np.ndarray, V_hist: np.ndarray,
                     k_cur: np.ndarray, v_cur: np.ndarray, S: Sequence[int]) -> np.ndarray:
    """All query heads of one sequence and one layer.

    q: [Hq][d] bf16 bits or floats; K_hist, V_hist: [Hkv][pos][d] committed
    history; k_cur, v_cur: [Hkv][d] the branch's own staged current key/value.
    Returns [Hq][d] float64."""
    q = _as_f64(q)
    hq, hkv = q.shape[0], K_hist.shape[0]
    out = np.empty((hq, q.shape[1]), dtype=np.float64)
    for h in range(hq):
        g = kv_group(h, hq, hkv)
        Kt = tilde(_as_f64(K_hist[g]), _as_f64(k_cur[g]))
        Vt = tilde(_as_f64(V_hist[g]), _as_f64(v_cur[g]))
        out[h] = attention(q[h], Kt, Vt, S)
    return out


def _as_f64(x) -> np.ndarray:
    x = np.asarray(x)
    return bf16_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)


# ---------------------------------------------------------------------------
# recall head  [ODA notes §2.2, equation for q_t and the architecture paragraph]
# ---------------------------------------------------------------------------
def head_layout(hidden: int, tower: int = HEAD_TOWER, ffn: int = HEAD_FFN) -> List[Tuple[str, tuple]]:
    """Packed fp32 parameter order of the recall head R_psi.

    Reading of the page's description (three independent towers of norm,
    projection and activation to 1024 dims; a 9216-dim interaction of the
    three raw vectors, their pairwise products and pairwise absolute
    differences; a projection with residual fusion; two residual gated
    feed-forward blocks; a scalar output), sized so that the total is the
    page's 28,325,889 parameters at hidden 2048:
      towers   3 x [gamma (D), W (T x D), c (T)]
      interact W_I (T x 9T), c_I (T)
      ffn      2 x [gamma (T), W_gate (F x T), W_up (F x T), W_down (T x F)]
      out      gamma_o (T), w_o (1 x T), c_o (1)
    Matrices are row-major [out][in]."""
    t, f, D = tower, ffn, hidden
    lay: List[Tuple[str, tuple]] = []
    for s in ("H", "E", "L"):
        lay += [(f"gamma_{s}", (D,)), (f"W_{s}", (t, D)), (f"c_{s}", (t,))]
    lay += [("W_I", (t, 9 * t)), ("c_I", (t,))]
    for k in (1, 2):
        lay += [(f"gamma_{k}", (t,)), (f"Wg_{k}", (f, t)), (f"Wu_{k}", (f, t)), (f"Wd_{k}", (t, f))]
    lay += [("gamma_o", (t,)), ("w_o", (1, t)), ("c_o", (1,))]
    return lay


def head_param_count(hidden: int, tower: int = HEAD_TOWER, ffn: int = HEAD_FFN) -> int:
    return int(sum(int(np.prod(s)) for _, s in head_layout(hidden, tower, ffn)))


def unpack_head(blob: np.ndarray, hidden: int, tower: int = HEAD_TOWER,
                ffn: int = HEAD_FFN) -> Dict[str, np.ndarray]:
    """Split a packed fp32 blob into float64 tensors (exact widening)."""
    blob = np.asarray(blob, dtype=np.float32)
    lay = head_layout(hidden, tower, ffn)
    n = sum(int(np.prod(s)) for _, s in lay)
    if blob.size != n:
        raise ValueError(f"head blob has {blob.size} floats, layout needs {n}")
    P, at = {}, 0
    for name, shape in lay:
        k = int(np.prod(shape))
        P[name] = blob[at:at + k].astype(np.float64).reshape(shape)
        at += k
    return P


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float = HEAD_EPS) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gamma."""
    x = np.asarray(x, dtype=np.float64)
    return x / math.sqrt(float(np.mean(x * x)) + eps) * gamma


def silu(x: np.ndarray) -> np.ndarray:
    """x * sigmoid(x)."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def tower(x: np.ndarray, gamma, W, c) -> np.ndarray:
    """One input tower: norm, projection, activation."""
    return silu(W @ rms_norm(x, gamma) + c)


def interaction(a: np.ndarray, b: np.ndarray, c: np.ndarray) -> np.ndarray:
    """The 9T-dim interaction: the three raw vectors, the pairwise products
    and the pairwise absolute differences, in the order
    [a, b, c, a*b, a*c, b*c, |a-b|, |a-c|, |b-c|]."""
    return np.concatenate([a, b, c, a * b, a * c, b * c, np.abs(a - b), np.abs(a - c), np.abs(b - c)])


def gated_ffn_block(u: np.ndarray, gamma, Wg, Wu, Wd) -> np.ndarray:
    """Residual gated feed-forward block: u + W_down(silu(W_gate r) * (W_up r)),
    r = rmsnorm(u)."""
    r = rms_norm(u, gamma)
    return u + Wd @ (silu(Wg @ r) * (Wu @ r))


def recall_score(P: Dict[str, np.ndarray], h_prev, emb, h_local) -> float:
    """q_t = R_psi(h_{t-1}, E(x_t), h_t^L), float64 from fp32 weights.

    h_prev: the previous step's chosen hidden state; emb: the current token's
    embedding; h_local: this step's local-branch hidden state.  All [D]."""
    a = tower(_as_f64(h_prev), P["gamma_H"], P["W_H"], P["c_H"])
    b = tower(_as_f64(emb), P["gamma_E"], P["W_E"], P["c_E"])
    c = tower(_as_f64(h_local), P["gamma_L"], P["W_L"], P["c_L"])
    u = P["W_I"] @ interaction(a, b, c) + P["c_I"] + (a + b + c)
    for k in (1, 2):
        u = gated_ffn_block(u, P[f"gamma_{k}"], P[f"Wg_{k}"], P[f"Wu_{k}"], P[f"Wd_{k}"])
    return float((P["w_o"] @ rms_norm(u, P["gamma_o"]))[0] + P["c_o"][0])


# ---------------------------------------------------------------------------
# branch rule  [ODA notes §2.3, first paragraph]
# ---------------------------------------------------------------------------
def branch_rule(q: float, theta: float = THETA_DEFAULT, force: int = -1) -> int:
    """1 = full branch, 0 = local branch.

    The full branch runs when the score exceeds the threshold (strictly), and
    a non-finite score falls back to full.  The head runs in fp32 [ODA notes
    §3.3], so the comparison is taken on the score rounded to fp32.  A forced
    flag (force >= 0, used for controlled schedules such as the random-call
    policy of §3.2) overrides the head."""
    if force >= 0:
        return 1 if force else 0
    q32 = np.float32(q)
    if not np.isfinite(q32):
        return 1
    return 1 if q32 > np.float32(theta) else 0


# ---------------------------------------------------------------------------
# work list for the conditional full branch
# ---------------------------------------------------------------------------
def full_worklist(flags: Sequence[int], nsplit: Sequence[int],
                  lengths: Sequence[int] = None) -> List[Tuple[int, int]]:
    """Compacted work list of the conditional full branch: the splits
    0..nsplit[b]-1 of every flagged sequence b.  How many splits a sequence
    is cut into, and the order in which sequences are listed, are kernel
    scheduling choices, not the method: the counts are passed in, and with
    `lengths` (t_b = keys of sequence b) the sequences are listed longest
    unit first, by ceil(t_b / nsplit[b]) descending with ties by ascending
    b; without it, by ascending b.  Pinned by brute force (tests)."""
    seqs = [b for b, f in enumerate(flags) if f]
    if lengths is not None:
        unit = {b: -(-int(lengths[b]) // int(nsplit[b])) if int(nsplit[b]) > 0 else 0 for b in seqs}
        seqs.sort(key=lambda b: (-unit[b], b))
    items: List[Tuple[int, int]] = []
    for b in seqs:
        for s in range(int(nsplit[b])):
            items.append((b, s))
    return items


# ---------------------------------------------------------------------------
# commit  [ODA notes §2.3, equation h_t = h_t^{b_t}, C_t = C_{t-1} || dC^{b_t}]
# ---------------------------------------------------------------------------
def commit(K: np.ndarray, V: np.ndarray, pos: np.ndarray, flags: Sequence[int],
           kL: np.ndarray, vL: np.ndarray, kF: np.ndarray, vF: np.ndarray,
           oL_last: np.ndarray, oF_last: np.ndarray):
    """Append the chosen branch's staged K/V and carry its hidden state.

    K, V: [L][B][Hkv][T][d] bf16 bits (logical positions); kL..vF:
    [L][B][Hkv][d]; oL_last, oF_last: [B][D] bf16 bits of the last layer's
    outputs.  Returns (K', V', pos', h_prev) as new arrays: slot pos_b of every
    layer receives the chosen branch's staged row, h_prev_b is the chosen
    branch's output, pos_b grows by one.  Output and cache always come from
    the same branch."""
    K2, V2, pos2 = K.copy(), V.copy(), np.asarray(pos).copy()
    h = np.empty_like(oL_last)
    for b, f in enumerate(flags):
        p = int(pos[b])
        src_k, src_v, src_o = (kF, vF, oF_last) if f else (kL, vL, oL_last)
        K2[:, b, :, p, :] = src_k[:, b]
        V2[:, b, :, p, :] = src_v[:, b]
        h[b] = src_o[b]
        pos2[b] = p + 1
    return K2, V2, pos2, h


# ---------------------------------------------------------------------------
# training-side utilities  [ODA notes §2.1 eq. g, §2.2 eqs. d, y, L]
# ---------------------------------------------------------------------------
def penalised_benefit(g: float, lam: float) -> float:
    """d_t = g_t - lambda."""
    return g - lam


def benefit_label(g: float, lam: float = 0.0) -> float:
    """y_t = sign(d_t) * log(1 + |d_t|), d_t = g_t - lambda (natural log)."""
    d = penalised_benefit(g, lam)
    return math.copysign(math.log1p(abs(d)), d) if d != 0 else 0.0


def huber(r: float, delta: float = 1.0) -> float:
    """Huber loss with threshold delta: quadratic inside, linear outside."""
    a = abs(r)
    return 0.5 * r * r if a <= delta else delta * (a - 0.5 * delta)


def huber_loss(q: Sequence[float], y: Sequence[float], valid: Sequence[bool]) -> float:
    """Mean Huber(delta=1) of q - y over the valid set E (labels finite and
    local set different from full set)."""
    terms = [huber(qi - yi) for qi, yi, v in zip(q, y, valid) if v]
    if not terms:
        return 0.0
    return sum(terms) / len(terms)


def label_valid(t: int, g: float, s: int = SINK, w: int = WINDOW) -> bool:
    """Position t (1-based) belongs to E when its label is finite and its
    local index set differs from the full one (t > s + w)."""
    return math.isfinite(g) and t > s + w
