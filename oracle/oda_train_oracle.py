"""CPU oracle of one recall-head training step on paired branch outputs.

TEST INFRASTRUCTURE ONLY, like ``oda_oracle``: only the tests, the smoke
check and the bench's CPU baseline may import it; the product path never
does, and nothing here is shared with it.

What it computes ([ODA notes] = the page "On-Demand Attention：让语言模型按需
读取完整历史", §2.1 equation for g, §2.2 equations for d, y and the loss, and
the paragraph on paired supervision).  A micro-batch holds N positions of one
or more sequences.  For each row n the caller supplies the two candidates'
final hidden states at that position, computed from the same committed
history: h^L (local index set) and h^F (full index set), the current token
x_t and the reference next token x_{t+1}.  Then

    log p^B(x) = (E h^B)[x] - logsumexp(E h^B)      B in {L, F}; E is the
                                                     frozen tied LM head
    g   = log p^F(x_{t+1}) - log p^L(x_{t+1})      (nats)
    d   = g - lambda
    y   = sign(d) log(1 + |d|)
    row n is in the valid set E when it has a reference token, g is finite
        and the two index sets differ (t > s + w, i.e. 0-based pos >= s + w)
    h_prev(n) = 0                        at a sequence start (prev = -1)
              = h^F(prev)  if d(prev) > 0 or d(prev) is not finite
              = h^L(prev)  otherwise
    q   = R_psi(h_prev, E[x_t], h^L)    (the recall head, as in the decode step)
    L   = (1/|E|) sum over E of Huber_1(q - y)

and the step returns L and dL/dpsi for every packed head parameter; no other
parameter receives a gradient.

Readings where the pages leave a step open:
* The previous hidden state of a training row is picked "by the previous
  position's reference benefit": read here as the branch that the deployed
  rule would pick for a score equal to that row's label sign, i.e. full when
  d(prev) > 0 (non-finite counts as full, as the rule's fallback does).
* The loss is the mean over the valid rows of the micro-batch (the main
  configuration's normalisation); a micro-batch without valid rows has loss
  0 and a zero gradient.
* |x| has derivative sign(x), taken as 0 at x = 0.
* The pages name no optimiser; the step ends at the gradient.

Arithmetic: float64 throughout, from the exact widening of the bf16 inputs
and of the fp32 parameters.  The backward pass is written out by hand from
the forward below and pinned by central finite differences of the forward.
"""
from __future__ import annotations

import math
from typing import Dict, Tuple

import numpy as np

from .oda_oracle import (HEAD_EPS, SINK, WINDOW, benefit_label, bf16_to_f64,
                         head_layout)


# ---------------------------------------------------------------------------
# labels  [ODA notes §2.1 equation for g; §2.2 equations for d and y]
# ---------------------------------------------------------------------------
def log_prob(E: np.ndarray, h: np.ndarray, x: int) -> float:
    """log softmax(E h)[x] in float64; E [V][D], h [D] (float64 values)."""
    z = E @ h
    m = float(np.max(z))
    return float(z[x] - (m + math.log(float(np.sum(np.exp(z - m))))))


def gain(E: np.ndarray, h_full: np.ndarray, h_local: np.ndarray, x_next: int) -> float:
    """g = log p^F(x_{t+1}) - log p^L(x_{t+1})."""
    return log_prob(E, h_full, x_next) - log_prob(E, h_local, x_next)


def labels(E_bits, hL_bits, hF_bits, next_tok, pos, lam: float = 0.0,
           s: int = SINK, w: int = WINDOW) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Per row: gain g, label y and membership of the valid set.

    E_bits [V][D], hL_bits / hF_bits [N][D] raw bf16 bits; next_tok [N]
    (-1 = no reference token); pos [N] 0-based positions.  Rows without a
    reference token get g = y = 0 and are not valid."""
    E = bf16_to_f64(E_bits)
    hL, hF = bf16_to_f64(hL_bits), bf16_to_f64(hF_bits)
    n = hL.shape[0]
    g = np.zeros(n)
    y = np.zeros(n)
    valid = np.zeros(n, dtype=bool)
    for i in range(n):
        x = int(next_tok[i])
        if x < 0:
            continue
        g[i] = gain(E, hF[i], hL[i], x)
        if math.isfinite(g[i]):
            y[i] = benefit_label(g[i], lam)
        valid[i] = math.isfinite(g[i]) and int(pos[i]) >= s + w
    return g, y, valid


def prev_choice(g_prev: float, lam: float) -> int:
    """1 (full) or 0 (local): the branch whose state a row's successor sees."""
    d = g_prev - lam
    return 1 if (not math.isfinite(d)) or d > 0 else 0


def prev_hidden(hL: np.ndarray, hF: np.ndarray, prev, g: np.ndarray, lam: float) -> np.ndarray:
    """h_prev rows (float64) for every row: zeros at sequence starts, else the
    previous row's chosen candidate."""
    out = np.zeros_like(hL, dtype=np.float64)
    for i, p in enumerate(prev):
        p = int(p)
        if p >= 0:
            out[i] = hF[p] if prev_choice(float(g[p]), lam) else hL[p]
    return out


# ---------------------------------------------------------------------------
# head forward, batched over rows  [ODA notes §2.2, architecture paragraph]
# ---------------------------------------------------------------------------
def unpack(blob: np.ndarray, hidden: int, tower: int, ffn: int) -> Dict[str, np.ndarray]:
    """Named float64 tensors of a packed blob (fp32 widened exactly; a float64
    blob is taken as it is)."""
    blob = np.asarray(blob)
    if blob.dtype != np.float64:
        blob = blob.astype(np.float32)
    P, at = {}, 0
    for name, shape in head_layout(hidden, tower, ffn):
        k = int(np.prod(shape))
        P[name] = blob[at:at + k].astype(np.float64).reshape(shape)
        at += k
    assert at == blob.size, "head blob does not match the layout"
    return P


def pack(G: Dict[str, np.ndarray], hidden: int, tower: int, ffn: int) -> np.ndarray:
    return np.concatenate([G[name].reshape(-1) for name, _ in head_layout(hidden, tower, ffn)])


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def _silu(z):
    return z * _sigmoid(z)


def _silu_grad(z):
    s = _sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def _rms_inv(X):
    """1 / sqrt(mean(x^2) + eps) per row, shape [N][1]."""
    return 1.0 / np.sqrt(np.mean(X * X, axis=1, keepdims=True) + HEAD_EPS)


def head_forward(P: Dict[str, np.ndarray], Hp: np.ndarray, Em: np.ndarray, HL: np.ndarray):
    """q [N] and the activations the backward pass reads.  Rows are the
    batch; every weight matrix is [out][in]."""
    c = {}
    towers = []
    for s, X in (("H", Hp), ("E", Em), ("L", HL)):
        ri = _rms_inv(X)
        xn = X * ri * P[f"gamma_{s}"]
        pre = xn @ P[f"W_{s}"].T + P[f"c_{s}"]
        c[s] = (X, ri, xn, pre)
        towers.append(_silu(pre))
    a, b, cc = towers
    Z = np.concatenate([a, b, cc, a * b, a * cc, b * cc, np.abs(a - b), np.abs(a - cc), np.abs(b - cc)], axis=1)
    u = Z @ P["W_I"].T + P["c_I"] + a + b + cc
    c["abc"], c["Z"] = (a, b, cc), Z
    for k in (1, 2):
        ri = _rms_inv(u)
        r = u * ri * P[f"gamma_{k}"]
        G = r @ P[f"Wg_{k}"].T
        U = r @ P[f"Wu_{k}"].T
        M = _silu(G) * U
        c[k] = (u, ri, r, G, U, M)
        u = u + M @ P[f"Wd_{k}"].T
    ri = _rms_inv(u)
    on = u * ri * P["gamma_o"]
    q = on @ P["w_o"][0] + P["c_o"][0]
    c["o"] = (u, ri, on)
    return q, c


def _norm_backward(dY, X, ri, gamma):
    """Input gradient of Y = X * ri * gamma (ri = 1/sqrt(mean(X^2)+eps) per
    row) and the gain gradient summed over rows."""
    gdy = dY * gamma
    n = X.shape[1]
    dX = gdy * ri - X * (ri ** 3) * np.sum(gdy * X, axis=1, keepdims=True) / n
    dgamma = np.sum(dY * X * ri, axis=0)
    return dX, dgamma


def head_backward(P: Dict[str, np.ndarray], c, dq: np.ndarray) -> Dict[str, np.ndarray]:
    """dL/dpsi for every named tensor, given dL/dq per row."""
    Gd = {}
    u2, ri, on = c["o"]
    Gd["w_o"] = (dq @ on)[None, :]
    Gd["c_o"] = np.array([np.sum(dq)])
    don = dq[:, None] * P["w_o"][0][None, :]
    du, Gd["gamma_o"] = _norm_backward(don, u2, ri, P["gamma_o"])
    for k in (2, 1):
        u, ri, r, G, U, M = c[k]
        Gd[f"Wd_{k}"] = du.T @ M
        dM = du @ P[f"Wd_{k}"]
        dG = dM * U * _silu_grad(G)
        dU = dM * _silu(G)
        Gd[f"Wg_{k}"] = dG.T @ r
        Gd[f"Wu_{k}"] = dU.T @ r
        dr = dG @ P[f"Wg_{k}"] + dU @ P[f"Wu_{k}"]
        dun, Gd[f"gamma_{k}"] = _norm_backward(dr, u, ri, P[f"gamma_{k}"])
        du = du + dun
    a, b, cc = c["abc"]
    T = a.shape[1]
    Gd["W_I"] = du.T @ c["Z"]
    Gd["c_I"] = np.sum(du, axis=0)
    dZ = du @ P["W_I"]
    seg = [dZ[:, i * T:(i + 1) * T] for i in range(9)]
    sab, sac, sbc = np.sign(a - b), np.sign(a - cc), np.sign(b - cc)
    da = du + seg[0] + seg[3] * b + seg[4] * cc + seg[6] * sab + seg[7] * sac
    db = du + seg[1] + seg[3] * a + seg[5] * cc - seg[6] * sab + seg[8] * sbc
    dc = du + seg[2] + seg[4] * a + seg[5] * b - seg[7] * sac - seg[8] * sbc
    for s, dt in (("H", da), ("E", db), ("L", dc)):
        X, ri, xn, pre = c[s]
        dpre = dt * _silu_grad(pre)
        Gd[f"W_{s}"] = dpre.T @ xn
        Gd[f"c_{s}"] = np.sum(dpre, axis=0)
        dxn = dpre @ P[f"W_{s}"]
        Gd[f"gamma_{s}"] = np.sum(dxn * X * ri, axis=0)
    return Gd


# ---------------------------------------------------------------------------
# loss  [ODA notes §2.2 loss equation]
# ---------------------------------------------------------------------------
def huber_vec(r: np.ndarray) -> np.ndarray:
    a = np.abs(r)
    return np.where(a <= 1.0, 0.5 * r * r, a - 0.5)


def huber_grad(r: np.ndarray) -> np.ndarray:
    return np.where(np.abs(r) <= 1.0, r, np.sign(r))


def loss_and_dq(q: np.ndarray, y: np.ndarray, valid: np.ndarray) -> Tuple[float, np.ndarray]:
    valid = np.asarray(valid, dtype=bool)
    n = int(np.sum(valid))
    if n == 0:
        return 0.0, np.zeros_like(q)
    r = q - y
    loss = float(np.sum(huber_vec(r[valid]))) / n
    dq = np.where(valid, huber_grad(r), 0.0) / n
    return loss, dq


def head_train_step(blob: np.ndarray, hidden: int, E_bits, hL_bits, hF_bits, tokens, prev, g, y, valid,
                    lam: float = 0.0, tower: int = 1024, ffn: int = 2048):
    """Loss, q [N] and the packed gradient (float64, head blob order) of one
    micro-batch, given its labels (from ``labels``)."""
    P = unpack(blob, hidden, tower, ffn)
    hL, hF = bf16_to_f64(hL_bits), bf16_to_f64(hF_bits)
    Em = bf16_to_f64(np.asarray(E_bits)[np.asarray(tokens, dtype=np.int64)])
    Hp = prev_hidden(hL, hF, prev, g, lam)
    q, c = head_forward(P, Hp, Em, hL)
    loss, dq = loss_and_dq(q, y, valid)
    Gd = head_backward(P, c, dq)
    return loss, q, pack(Gd, hidden, tower, ffn)


def loss_of(blob: np.ndarray, hidden: int, Hp, Em, HL, y, valid, tower: int, ffn: int) -> float:
    """The loss as a function of the packed parameters alone (float64 blob
    accepted), for finite-difference pins."""
    P = unpack(np.asarray(blob, dtype=np.float64), hidden, tower, ffn)
    q, _ = head_forward(P, Hp, Em, HL)
    return loss_and_dq(q, y, valid)[0]
