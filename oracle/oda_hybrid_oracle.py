"""CPU oracle of the recurrent-state transaction of a hybrid backbone.

TEST INFRASTRUCTURE ONLY, like ``oda_oracle``: only the tests, the smoke
check and the bench's CPU baseline may import it; the product path never
does, and nothing here is shared with it.

What the pages fix ([ODA notes] = the page "On-Demand Attention：让语言模型按需
读取完整历史", §2.3 state-commit paragraph and equation C_t; §3.3 cross-model
paragraph).  In a hybrid backbone only the full-attention layers are
restricted to S^L; the recurrent layers (Gated DeltaNet in the pages' model)
keep their native computation in both branches.  Their convolution and
recurrent states must be saved before the local trial and restored before the
full retry, so that both candidates start from the same pre-step state; only
the chosen branch's update is committed (C_t = C_{t-1} || dC^{b_t}, where ||
also applies the recurrent update).  Advancing the state twice (local, then
full on top of it) is the failure the transaction prevents.

What the pages leave open, and the reading taken here (a standard gated
delta rule decode layer):
* one layer holds, per sequence and head, a state S in R^{d_v x d_k} (fp32)
  and a causal depthwise convolution of width W over the C = 3 H d channels
  of the layer's q | k | v projection, whose state is the last W - 1 inputs;
* a step takes the projection x_t [C] (bf16) and per-head gates
  alpha_t in (0, 1], beta_t in (0, 1) (fp32), and computes
      c      = sum_{j < W-1} w[:, j] * s_j + w[:, W-1] * x_t   (s_0 oldest)
      q, k, v = SiLU(c) split by channel group, per head
      q^ = q / sqrt(|q|^2 + eps), k^ = k / sqrt(|k|^2 + eps)
      S'     = alpha S + beta (v - alpha S k^) k^T
             (= S alpha (I - beta k^ k^T) + beta v k^T)
      o      = S' q^ / sqrt(d_k)
  and the new convolution state (s_1, ..., s_{W-2}, x_t);
* per sequence the pool keeps three state slots; the committed slot c holds
  the pre-step state, the local trial writes slot (c + 1) mod 3, the full
  retry writes slot (c + 2) mod 3, both reading slot c, and the commit moves
  c to the chosen branch's slot.  (That is the GPU library's layout; the
  oracle below keeps explicit copies instead, the plain form of "save,
  restore, commit".)

Arithmetic: float64 from the exact widening of the bf16 inputs and of the
fp32 state, gates and weights.
"""
from __future__ import annotations

import copy
import math
from typing import Dict, List, Tuple

import numpy as np

from .oda_oracle import bf16_to_f64

GDN_EPS = 1e-6        # L2-norm epsilon (reading)


def silu(x):
    return x / (1.0 + np.exp(-x))


def l2_normalise(x: np.ndarray) -> np.ndarray:
    return x / math.sqrt(float(np.dot(x, x)) + GDN_EPS)


def conv_step(conv_state: np.ndarray, x: np.ndarray, w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Causal depthwise convolution of width W for one step.

    conv_state [W-1][C] (oldest first), x [C], w [C][W] -> (output [C],
    new state)."""
    W = w.shape[1]
    window = np.concatenate([conv_state, x[None, :]], axis=0)     # [W][C], oldest first
    y = np.sum(window.T * w, axis=1)
    return y, window[1:].copy() if W > 1 else conv_state.copy()


def delta_update(S: np.ndarray, k: np.ndarray, v: np.ndarray, alpha: float, beta: float) -> np.ndarray:
    """S' = S alpha (I - beta k k^T) + beta v k^T, written as the product."""
    dk = k.shape[0]
    return S @ (alpha * (np.eye(dk) - beta * np.outer(k, k))) + beta * np.outer(v, k)


def gdn_layer_step(S: np.ndarray, conv_state: np.ndarray, x_bits, w_bits, alpha, beta):
    """One decode step of one recurrent layer for one sequence.

    S [H][d_v][d_k] float64, conv_state [W-1][C] float64, x_bits [C] and
    w_bits [C][W] bf16 bits, alpha / beta [H].  Returns (o [H][d_v] float64,
    S', conv_state')."""
    H, dv, dk = S.shape
    x = bf16_to_f64(x_bits)
    w = bf16_to_f64(w_bits)
    y, conv_new = conv_step(conv_state, x, w)
    a = silu(y)
    o = np.zeros((H, dv))
    S_new = np.empty_like(S)
    for h in range(H):
        q = l2_normalise(a[h * dk:(h + 1) * dk])
        k = l2_normalise(a[H * dk + h * dk:H * dk + (h + 1) * dk])
        v = a[2 * H * dk + h * dv:2 * H * dk + (h + 1) * dv]
        S_new[h] = delta_update(S[h], k, v, float(alpha[h]), float(beta[h]))
        o[h] = S_new[h] @ q / math.sqrt(dk)
    return o, S_new, conv_new


class HybridState:
    """Committed recurrent and convolution states of every recurrent layer
    of one sequence (explicit arrays; the transaction copies them)."""

    def __init__(self, S: List[np.ndarray], conv: List[np.ndarray]):
        self.S = [np.asarray(s, dtype=np.float64) for s in S]
        self.conv = [np.asarray(c, dtype=np.float64) for c in conv]

    def copy(self) -> "HybridState":
        return copy.deepcopy(self)


def branch_pass(state: HybridState, inputs, w_bits) -> Tuple[List[np.ndarray], HybridState]:
    """Run every recurrent layer of one branch from `state` (not modified).

    inputs[l] = (x_bits, alpha, beta); w_bits[l] the layer's conv weights.
    Returns the per-layer outputs and the branch's candidate state."""
    cand = state.copy()
    outs = []
    for l, (x, al, be) in enumerate(inputs):
        o, cand.S[l], cand.conv[l] = gdn_layer_step(cand.S[l], cand.conv[l], x, w_bits[l], al, be)
        outs.append(o)
    return outs, cand


def transaction_step(state: HybridState, local_inputs, full_inputs, w_bits, flag: int):
    """One step of the transaction [ODA notes §2.3]: save the pre-step state,
    run the local trial from it, restore it and run the full retry when the
    rule asks, commit the chosen branch's state.  Returns (local outputs,
    full outputs or None, the new committed state)."""
    saved = state.copy()                                   # snapshot before the local trial
    out_l, cand_l = branch_pass(state, local_inputs, w_bits)
    if not flag:
        return out_l, None, cand_l
    restored = saved.copy()                                # restore before the full retry
    out_f, cand_f = branch_pass(restored, full_inputs, w_bits)
    return out_l, out_f, cand_f


def double_advance(state: HybridState, local_inputs, full_inputs, w_bits):
    """The failure the transaction prevents: the full retry run on top of the
    local trial's state.  Used only to show that the tests tell the two
    apart."""
    _, cand_l = branch_pass(state, local_inputs, w_bits)
    out_f, cand_f = branch_pass(cand_l, full_inputs, w_bits)
    return out_f, cand_f
