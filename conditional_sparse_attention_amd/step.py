"""One ODA decode step: the four library calls in their required order.

[On-Demand Attention notes §2.3]: run the local forward, score it, recompute
the full branch only where the rule asks, then commit the chosen branch.
Here the "forward" is the attention of every layer (the step's q, k, v per
layer and branch are inputs), so one step is

    oda_local_attn(l)   for l in 0..L-1
    oda_recall_score    (h_prev, emb, local output of layer L-1)
    oda_full_attn_if(l) for l in 0..L-1   (device-side work list)
    oda_commit          (cache slot, h_prev, pos += 1)

``StepPlan`` resolves every pointer once and replays the calls with
pre-built ctypes arguments, so a step costs ~2L+2 foreign calls and no
Python-side marshalling; it can also be captured into a HIP graph.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib as C


@dataclass
class StepBuffers:
    """Device tensors of one step.  Per-layer tensors are [L][B][H][d]."""
    pos: torch.Tensor        # [B] int32, in/out
    qL: torch.Tensor
    kL: torch.Tensor
    vL: torch.Tensor
    qF: torch.Tensor
    kF: torch.Tensor
    vF: torch.Tensor
    emb: torch.Tensor        # [B][D] bf16 bits (int16 storage)
    h_prev: torch.Tensor     # [B][D], in/out
    head_w: torch.Tensor     # packed fp32
    oL: torch.Tensor         # [L][B][Hq][d]
    oF: torch.Tensor
    score: torch.Tensor      # [B] float32
    flag: torch.Tensor       # [B] uint8
    force: Optional[torch.Tensor] = None   # [B] int8 or None
    lseL: Optional[torch.Tensor] = None    # [L][B][Hq] float32 or None
    lseF: Optional[torch.Tensor] = None


class StepPlan:
    def __init__(self, dims: C.oda_dims, kv: C.oda_kv, ws: torch.Tensor, bufs: StepBuffers, theta: float,
                 stream: Optional[torch.cuda.Stream] = None):
        self.dims, self.kv, self.ws, self.bufs = dims, kv, ws, bufs
        self.theta = float(theta)
        self.L = dims.num_layers
        lib = C.lib()
        self._lib = lib
        b = bufs
        dp, kp = ctypes.byref(dims), ctypes.byref(kv)
        wsb = ws.numel() * ws.element_size()

        def ptr(t, l=None):
            if t is None:
                return None
            return (t[l] if l is not None else t).data_ptr()

        self._stream_handle = (stream or torch.cuda.current_stream()).cuda_stream
        s = self._stream_handle
        self.local_args = [(dp, l, kp, ptr(b.pos), ptr(b.qL, l), ptr(b.kL, l), ptr(b.vL, l), ptr(b.oL, l),
                            ptr(b.lseL, l) if b.lseL is not None else None, ptr(ws), wsb, s) for l in range(self.L)]
        self.score_args = (dp, ptr(b.head_w), ptr(b.h_prev), ptr(b.emb), ptr(b.oL, self.L - 1),
                           ctypes.c_float(self.theta), ptr(b.force), ptr(b.pos), ptr(b.score), ptr(b.flag),
                           ptr(ws), wsb, s)
        self.full_args = [(dp, l, kp, ptr(b.pos), ptr(b.qF, l), ptr(b.kF, l), ptr(b.vF, l), ptr(b.oF, l),
                           ptr(b.lseF, l) if b.lseF is not None else None, ptr(ws), wsb, s) for l in range(self.L)]
        self.commit_args = (dp, kp, ptr(b.pos), ptr(b.flag), ptr(b.kL), ptr(b.vL), ptr(b.kF), ptr(b.vF),
                            ptr(b.oL, self.L - 1), ptr(b.oF, self.L - 1), ptr(b.h_prev), ptr(ws), wsb, s)

    def set_theta(self, theta: float) -> None:
        self.theta = float(theta)
        a = list(self.score_args)
        a[5] = ctypes.c_float(self.theta)
        self.score_args = tuple(a)

    def local(self) -> None:
        f = self._lib.oda_local_attn
        for a in self.local_args:
            C.check(f(*a), "oda_local_attn")

    def score(self) -> None:
        C.check(self._lib.oda_recall_score(*self.score_args), "oda_recall_score")

    def full(self) -> None:
        f = self._lib.oda_full_attn_if
        for a in self.full_args:
            C.check(f(*a), "oda_full_attn_if")

    def commit(self) -> None:
        C.check(self._lib.oda_commit(*self.commit_args), "oda_commit")

    def run(self) -> None:
        """One whole decode step on the plan's stream."""
        self.local()
        self.score()
        self.full()
        self.commit()


def tune_theta(scores, rate: float) -> float:
    """Threshold that sends a fraction `rate` of the given recall scores to
    the full branch under the strict rule q > theta [On-Demand Attention
    notes §2.3]: the midpoint between the k-th and (k+1)-th largest score,
    k = round(rate * n).  k = 0 gives +inf (never full), k = n gives -inf.
    The pages treat the threshold as a tunable knob; this is how a target
    call rate is turned into one from a calibration pass (all-local scores)."""
    import math

    import numpy as np

    sc = np.sort(np.asarray(scores, dtype=np.float64).reshape(-1))[::-1]
    k = int(round(rate * sc.size))
    if k <= 0:
        return math.inf
    if k >= sc.size:
        return -math.inf
    return float((sc[k - 1] + sc[k]) / 2)


def match_rate(run_pass, theta0: float, rate: float, max_passes: int = 12):
    """Threshold whose own trajectory sends round(rate * n) of its n
    decisions to the full branch.  theta0 comes from an all-local
    calibration pass (tune_theta); once sequences take the full branch their
    hidden states and caches change, so the later scores, and the realised
    count, drift away from it.  run_pass(theta) runs the steps from the same
    start state with threshold theta and returns (recall scores, flags), one
    entry per decision.  Each further pass takes the threshold that would
    have hit the count on the previous pass's own scores, kept strictly
    between the thresholds found so far to send too many and too few (their
    midpoint when it falls outside).  Returns (theta, realised count, target
    count, passes run), theta being the first of the passes closest to the
    target."""
    import math

    import numpy as np

    theta, lo, hi = float(theta0), -math.inf, math.inf
    best, passes = None, 0
    while True:
        scores, flags = run_pass(theta)
        passes += 1
        n = int(np.count_nonzero(flags))
        k = int(round(rate * np.asarray(flags).size))
        if best is None or abs(n - k) < abs(best[1] - k):
            best = (theta, n, k)
        if n == k or passes >= max_passes:
            break
        if n > k:
            lo = max(lo, theta)
        else:
            hi = min(hi, theta)
        cand = tune_theta(scores, rate)
        inside = (cand > lo or cand == lo == -math.inf) and (cand < hi or cand == hi == math.inf)
        if not inside:
            if not (math.isfinite(lo) and math.isfinite(hi)):
                break
            cand = (lo + hi) / 2
        if cand == theta:
            break
        theta = cand
    return best[0], best[1], best[2], passes
