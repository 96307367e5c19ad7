"""One ODA decode step of a hybrid backbone: full-attention layers on the
ODA path (include/oda.h) interleaved with recurrent layers whose states go
through the transaction of include/oda_hybrid.h.

[On-Demand Attention notes §2.3, §3.3]: only the attention layers are
restricted in the local trial; the recurrent layers run natively in both
branches, each branch from the same pre-step state, and only the chosen
branch's state is committed.  With `pattern` giving the layer order ("A" an
attention layer, "G" a recurrent layer), a step is

    in pattern order: oda_local_attn(a) / oda_gdn_step(g, LOCAL)
    oda_recall_score                      (h^L = the last attention layer's local output)
    in pattern order: oda_full_attn_if(a) / oda_gdn_step(g, FULL)
    oda_commit, oda_gdn_commit

``HybridPlan`` resolves every pointer once, so the step is a fixed list of
library calls with no host synchronisation and can be captured into a HIP
graph.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib as C
from .step import StepPlan


@dataclass
class GdnBuffers:
    """Device tensors of the recurrent layers (bf16 as int16)."""
    state: torch.Tensor      # uint8 pool of oda_gdn_state_bytes
    slot: torch.Tensor       # [B] uint8 committed slot
    xL: torch.Tensor         # [Lg][B][C] q|k|v projection, local branch
    xF: torch.Tensor
    aL: torch.Tensor         # [Lg][B][H] alpha, local branch
    bL: torch.Tensor         # [Lg][B][H] beta
    aF: torch.Tensor
    bF: torch.Tensor
    conv_w: torch.Tensor     # [Lg][C][W]
    oL: torch.Tensor         # [Lg][B][H][d] outputs
    oF: torch.Tensor

    @staticmethod
    def allocate(gd: C.oda_gdn_dims, device="cuda") -> "GdnBuffers":
        L, B, H, d, W = gd.num_layers, gd.batch, gd.heads, gd.head_dim, gd.conv_width
        Cc = 3 * H * d
        z = lambda *s, dt=torch.int16: torch.zeros(s, dtype=dt, device=device)
        return GdnBuffers(state=z(C.oda_gdn_state_bytes(gd), dt=torch.uint8), slot=z(B, dt=torch.uint8),
                          xL=z(L, B, Cc), xF=z(L, B, Cc), aL=z(L, B, H, dt=torch.float32),
                          bL=z(L, B, H, dt=torch.float32), aF=z(L, B, H, dt=torch.float32),
                          bF=z(L, B, H, dt=torch.float32), conv_w=z(L, Cc, W), oL=z(L, B, H, d), oF=z(L, B, H, d))

    def views(self, gd: C.oda_gdn_dims):
        """(recurrent [L][B][3][H][d][d] fp32, convolution [L][B][3][W-1][C] int16) views of the pool."""
        L, B, H, d, W = gd.num_layers, gd.batch, gd.heads, gd.head_dim, gd.conv_width
        off = C.oda_gdn_conv_offset(gd)
        rec = self.state[:off].view(torch.float32).view(L, B, C.ODA_GDN_SLOTS, H, d, d)
        conv = self.state[off:].view(torch.int16).view(L, B, C.ODA_GDN_SLOTS, W - 1, 3 * H * d)
        return rec, conv


class HybridPlan:
    def __init__(self, plan: StepPlan, gd: C.oda_gdn_dims, g: GdnBuffers, pattern: str, stream=None):
        if pattern.count("A") != plan.L or pattern.count("G") != gd.num_layers or pattern[-1] != "A":
            raise ValueError("pattern must name every attention and recurrent layer and end with attention")
        self.plan, self.gd, self.g, self.pattern = plan, gd, g, pattern
        lib = C.lib()
        self._lib = lib
        s = (stream or torch.cuda.current_stream()).cuda_stream
        gdp = ctypes.byref(gd)
        P = lambda t: t.data_ptr()
        flag = plan.bufs.flag
        self.local_calls, self.full_calls = [], []
        a = gi = 0
        for kind in pattern:
            if kind == "A":
                self.local_calls.append((lib.oda_local_attn, plan.local_args[a], "oda_local_attn"))
                self.full_calls.append((lib.oda_full_attn_if, plan.full_args[a], "oda_full_attn_if"))
                a += 1
            else:
                self.local_calls.append((lib.oda_gdn_step, (gdp, gi, C.ODA_GDN_LOCAL, P(g.state), P(g.slot), None,
                                                            P(g.xL[gi]), P(g.conv_w[gi]), P(g.aL[gi]),
                                                            P(g.bL[gi]), P(g.oL[gi]), s), "oda_gdn_step"))
                self.full_calls.append((lib.oda_gdn_step, (gdp, gi, C.ODA_GDN_FULL, P(g.state), P(g.slot), P(flag),
                                                           P(g.xF[gi]), P(g.conv_w[gi]), P(g.aF[gi]),
                                                           P(g.bF[gi]), P(g.oF[gi]), s), "oda_gdn_step"))
                gi += 1
        self.gdn_commit_args = (gdp, P(g.slot), P(flag), s)

    @staticmethod
    def _run(calls) -> None:
        for f, args, name in calls:
            C.check(f(*args), name)

    def local(self) -> None:
        self._run(self.local_calls)

    def score(self) -> None:
        self.plan.score()

    def full(self) -> None:
        self._run(self.full_calls)

    def commit(self) -> None:
        self.plan.commit()
        C.check(self._lib.oda_gdn_commit(*self.gdn_commit_args), "oda_gdn_commit")

    def run(self) -> None:
        """One whole decode step on the plan's stream."""
        self.local()
        self.score()
        self.full()
        self.commit()
