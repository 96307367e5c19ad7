"""One ODA decode step with the dense decoder backbone around the path.

[On-Demand Attention notes §2.3]: the local branch runs the whole model with
local attention, the recall head scores (h_{t-1}, E(x_t), h^L), the full
branch reruns the whole model from the same pre-step state where the rule
asks, and the chosen branch's token, hidden state and K/V are committed.
With include/oda_decoder.h that is

    oda_dec_embed                            x_L = x_F = E[token], e = E[token]
    oda_dec_layer(l, LOCAL)   l = 0..L-1     (oda_local_attn inside)
    oda_dec_final_norm(LOCAL)                h^L
    oda_recall_score(h_prev, e, h^L)         rule + work list
    oda_dec_layer(l, FULL)    l = 0..L-1     (oda_full_attn_if inside; no work when nothing is flagged)
    oda_dec_final_norm(FULL)                 h^F
    oda_dec_next_token                       argmax of E h^{b_t}
    oda_commit                               cache slot, h_prev, pos += 1

``DecoderPlan`` resolves every pointer once; a step is a fixed sequence of
library calls with no host synchronisation, so it can be captured into a HIP
graph.  The next step's token is written on the device by the previous one.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib as C


@dataclass
class DecoderWeights:
    layers: torch.Tensor     # [L][layer numel] bf16 bits (int16 storage)
    embed: torch.Tensor      # [V][D] bf16 bits, also the tied LM head
    gamma_f: torch.Tensor    # [D] bf16 bits


@dataclass
class DecoderBuffers:
    """Device state and scratch of the decoder step (bf16 as int16)."""
    tokens: torch.Tensor     # [B] int32, in/out: this step's tokens, then the next
    pos: torch.Tensor        # [B] int32, in/out
    h_prev: torch.Tensor     # [B][D], in/out
    head_w: torch.Tensor     # packed fp32 recall head
    xL: torch.Tensor         # [B][D] fp32 residual streams
    xF: torch.Tensor
    emb: torch.Tensor        # [B][D]  E(x_t)
    q: torch.Tensor          # [B][Hq][d] scratch
    oL: torch.Tensor         # [B][Hq][d] attention output of the current layer
    oF: torch.Tensor
    kL: torch.Tensor         # [L][B][Hkv][d] staged current K/V of each branch
    vL: torch.Tensor
    kF: torch.Tensor
    vF: torch.Tensor
    hL: torch.Tensor         # [B][D] step hidden states of each branch
    hF: torch.Tensor
    score: torch.Tensor      # [B] fp32
    flag: torch.Tensor       # [B] uint8
    max_logit: torch.Tensor  # [B] fp32
    force: Optional[torch.Tensor] = None   # [B] int8 or None

    @staticmethod
    def allocate(dd: C.oda_dec_dims, head_w: torch.Tensor, tokens: torch.Tensor, pos: torch.Tensor,
                 h_prev: torch.Tensor, device="cuda") -> "DecoderBuffers":
        a = dd.attn
        L, B, Hq, Hkv, d, D = a.num_layers, a.batch, a.num_q_heads, a.num_kv_heads, a.head_dim, a.hidden
        z = lambda *s, dt=torch.int16: torch.zeros(s, dtype=dt, device=device)
        return DecoderBuffers(tokens=tokens, pos=pos, h_prev=h_prev, head_w=head_w, xL=z(B, D, dt=torch.float32),
                              xF=z(B, D, dt=torch.float32), emb=z(B, D), q=z(B, Hq, d), oL=z(B, Hq, d),
                              oF=z(B, Hq, d), kL=z(L, B, Hkv, d), vL=z(L, B, Hkv, d), kF=z(L, B, Hkv, d),
                              vF=z(L, B, Hkv, d), hL=z(B, D), hF=z(B, D), score=z(B, dt=torch.float32),
                              flag=z(B, dt=torch.uint8), max_logit=z(B, dt=torch.float32),
                              force=torch.full((B,), -1, dtype=torch.int8, device=device))


class DecoderPlan:
    def __init__(self, dd: C.oda_dec_dims, kv: C.oda_kv, weights: DecoderWeights, bufs: DecoderBuffers,
                 ws: torch.Tensor, dws: torch.Tensor, theta: float, stream: Optional[torch.cuda.Stream] = None):
        self.dd, self.kv, self.w, self.b, self.ws, self.dws = dd, kv, weights, bufs, ws, dws
        self.theta = float(theta)
        self.L = dd.attn.num_layers
        lib = C.lib()
        self._lib = lib
        b, w = bufs, weights
        ddp, dp, kp = ctypes.byref(dd), ctypes.byref(dd.attn), ctypes.byref(kv)
        wsb, dwsb = ws.numel() * ws.element_size(), dws.numel() * dws.element_size()
        s = (stream or torch.cuda.current_stream()).cuda_stream
        P = lambda t: None if t is None else t.data_ptr()
        self.embed_args = (ddp, P(w.embed), P(b.tokens), P(b.xL), P(b.xF), P(b.emb), P(ws), wsb, s)
        self.layer_args = {br: [(ddp, l, br, P(w.layers[l]), kp, P(b.pos), P(b.xL if br == 0 else b.xF), P(b.q),
                                 P((b.kL if br == 0 else b.kF)[l]), P((b.vL if br == 0 else b.vF)[l]),
                                 P(b.oL if br == 0 else b.oF), P(ws), wsb, P(dws), dwsb, s) for l in range(self.L)]
                           for br in (C.ODA_DEC_LOCAL, C.ODA_DEC_FULL)}
        self.norm_args = {br: (ddp, br, P(w.gamma_f), P(b.xL if br == 0 else b.xF), P(b.hL if br == 0 else b.hF),
                               P(ws), wsb, s) for br in (C.ODA_DEC_LOCAL, C.ODA_DEC_FULL)}
        self.score_args = (dp, P(b.head_w), P(b.h_prev), P(b.emb), P(b.hL), ctypes.c_float(self.theta), P(b.force),
                           P(b.pos), P(b.score), P(b.flag), P(ws), wsb, s)
        self.token_args = (ddp, P(w.embed), P(b.hL), P(b.hF), P(b.flag), P(b.tokens), P(b.max_logit), P(dws), dwsb, s)
        self.commit_args = (dp, kp, P(b.pos), P(b.flag), P(b.kL), P(b.vL), P(b.kF), P(b.vF), P(b.hL), P(b.hF),
                            P(b.h_prev), P(ws), wsb, s)
        self._s = s
        self._wsb = wsb

    def set_theta(self, theta: float) -> None:
        self.theta = float(theta)
        a = list(self.score_args)
        a[5] = ctypes.c_float(self.theta)
        self.score_args = tuple(a)

    def _call(self, name, args):
        C.check(getattr(self._lib, name)(*args), name)

    def branch(self, br: int) -> None:
        for a in self.layer_args[br]:
            self._call("oda_dec_layer", a)
        self._call("oda_dec_final_norm", self.norm_args[br])

    def run(self) -> None:
        """One decode step of the batch: local branch, score and rule, the
        full branch where flagged, next token, commit."""
        self._call("oda_dec_embed", self.embed_args)
        self.branch(C.ODA_DEC_LOCAL)
        self._call("oda_recall_score", self.score_args)
        self.branch(C.ODA_DEC_FULL)
        self._call("oda_dec_next_token", self.token_args)
        self._call("oda_commit", self.commit_args)

    def run_always_full(self, flag_all: torch.Tensor) -> None:
        """The always-full baseline's step: every sequence takes the full
        branch; no local branch and no recall head.  `flag_all` is a [B]
        uint8 tensor of ones."""
        b = self.b
        self._call("oda_dec_embed", self.embed_args)
        self._call("oda_worklist", (ctypes.byref(self.dd.attn), flag_all.data_ptr(), b.pos.data_ptr(),
                                    self.ws.data_ptr(), self._wsb, self._s))
        self.branch(C.ODA_DEC_FULL)
        ta = list(self.token_args)
        ta[4] = flag_all.data_ptr()
        self._call("oda_dec_next_token", tuple(ta))
        ca = list(self.commit_args)
        ca[3] = flag_all.data_ptr()
        self._call("oda_commit", tuple(ca))
