"""ctypes binding of liboda (include/oda.h, oda_decoder.h, oda_train.h, oda_hybrid.h).

Argument marshalling only: every function takes torch tensors (or None for a
nullable pointer), passes their device pointers and the current HIP stream
to the C entry point of the same name, and raises OdaError on a non-zero
status.  All work runs in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboda.so")

ODA_OK = 0
ODA_E_NULL, ODA_E_DIMS, ODA_E_UNSUPPORTED, ODA_E_WORKSPACE, ODA_E_LAYER, ODA_E_LAUNCH, ODA_E_ALIGN = \
    -1, -2, -3, -4, -5, -6, -7
ODA_KV_CONTIG, ODA_KV_PAGED = 0, 1
ODA_ERR_CAPACITY, ODA_ERR_BLOCK, ODA_ERR_TOKEN, ODA_ERR_ROW = 1, 2, 4, 8
ODA_DEC_LOCAL, ODA_DEC_FULL = 0, 1
ODA_GDN_LOCAL, ODA_GDN_FULL, ODA_GDN_SLOTS = 0, 1, 3
ODA_DEC_NTENSORS = 9
ODA_HEAD_NTENSORS = 22
ODA_FULL_MIN_CHUNK = 1024
ODA_FULL_FINE_CHUNK = 256
ODA_FULL_FILL_UNITS = 128
ODA_FULL_ROUND_UNITS = 256
ODA_FULL_MAX_SPLITS = 32
ODA_FULL_RAGGED_ROUNDS = 4
ODA_FULL_UNIT_COST_KEYS = 128
ODA_NOALLOC_SCRATCH_BYTES = 16 << 20

EXPORTED = (
    "oda_abi_version", "oda_status_str", "oda_head_param_count", "oda_head_offsets",
    "oda_workspace_bytes", "oda_workspace_worklist_offset", "oda_workspace_init",
    "oda_local_ranges", "oda_local_attn", "oda_recall_score", "oda_worklist", "oda_full_attn_if", "oda_commit",
    "oda_dec_layer_numel", "oda_dec_layer_offsets", "oda_dec_workspace_bytes", "oda_dec_workspace_init",
    "oda_dec_embed", "oda_dec_layer", "oda_dec_final_norm", "oda_dec_next_token",
    "oda_train_workspace_bytes", "oda_train_workspace_init", "oda_train_labels", "oda_train_head_step",
    "oda_gdn_state_bytes", "oda_gdn_conv_offset", "oda_gdn_step", "oda_gdn_commit",
    "oda_local_attn_noalloc",
)


class OdaError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({status_str(status)})")


class oda_dims(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32), ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("hidden", ctypes.c_int32),
        ("sink", ctypes.c_int32), ("window", ctypes.c_int32),
        ("kv_layout", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32), ("reserved0", ctypes.c_int32),
        ("t_cap", ctypes.c_int64), ("num_blocks", ctypes.c_int64),
    ]


class oda_kv(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("block_tables", ctypes.c_void_p)]


class oda_dec_dims(ctypes.Structure):
    _fields_ = [("attn", oda_dims), ("inter", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("eps", ctypes.c_float)]


class oda_train_dims(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int32), ("hidden", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("sink", ctypes.c_int32), ("window", ctypes.c_int32), ("lam", ctypes.c_float)]


class oda_gdn_dims(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("conv_width", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m conditional_sparse_attention_amd.build` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
        dp, kp, ddp = ctypes.POINTER(oda_dims), ctypes.POINTER(oda_kv), ctypes.POINTER(oda_dec_dims)
        tdp = ctypes.POINTER(oda_train_dims)
        gdp = ctypes.POINTER(oda_gdn_dims)
        sig = {
            "oda_abi_version": (ctypes.c_int, []),
            "oda_status_str": (ctypes.c_char_p, [ctypes.c_int]),
            "oda_head_param_count": (i64, [i32]),
            "oda_head_offsets": (ctypes.c_int, [i32, ctypes.POINTER(i64)]),
            "oda_workspace_bytes": (sz, [dp]),
            "oda_workspace_worklist_offset": (sz, [dp]),
            "oda_workspace_init": (ctypes.c_int, [dp, vp, sz, vp]),
            "oda_local_ranges": (ctypes.c_int, [dp, vp, vp, vp]),
            "oda_local_attn": (ctypes.c_int, [dp, i32, kp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "oda_local_attn_noalloc": (ctypes.c_int, [dp, i32, kp, vp, vp, vp, vp, vp, vp, vp, vp]),
            "oda_recall_score": (ctypes.c_int, [dp, vp, vp, vp, vp, f32, vp, vp, vp, vp, vp, sz, vp]),
            "oda_worklist": (ctypes.c_int, [dp, vp, vp, vp, sz, vp]),
            "oda_full_attn_if": (ctypes.c_int, [dp, i32, kp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "oda_commit": (ctypes.c_int, [dp, kp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "oda_dec_layer_numel": (i64, [ddp]),
            "oda_dec_layer_offsets": (ctypes.c_int, [ddp, ctypes.POINTER(i64)]),
            "oda_dec_workspace_bytes": (sz, [ddp]),
            "oda_dec_workspace_init": (ctypes.c_int, [ddp, vp, sz, vp]),
            "oda_dec_embed": (ctypes.c_int, [ddp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "oda_dec_layer": (ctypes.c_int, [ddp, i32, i32, vp, kp, vp, vp, vp, vp, vp, vp, vp, sz, vp, sz, vp]),
            "oda_dec_final_norm": (ctypes.c_int, [ddp, i32, vp, vp, vp, vp, sz, vp]),
            "oda_dec_next_token": (ctypes.c_int, [ddp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "oda_train_workspace_bytes": (sz, [tdp]),
            "oda_train_workspace_init": (ctypes.c_int, [tdp, vp, sz, vp]),
            "oda_train_labels": (ctypes.c_int, [tdp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "oda_train_head_step": (ctypes.c_int, [tdp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                                   vp]),
            "oda_gdn_state_bytes": (sz, [gdp]),
            "oda_gdn_conv_offset": (sz, [gdp]),
            "oda_gdn_step": (ctypes.c_int, [gdp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
            "oda_gdn_commit": (ctypes.c_int, [gdp, vp, vp, vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().oda_status_str(int(status)).decode()


def check(status: int, fn: str) -> None:
    """Raise OdaError for a non-zero status returned by the C function `fn`."""
    if status != ODA_OK:
        raise OdaError(status, fn)


def _p(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("device tensor required")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor required")
    return t.data_ptr()


def _s(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _bytes(ws: torch.Tensor) -> int:
    return ws.numel() * ws.element_size()


# ---------------------------------------------------------------------------
# struct helpers
# ---------------------------------------------------------------------------
def make_dims(num_layers: int, batch: int, num_q_heads: int, num_kv_heads: int, *, head_dim: int = 128,
              sink: int = 4, window: int = 2048, kv_layout: int = ODA_KV_CONTIG, t_cap: int = 0,
              block_size: int = 16, max_blocks_per_seq: int = 0, num_blocks: int = 0) -> oda_dims:
    return oda_dims(num_layers, batch, num_q_heads, num_kv_heads, head_dim, num_q_heads * head_dim, sink, window,
                    kv_layout, block_size if kv_layout == ODA_KV_PAGED else 0,
                    max_blocks_per_seq if kv_layout == ODA_KV_PAGED else 0, 0,
                    t_cap if kv_layout == ODA_KV_CONTIG else 0,
                    num_blocks if kv_layout == ODA_KV_PAGED else 0)


def make_kv(k: torch.Tensor, v: torch.Tensor, block_tables: Optional[torch.Tensor] = None) -> oda_kv:
    return oda_kv(_p(k), _p(v), _p(block_tables))


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def oda_abi_version() -> int:
    return lib().oda_abi_version()


def oda_head_param_count(hidden: int) -> int:
    return int(lib().oda_head_param_count(hidden))


def oda_head_offsets(hidden: int):
    arr = (ctypes.c_int64 * (ODA_HEAD_NTENSORS + 1))()
    check(lib().oda_head_offsets(hidden, arr), "oda_head_offsets")
    return [int(x) for x in arr]


def oda_workspace_bytes(dims: oda_dims) -> int:
    n = int(lib().oda_workspace_bytes(ctypes.byref(dims)))
    if n == 0:
        raise OdaError(ODA_E_DIMS, "oda_workspace_bytes")
    return n


def oda_workspace_worklist_offset(dims: oda_dims) -> int:
    return int(lib().oda_workspace_worklist_offset(ctypes.byref(dims)))


def oda_workspace_init(dims, ws, stream=None) -> None:
    check(lib().oda_workspace_init(ctypes.byref(dims), _p(ws), _bytes(ws), _s(stream)), "oda_workspace_init")


def oda_local_ranges(dims, pos, ranges, stream=None) -> None:
    check(lib().oda_local_ranges(ctypes.byref(dims), _p(pos), _p(ranges), _s(stream)), "oda_local_ranges")


def oda_local_attn(dims, layer, kv: oda_kv, pos, q, k_cur, v_cur, out, lse, ws, stream=None) -> None:
    check(lib().oda_local_attn(ctypes.byref(dims), layer, ctypes.byref(kv), _p(pos), _p(q), _p(k_cur), _p(v_cur),
                                _p(out), _p(lse), _p(ws), _bytes(ws), _s(stream)), "oda_local_attn")


def oda_local_attn_noalloc(dims, layer, kv: oda_kv, pos, q, k_cur, v_cur, out, lse, err, stream=None) -> None:
    check(lib().oda_local_attn_noalloc(ctypes.byref(dims), layer, ctypes.byref(kv), _p(pos), _p(q), _p(k_cur),
                                       _p(v_cur), _p(out), _p(lse), _p(err), _s(stream)), "oda_local_attn_noalloc")


def oda_recall_score(dims, head_w, h_prev, emb, h_local, theta, force, pos, score, flag, ws, stream=None) -> None:
    check(lib().oda_recall_score(ctypes.byref(dims), _p(head_w), _p(h_prev), _p(emb), _p(h_local),
                                  ctypes.c_float(theta), _p(force), _p(pos), _p(score), _p(flag), _p(ws),
                                  _bytes(ws), _s(stream)), "oda_recall_score")


def oda_worklist(dims, flag, pos, ws, stream=None) -> None:
    check(lib().oda_worklist(ctypes.byref(dims), _p(flag), _p(pos), _p(ws), _bytes(ws), _s(stream)), "oda_worklist")


def oda_full_attn_if(dims, layer, kv: oda_kv, pos, q, k_cur, v_cur, out, lse, ws, stream=None) -> None:
    check(lib().oda_full_attn_if(ctypes.byref(dims), layer, ctypes.byref(kv), _p(pos), _p(q), _p(k_cur),
                                  _p(v_cur), _p(out), _p(lse), _p(ws), _bytes(ws), _s(stream)), "oda_full_attn_if")


def oda_commit(dims, kv: oda_kv, pos, flag, k_cur_L, v_cur_L, k_cur_F, v_cur_F, out_last_L, out_last_F, h_prev, ws,
               stream=None) -> None:
    check(lib().oda_commit(ctypes.byref(dims), ctypes.byref(kv), _p(pos), _p(flag), _p(k_cur_L), _p(v_cur_L),
                            _p(k_cur_F), _p(v_cur_F), _p(out_last_L), _p(out_last_F), _p(h_prev), _p(ws),
                            _bytes(ws), _s(stream)), "oda_commit")


# ---------------------------------------------------------------------------
# decoder backbone around the path (include/oda_decoder.h)
# ---------------------------------------------------------------------------
def make_dec_dims(attn: oda_dims, inter: int, vocab: int, rope_theta: float = 1.0e6,
                  eps: float = 1e-6) -> oda_dec_dims:
    return oda_dec_dims(attn, inter, vocab, rope_theta, eps)


def oda_dec_layer_numel(dd: oda_dec_dims) -> int:
    n = int(lib().oda_dec_layer_numel(ctypes.byref(dd)))
    if n < 0:
        raise OdaError(ODA_E_DIMS, "oda_dec_layer_numel")
    return n


def oda_dec_layer_offsets(dd: oda_dec_dims):
    arr = (ctypes.c_int64 * (ODA_DEC_NTENSORS + 1))()
    check(lib().oda_dec_layer_offsets(ctypes.byref(dd), arr), "oda_dec_layer_offsets")
    return list(arr)


def oda_dec_workspace_bytes(dd: oda_dec_dims) -> int:
    n = int(lib().oda_dec_workspace_bytes(ctypes.byref(dd)))
    if n == 0:
        raise OdaError(ODA_E_DIMS, "oda_dec_workspace_bytes")
    return n


def oda_dec_workspace_init(dd, dws, stream=None) -> None:
    check(lib().oda_dec_workspace_init(ctypes.byref(dd), _p(dws), _bytes(dws), _s(stream)), "oda_dec_workspace_init")


def oda_dec_embed(dd, embed, tokens, x_local, x_full, emb, ws=None, stream=None) -> None:
    check(lib().oda_dec_embed(ctypes.byref(dd), _p(embed), _p(tokens), _p(x_local), _p(x_full), _p(emb), _p(ws),
                              _bytes(ws) if ws is not None else 0, _s(stream)), "oda_dec_embed")


def oda_dec_layer(dd, layer, branch, w_layer, kv: oda_kv, pos, x, q, k_cur, v_cur, o, ws, dws, stream=None) -> None:
    check(lib().oda_dec_layer(ctypes.byref(dd), layer, branch, _p(w_layer), ctypes.byref(kv), _p(pos), _p(x), _p(q),
                              _p(k_cur), _p(v_cur), _p(o), _p(ws), _bytes(ws), _p(dws), _bytes(dws), _s(stream)),
          "oda_dec_layer")


def oda_dec_final_norm(dd, branch, gamma_f, x, h, ws=None, stream=None) -> None:
    check(lib().oda_dec_final_norm(ctypes.byref(dd), branch, _p(gamma_f), _p(x), _p(h), _p(ws),
                                   _bytes(ws) if ws is not None else 0, _s(stream)), "oda_dec_final_norm")


def oda_dec_next_token(dd, embed, h_local, h_full, flag, tokens, max_logit, dws, stream=None) -> None:
    check(lib().oda_dec_next_token(ctypes.byref(dd), _p(embed), _p(h_local), _p(h_full), _p(flag), _p(tokens),
                                   _p(max_logit), _p(dws), _bytes(dws), _s(stream)), "oda_dec_next_token")


# --------------------------------------------------------------------------
# recall-head training step (include/oda_train.h)
# --------------------------------------------------------------------------
def make_train_dims(rows: int, hidden: int, vocab: int, lam: float = 0.0, sink: int = 4,
                    window: int = 2048) -> oda_train_dims:
    return oda_train_dims(rows=rows, hidden=hidden, vocab=vocab, sink=sink, window=window, lam=lam)


def oda_train_workspace_bytes(td: oda_train_dims) -> int:
    n = int(lib().oda_train_workspace_bytes(ctypes.byref(td)))
    if n == 0:
        raise OdaError(ODA_E_DIMS, "oda_train_workspace_bytes")
    return n


def oda_train_workspace_init(td, ws, stream=None) -> None:
    check(lib().oda_train_workspace_init(ctypes.byref(td), _p(ws), _bytes(ws), _s(stream)),
          "oda_train_workspace_init")


def oda_train_labels(td, lm_head, h_local, h_full, next_tok, pos, gain, label, valid, ws, stream=None) -> None:
    check(lib().oda_train_labels(ctypes.byref(td), _p(lm_head), _p(h_local), _p(h_full), _p(next_tok), _p(pos),
                                 _p(gain), _p(label), _p(valid), _p(ws), _bytes(ws), _s(stream)), "oda_train_labels")


def oda_train_head_step(td, head_w, lm_head, h_local, h_full, tokens, prev, gain, label, valid, score, loss, grad,
                        ws, stream=None) -> None:
    check(lib().oda_train_head_step(ctypes.byref(td), _p(head_w), _p(lm_head), _p(h_local), _p(h_full), _p(tokens),
                                    _p(prev), _p(gain), _p(label), _p(valid), _p(score), _p(loss), _p(grad), _p(ws),
                                    _bytes(ws), _s(stream)), "oda_train_head_step")


# --------------------------------------------------------------------------
# recurrent layers of a hybrid backbone (include/oda_hybrid.h)
# --------------------------------------------------------------------------
def make_gdn_dims(num_layers: int, batch: int, heads: int, head_dim: int = 128, conv_width: int = 4) -> oda_gdn_dims:
    return oda_gdn_dims(num_layers=num_layers, batch=batch, heads=heads, head_dim=head_dim, conv_width=conv_width)


def oda_gdn_state_bytes(gd: oda_gdn_dims) -> int:
    n = int(lib().oda_gdn_state_bytes(ctypes.byref(gd)))
    if n == 0:
        raise OdaError(ODA_E_DIMS, "oda_gdn_state_bytes")
    return n


def oda_gdn_conv_offset(gd: oda_gdn_dims) -> int:
    return int(lib().oda_gdn_conv_offset(ctypes.byref(gd)))


def oda_gdn_step(gd, layer, branch, state, slot, flag, x, conv_w, alpha, beta, out, stream=None) -> None:
    check(lib().oda_gdn_step(ctypes.byref(gd), layer, branch, _p(state), _p(slot), _p(flag), _p(x), _p(conv_w),
                             _p(alpha), _p(beta), _p(out), _s(stream)), "oda_gdn_step")


def oda_gdn_commit(gd, slot, flag, stream=None) -> None:
    check(lib().oda_gdn_commit(ctypes.byref(gd), _p(slot), _p(flag), _s(stream)), "oda_gdn_commit")
