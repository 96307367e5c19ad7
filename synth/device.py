"""ctypes binding of the device-side generator (synth/csrc/fill.hip).

Fills KV caches and per-step inputs on the GPU with the same bits as
synth/gen.py, for workloads too large to generate on the host.
"""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

import numpy as np

from . import gen

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libodasynth.so")
_lib = None


def build() -> str:
    hipcc = os.environ.get("HIPCC") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc")
                                        else shutil.which("hipcc"))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(_HERE, "csrc", "fill.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} missing: run `python -c 'import synth.device as d; d.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint64
        L.synth_fill_cache.restype = ctypes.c_int
        L.synth_fill_cache.argtypes = [vp, u64, i32, i32, i32, i32, i32, i32, i64, vp, i64, vp, i32, i32, i64,
                                       i32, ctypes.POINTER(ctypes.c_int32), vp]
        L.synth_fill_step.restype = ctypes.c_int
        L.synth_fill_step.argtypes = [vp] * 7 + [u64, i32, i32, i32, i32, i32, vp, vp, i32, vp]
        L.synth_fill_dec_matrix.restype = ctypes.c_int
        L.synth_fill_dec_matrix.argtypes = [vp, i64, u64, u64, ctypes.c_uint32, vp]
        _lib = L
    return _lib


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def fill_cache(dst, wl: "gen.Workload", tag: int, t0_dev, *, tables=None, num_blocks: int = 0,
               layer0: int = 0, layers: int = None) -> None:
    """Fill K (tag 1) or V (tag 2) of `wl` into the device tensor `dst`."""
    layers = wl.layers if layers is None else layers
    needles = (ctypes.c_int32 * 4)(*(list(wl.needles) + [-1] * (4 - len(wl.needles))))
    paged = tables is not None
    lb = int(np.log2(wl.block_size)) if paged else 0
    rc = lib().synth_fill_cache(dst.data_ptr(), wl.seed, tag, layer0, layers, wl.batch, wl.hkv, wl.head_dim,
                                int(np.max(wl.t0)), t0_dev.data_ptr(), wl.t_cap if not paged else 0,
                                tables.data_ptr() if paged else None, tables.shape[1] if paged else 0, lb,
                                num_blocks, len(wl.needles), needles, _stream())
    if rc != 0:
        raise RuntimeError(f"synth_fill_cache failed: {rc}")


def fill_step(bufs: dict, wl: "gen.Workload", pos_dev, t0_dev) -> None:
    """Per-step inputs of step pos[0] - t0[0] into bufs qL qF kL vL kF vF e."""
    rc = lib().synth_fill_step(*(bufs[k].data_ptr() for k in ("qL", "qF", "kL", "vL", "kF", "vF", "e")),
                               wl.seed, wl.layers, wl.batch, wl.hq, wl.hkv, wl.head_dim, pos_dev.data_ptr(),
                               t0_dev.data_ptr(), len(wl.needles), _stream())
    if rc != 0:
        raise RuntimeError(f"synth_fill_step failed: {rc}")


def fill_dec_matrix(dst, seed: int, tensor_id: int) -> None:
    """Decoder matrix `tensor_id` (gen.dec_matrix_bits) into the contiguous
    device tensor `dst` (int16 storage), element order = flat order."""
    scale_bits = int(np.asarray(gen.DEC_SCALE, dtype=np.float32).view(np.uint32))
    rc = lib().synth_fill_dec_matrix(dst.data_ptr(), dst.numel(), seed, tensor_id, scale_bits, _stream())
    if rc != 0:
        raise RuntimeError(f"synth_fill_dec_matrix failed: {rc}")


def fill_dec_layer(blob, seed: int, shape: "gen.DecoderShape", layer: int, perturb: bool = False) -> None:
    """One layer's blob (gen.dec_layer_blob) on the device: matrices from the
    device generator, norm gains from the host generator."""
    import torch
    at = 0
    for name, sh in gen.dec_layer_tensors(shape):
        n = int(np.prod(sh))
        part = blob[at:at + n]
        if name.startswith("gamma"):
            part.copy_(torch.from_numpy(gen.dec_gain_bits(seed, layer, name, n, perturb).view(np.int16)))
        else:
            fill_dec_matrix(part, seed, gen.dec_tensor_id(layer, name))
        at += n


def fill_dec_embed(table, seed: int) -> None:
    """The token-embedding table [V][D] (gen.dec_embed_bits) on the device."""
    fill_dec_matrix(table, seed, gen.DEC_EMBED_ID)
