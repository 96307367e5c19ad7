"""Seeded synthetic inputs for the On-Demand Attention decode step.

This module is the one source of inputs shared by the CPU oracle and the HIP
path.  It holds none of the method's arithmetic: it only turns
(seed, tag, logical index) into bf16 / float values, and describes the shapes
of the synthetic workloads (lengths, needle positions, head-weight init,
forced flags, paged block tables).

Generator G
-----------
* ``splitmix64`` is Vigna's public-domain mixer (the SplitMix64 output
  function): add the golden gamma 0x9E3779B97F4A7C15, then two xor-shift /
  multiply rounds (constants 0xBF58476D1CE4E5B9, 0x94D049BB133111EB) and a
  final xor-shift.
* Stream key: ``key = splitmix64(seed * 256 + tag)``.
* One 64-bit hash feeds two values: ``h = splitmix64(key + (idx >> 1))`` and
  value ``idx`` takes the 32-bit half ``(h >> (32 * (idx & 1))) & 0xFFFFFFFF``.
* bf16 value of a 32-bit word w: ``x = sum of its four bytes - 510`` (an
  integer in [-510, 510]; mean 0, variance 4 * (256**2 - 1) / 12 = 21845),
  ``v = float32(x) * VALUE_SCALE`` with ``VALUE_SCALE = float32(1/sqrt(21845))``
  (one IEEE multiply, no fused op), then round-to-nearest-even to bf16.
  The result has unit variance and support of about +-3.45.
* Uniform doubles (head weights, lengths, Bernoulli draws) use the whole hash:
  ``u = (splitmix64(key + idx) >> 11) * 2**-53``.

The device-side fill kernels in ``synth/csrc/fill.hip`` implement the same
definition and are checked against this file bit for bit.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Tuple

import numpy as np

_U64 = np.uint64
GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

VALUE_SCALE = np.float32(1.0 / math.sqrt(21845.0))  # bit pattern 0x3BDDB446
assert VALUE_SCALE.view(np.uint32) == np.uint32(1004385350)

# Stream tags.
TAG_K, TAG_V = 1, 2            # KV cache contents
TAG_QL, TAG_QF = 3, 4          # per-step attention queries, local / full branch
TAG_KL, TAG_VL = 5, 6          # per-step staged current k, v (local branch)
TAG_KF, TAG_VF = 7, 8          # per-step staged current k, v (full branch)
TAG_E, TAG_H0 = 9, 10          # current-token embedding, initial previous hidden state
TAG_NEEDLE = 11                # needle sign patterns
TAG_HEAD = 12                  # recall-head weights
TAG_LEN = 13                   # ragged context lengths
TAG_BERN = 14                  # Bernoulli forced flags
TAG_SHUF = 15                  # paged block shuffle
TAG_DEC_W = 16                 # decoder weight matrices and the token-embedding table
TAG_DEC_G = 17                 # decoder norm gains (perturbed variants)
TAG_TOK = 18                   # first tokens of the decoder workloads
TAG_TRAIN_HL = 19              # training rows: local-branch final hidden states
TAG_TRAIN_HF = 20              # training rows: full-branch final hidden states (rows that differ)
TAG_TRAIN_TOK = 21             # training rows: token streams
TAG_TRAIN_SEL = 22             # training rows: which rows' full state differs
TAG_GDN_XL, TAG_GDN_XF = 23, 24  # recurrent layers: per-step q|k|v projection, local / full branch
TAG_GDN_GATE = 25              # recurrent layers: per-step alpha, beta
TAG_GDN_W = 26                 # recurrent layers: convolution weights
TAG_GDN_S0 = 27                # recurrent layers: initial recurrent state
TAG_GDN_C0 = 28                # recurrent layers: initial convolution state

MAX_B = 32          # logical batch stride of the index space
POS_BITS = 18       # logical position stride 2**18
NEEDLE_SCALE_BITS = np.uint16(0x3FC0)  # bf16 of +1.5
NEEDLE_NEG_BITS = np.uint16(0xBFC0)    # bf16 of -1.5


# --------------------------------------------------------------------------
# generator core
# --------------------------------------------------------------------------
def splitmix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output function on a uint64 array (wrapping arithmetic)."""
    z = np.asarray(z, dtype=_U64)
    with np.errstate(over="ignore"):
        z = z + _U64(GAMMA)
        z = (z ^ (z >> _U64(30))) * _U64(MIX1)
        z = (z ^ (z >> _U64(27))) * _U64(MIX2)
    return z ^ (z >> _U64(31))


def splitmix64_int(z: int) -> int:
    z = (z + GAMMA) & MASK64
    z = ((z ^ (z >> 30)) * MIX1) & MASK64
    z = ((z ^ (z >> 27)) * MIX2) & MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, tag: int) -> int:
    return splitmix64_int((seed * 256 + tag) & MASK64)


def hash_at(seed: int, tag: int, idx) -> np.ndarray:
    key = _U64(stream_key(seed, tag))
    idx = np.asarray(idx, dtype=_U64)
    with np.errstate(over="ignore"):
        return splitmix64(key + idx)


def word32_at(seed: int, tag: int, idx) -> np.ndarray:
    idx = np.asarray(idx, dtype=_U64)
    h = hash_at(seed, tag, idx >> _U64(1))
    shift = (idx & _U64(1)) * _U64(32)
    return ((h >> shift) & _U64(0xFFFFFFFF)).astype(np.uint32)


def f32_to_bf16_rne(v: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 bits, nearest-even."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = _U64(0x7FFF) + ((u >> _U64(16)) & _U64(1))
    return ((u + bias) >> _U64(16)).astype(np.uint16)


def bf16_at(seed: int, tag: int, idx) -> np.ndarray:
    """bf16 bits of G(seed, tag, idx) for an array of logical indices."""
    w = word32_at(seed, tag, idx)
    x = ((w & 0xFF) + ((w >> 8) & 0xFF) + ((w >> 16) & 0xFF) + (w >> 24)).astype(np.int32) - 510
    v = x.astype(np.float32) * VALUE_SCALE
    return f32_to_bf16_rne(v)


def uniform_at(seed: int, tag: int, idx) -> np.ndarray:
    h = hash_at(seed, tag, idx)
    return (h >> _U64(11)).astype(np.float64) * (2.0 ** -53)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    """Shape and structure of one synthetic decode workload.

    ``t0[b]`` is the committed length of sequence b before the first routed
    step; step j (0-based) decodes the token at 0-based position t0[b] + j.
    """
    name: str
    layers: int
    hq: int
    hkv: int
    head_dim: int
    batch: int
    t0: np.ndarray
    steps: int
    seed: int
    head_seed: int
    layout: str = "contig"           # "contig" | "paged"
    block_size: int = 16
    needles: Tuple[int, ...] = ()
    sink: int = 4
    window: int = 2048
    rate: Optional[float] = None     # target full-branch rate when theta is tuned
    theta: float = 0.0               # threshold when not tuned
    bernoulli_odd: Optional[float] = None  # odd sequences forced by Bernoulli(p)
    t_cap_slack: int = 256

    @property
    def hidden(self) -> int:
        return self.hq * self.head_dim

    @property
    def t_cap(self) -> int:
        """Per-sequence capacity for the contiguous layout."""
        return int(np.max(self.t0)) + self.steps + self.t_cap_slack

    def kv_bytes(self) -> int:
        tok = int(np.sum(self.t0 + self.steps + self.t_cap_slack))
        return self.layers * tok * self.hkv * self.head_dim * 2 * 2

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def log_uniform_lengths(seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    u = uniform_at(seed, TAG_LEN, np.arange(batch))
    return np.rint(np.exp(np.log(lo) + u * (np.log(hi) - np.log(lo)))).astype(np.int64)


def workloads() -> dict:
    """The five synthetic workloads, keyed by number (plus "5-4k")."""
    w = {}
    w[1] = Workload("tiny-1layer-4k", 1, 16, 8, 128, 1, np.full(1, 4096), 64, seed=1,
                    head_seed=101, needles=(100, 500, 900), theta=0.0)
    w[2] = Workload("qwen3-1.7b-16k-b8", 28, 16, 8, 128, 8, np.full(8, 16384), 256, seed=2,
                    head_seed=102, rate=0.416)
    w[3] = Workload("qwen3-1.7b-128k-b4", 28, 16, 8, 128, 4, np.full(4, 131072), 128, seed=3,
                    head_seed=103, needles=(32768, 65536, 98304), rate=0.125)
    w[4] = Workload("qwen3-8b-64k-b16", 36, 32, 8, 128, 16, np.full(16, 65536), 128, seed=4,
                    head_seed=104, rate=0.47)
    w[5] = Workload("ragged-paged-b32", 28, 16, 8, 128, 32,
                    log_uniform_lengths(5, 32, 4096, 131072), 64, seed=5, head_seed=105,
                    layout="paged", theta=0.0, bernoulli_odd=0.3, t_cap_slack=16)
    w["5-4k"] = Workload("paged-4k-b32", 28, 16, 8, 128, 32, np.full(32, 4096), 64, seed=6,
                         head_seed=106, layout="paged", theta=0.0, t_cap_slack=16)
    # the attention layers of a hybrid backbone: 6 full-attention layers
    # between 18 recurrent ones (GdnShape), at the pages' hybrid call rate
    w["hybrid"] = Workload("hybrid-6attn-18gdn-32k-b8", 6, 16, 8, 128, 8, np.full(8, 32768), 64, seed=7,
                           head_seed=107, rate=0.443)
    return w


# --------------------------------------------------------------------------
# logical indices
# --------------------------------------------------------------------------
def cache_index(l, b, g, p, i, hkv: int, d: int):
    l, b, g, p, i = (np.asarray(a, dtype=np.uint64) for a in (l, b, g, p, i))
    return ((((l * _U64(MAX_B) + b) * _U64(hkv) + g) << _U64(POS_BITS)) + p) * _U64(d) + i


def step_index(j, l, b, h, i, layers: int, heads: int, d: int):
    j, l, b, h, i = (np.asarray(a, dtype=np.uint64) for a in (j, l, b, h, i))
    return ((((j * _U64(layers) + l) * _U64(MAX_B) + b) * _U64(heads) + h) * _U64(d)) + i


def emb_index(j, b, i, hidden: int):
    j, b, i = (np.asarray(a, dtype=np.uint64) for a in (j, b, i))
    return (j * _U64(MAX_B) + b) * _U64(hidden) + i


# --------------------------------------------------------------------------
# tensors
# --------------------------------------------------------------------------
def needle_signs(seed: int, n: int, d: int) -> np.ndarray:
    """+-1 pattern of needle n (bit 0 of tag-11 words)."""
    w = word32_at(seed, TAG_NEEDLE, np.arange(n * d, (n + 1) * d))
    return np.where((w & 1) == 1, 1, -1).astype(np.int8)


def needle_bits(seed: int, n: int, d: int) -> np.ndarray:
    return np.where(needle_signs(seed, n, d) > 0, NEEDLE_SCALE_BITS, NEEDLE_NEG_BITS).astype(np.uint16)


def cache_rows(wl: Workload, tag: int, l: int, b: int, g: int, p0: int, p1: int) -> np.ndarray:
    """bf16 bits [p1-p0][d] of the initial cache (K if tag==TAG_K else V)
    for logical positions [p0, p1).  Needle rows override K."""
    d = wl.head_dim
    p = np.arange(p0, p1, dtype=np.uint64)[:, None]
    i = np.arange(d, dtype=np.uint64)[None, :]
    out = bf16_at(wl.seed, tag, cache_index(l, b, g, p, i, wl.hkv, d))
    if tag == TAG_K:
        for n, pn in enumerate(wl.needles):
            if p0 <= pn < p1:
                out[pn - p0] = needle_bits(wl.seed, n, d)
    return out


def aligned_needle(wl: Workload, j: int) -> Optional[int]:
    """Needle targeted by every query at step j, or None."""
    if wl.needles and j % 8 == 0:
        return (j // 8) % len(wl.needles)
    return None


_STEP_TAGS = {"qL": TAG_QL, "qF": TAG_QF, "kL": TAG_KL, "vL": TAG_VL, "kF": TAG_KF, "vF": TAG_VF}
_LAYER0_ALIAS = {"qF": "qL", "kF": "kL", "vF": "vL"}


def step_tensor(wl: Workload, which: str, j: int, l: int) -> np.ndarray:
    """bf16 bits [B][H][d] of a per-step input for layer l.

    which: qL / qF (H = hq) or kL / vL / kF / vF (H = hkv).  Layer 0 takes the
    same values for both branches (same pre-step state and token embedding);
    at aligned steps every query equals 1.5 * the targeted needle pattern."""
    if l == 0 and which in _LAYER0_ALIAS:
        which = _LAYER0_ALIAS[which]
    heads = wl.hq if which.startswith("q") else wl.hkv
    d = wl.head_dim
    b = np.arange(wl.batch, dtype=np.uint64)[:, None, None]
    h = np.arange(heads, dtype=np.uint64)[None, :, None]
    i = np.arange(d, dtype=np.uint64)[None, None, :]
    out = bf16_at(wl.seed, _STEP_TAGS[which], step_index(j, l, b, h, i, wl.layers, heads, d))
    n = aligned_needle(wl, j)
    if which.startswith("q") and n is not None:
        out[:] = needle_bits(wl.seed, n, d)[None, None, :]
    return out


def step_tensor_all_layers(wl: Workload, which: str, j: int) -> np.ndarray:
    return np.stack([step_tensor(wl, which, j, l) for l in range(wl.layers)])


def embedding(wl: Workload, j: int) -> np.ndarray:
    D = wl.hidden
    b = np.arange(wl.batch, dtype=np.uint64)[:, None]
    i = np.arange(D, dtype=np.uint64)[None, :]
    return bf16_at(wl.seed, TAG_E, emb_index(j, b, i, D))


def h_prev0(wl: Workload) -> np.ndarray:
    D = wl.hidden
    b = np.arange(wl.batch, dtype=np.uint64)[:, None]
    i = np.arange(D, dtype=np.uint64)[None, :]
    return bf16_at(wl.seed, TAG_H0, b * _U64(D) + i)


def bernoulli_force(wl: Workload, j: int) -> np.ndarray:
    """int8 force vector for step j: -1 = decided by the head, 0/1 = forced."""
    force = np.full(wl.batch, -1, dtype=np.int8)
    if wl.bernoulli_odd is not None:
        odd = np.arange(1, wl.batch, 2)
        u = uniform_at(wl.seed, TAG_BERN, j * MAX_B + odd)
        force[odd] = (u < wl.bernoulli_odd).astype(np.int8)
    return force


def forced_rate_flags(seed: int, steps: int, batch: int, rate: float) -> np.ndarray:
    """[steps][B] int8 forced flags with an exact count round(rate*steps*batch),
    placed by the order of tag-14 uniforms (used for controlled-rate sweeps)."""
    n = steps * batch
    k = int(round(rate * n))
    u = uniform_at(seed, TAG_BERN, np.arange(n) + 7919)
    order = np.argsort(u, kind="stable")
    flags = np.zeros(n, dtype=np.int8)
    flags[order[:k]] = 1
    return flags.reshape(steps, batch)


# --------------------------------------------------------------------------
# paged layout
# --------------------------------------------------------------------------
def paged_block_tables(wl: Workload) -> Tuple[np.ndarray, int]:
    """Per-sequence block tables [B][MB] int32 over a shuffled physical pool.

    Each sequence owns ceil((t0 + steps + slack) / block) blocks; the physical
    ids are a seeded permutation of the pool, so logical neighbours are
    scattered.  Unused table entries hold -1."""
    bs = wl.block_size
    need = [(int(t) + wl.steps + wl.t_cap_slack + bs - 1) // bs for t in wl.t0]
    nb = int(sum(need))
    mb = int(max(need))
    perm = np.argsort(hash_at(wl.seed, TAG_SHUF, np.arange(nb)), kind="stable").astype(np.int32)
    tables = np.full((wl.batch, mb), -1, dtype=np.int32)
    at = 0
    for b, n in enumerate(need):
        tables[b, :n] = perm[at:at + n]
        at += n
    return tables, nb


# --------------------------------------------------------------------------
# recall-head weights (fp32 blob)
# --------------------------------------------------------------------------
def head_tensor_shapes(hidden: int, tower: int = 1024, ffn: int = 2048) -> Sequence[Tuple[str, tuple, str]]:
    """(name, shape, init) of each packed tensor, in blob order.

    init: "xavier" (uniform +-sqrt(6/(fan_in+fan_out))), "zero" (bias) or
    "one" (norm gain)."""
    t, f, D = tower, ffn, hidden
    out = []
    for s in ("H", "E", "L"):
        out += [(f"gamma_{s}", (D,), "one"), (f"W_{s}", (t, D), "xavier"), (f"c_{s}", (t,), "zero")]
    out += [("W_I", (t, 9 * t), "xavier"), ("c_I", (t,), "zero")]
    for k in (1, 2):
        out += [(f"gamma_{k}", (t,), "one"), (f"Wg_{k}", (f, t), "xavier"),
                (f"Wu_{k}", (f, t), "xavier"), (f"Wd_{k}", (t, f), "xavier")]
    out += [("gamma_o", (t,), "one"), ("w_o", (1, t), "xavier"), ("c_o", (1,), "zero")]
    return out


def head_blob(hidden: int, seed: int, perturb: bool = False, tower: int = 1024,
              ffn: int = 2048) -> np.ndarray:
    """Packed fp32 recall-head parameters, Xavier-uniform init (gain 1).

    With ``perturb`` the biases are drawn U(-0.1, 0.1) and the norm gains
    1 + U(-0.1, 0.1) instead of 0 / 1, so parity runs exercise every term."""
    shapes = head_tensor_shapes(hidden, tower, ffn)
    total = sum(int(np.prod(s)) for _, s, _ in shapes)
    u = uniform_at(seed, TAG_HEAD, np.arange(total))
    blob = np.empty(total, dtype=np.float32)
    at = 0
    for name, shape, init in shapes:
        n = int(np.prod(shape))
        uu = u[at:at + n]
        if init == "xavier":
            fan_out, fan_in = shape
            bound = math.sqrt(6.0 / (fan_in + fan_out))
            blob[at:at + n] = ((2.0 * uu - 1.0) * bound).astype(np.float32)
        elif init == "zero":
            blob[at:at + n] = ((2.0 * uu - 1.0) * 0.1).astype(np.float32) if perturb else 0.0
        else:
            blob[at:at + n] = (1.0 + (2.0 * uu - 1.0) * 0.1).astype(np.float32) if perturb else 1.0
        at += n
    return blob


# --------------------------------------------------------------------------
# decoder backbone around the path (random-init, Qwen3-1.7B-shaped)
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class DecoderShape:
    """Shape of a dense decoder whose attention is the ODA path: pre-RMSNorm
    attention with QK-norm and RoPE, then a pre-RMSNorm SwiGLU MLP, a final
    RMSNorm and an LM head tied to the token embedding."""
    name: str
    hidden: int
    layers: int
    hq: int
    hkv: int
    head_dim: int
    inter: int
    vocab: int
    rope_theta: float = 1.0e6
    eps: float = 1e-6


def decoder_shapes() -> dict:
    return {
        "qwen3-1.7b": DecoderShape("qwen3-1.7b", 2048, 28, 16, 8, 128, 6144, 151936),
        "tiny": DecoderShape("tiny", 1024, 2, 8, 4, 128, 2048, 4096),
        # the same with one and with four query heads per KV head
        "tiny-g1": DecoderShape("tiny-g1", 1024, 2, 8, 8, 128, 2048, 4096),
        "tiny-g4": DecoderShape("tiny-g4", 1024, 2, 8, 2, 128, 2048, 4096),
        # an MLP width that is not a multiple of 2048: 3 K slices in the down projection
        "tiny-i3k": DecoderShape("tiny-i3k", 1024, 2, 8, 4, 128, 3072, 4096),
    }


# Matrices are uniform on (-a, a) with a = 0.02 * sqrt(3) (standard deviation
# 0.02), drawn on a 2^22-level grid so that host and device compute the same
# bits with one float32 multiply: value = bf16(((m - 2^21) + 0.5) * s), m the
# top 22 bits of the 64-bit hash of the logical index, s = float32(a / 2^21).
DEC_INIT_STD = 0.02
DEC_SCALE = np.float32(DEC_INIT_STD * math.sqrt(3.0) / 2.0 ** 21)
DEC_TENSOR_BITS = 40            # logical index = (tensor id << 40) + element
DEC_EMBED_ID = 1 << 20          # tensor id of the token-embedding table
DEC_MATRICES = ("W_qkv", "W_o", "W_gate", "W_up", "W_down")


def dec_tensor_id(layer: int, name: str) -> int:
    return layer * 8 + DEC_MATRICES.index(name)


def dec_matrix_bits(seed: int, tensor_id: int, elems) -> np.ndarray:
    """bf16 bits of elements `elems` of decoder matrix `tensor_id`."""
    idx = (np.uint64(tensor_id) << np.uint64(DEC_TENSOR_BITS)) + np.asarray(elems, dtype=_U64)
    h = hash_at(seed, TAG_DEC_W, idx)
    m = (h >> _U64(42)).astype(np.int64) - (1 << 21)
    x = m.astype(np.float32) + np.float32(0.5)
    return f32_to_bf16_rne(x * DEC_SCALE)


def dec_layer_tensors(shape: DecoderShape) -> Sequence[Tuple[str, tuple]]:
    """(name, shape) of one layer's tensors in blob order (bf16 each)."""
    D, d, I = shape.hidden, shape.head_dim, shape.inter
    nqkv = (shape.hq + 2 * shape.hkv) * d
    return [("gamma_in", (D,)), ("W_qkv", (nqkv, D)), ("gamma_q", (d,)), ("gamma_k", (d,)),
            ("W_o", (D, shape.hq * d)), ("gamma_post", (D,)), ("W_gate", (I, D)), ("W_up", (I, D)),
            ("W_down", (D, I))]


def dec_gain_bits(seed: int, layer: int, name: str, n: int, perturb: bool) -> np.ndarray:
    """Norm gains: 1, or 1 + U(-0.1, 0.1) when perturbed (host only)."""
    if not perturb:
        return np.full(n, 0x3F80, dtype=np.uint16)
    tid = {"gamma_in": 0, "gamma_q": 1, "gamma_k": 2, "gamma_post": 3, "gamma_final": 4}[name]
    u = uniform_at(seed, TAG_DEC_G, (np.uint64(layer * 8 + tid) << np.uint64(DEC_TENSOR_BITS)) +
                   np.arange(n, dtype=_U64))
    return f32_to_bf16_rne((1.0 + (2.0 * u - 1.0) * 0.1).astype(np.float32))


def dec_layer_blob(seed: int, shape: DecoderShape, layer: int, perturb: bool = False) -> np.ndarray:
    """One layer's bf16 blob (host; small shapes)."""
    parts = []
    for name, sh in dec_layer_tensors(shape):
        n = int(np.prod(sh))
        if name.startswith("gamma"):
            parts.append(dec_gain_bits(seed, layer, name, n, perturb))
        else:
            parts.append(dec_matrix_bits(seed, dec_tensor_id(layer, name), np.arange(n)))
    return np.concatenate(parts)


def dec_embed_bits(seed: int, shape: DecoderShape, rows) -> np.ndarray:
    """Rows of the token-embedding table [V][D] (also the tied LM head)."""
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    D = shape.hidden
    el = (rows[:, None] * D + np.arange(D)[None, :]).astype(_U64)
    return dec_matrix_bits(seed, DEC_EMBED_ID, el).reshape(len(rows), D)


def dec_first_tokens(seed: int, batch: int, vocab: int) -> np.ndarray:
    return (hash_at(seed, TAG_TOK, np.arange(batch)) % _U64(vocab)).astype(np.int32)


# --------------------------------------------------------------------------
# recall-head training micro-batches (paired branch outputs)
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class TrainShape:
    """A training micro-batch: `runs` stretches of `rows_per_run` consecutive
    positions, the first at 0-based position `first_pos`.  Every row carries
    the local and the full branch's final hidden state at its position; the
    two are identical where the index sets coincide (pos < s + w) and, past
    that, differ on a `differ_rate` share of the rows (independent draws) and
    coincide on the rest."""
    name: str
    hidden: int
    vocab: int
    runs: int
    rows_per_run: int
    first_pos: int
    differ_rate: float
    seed: int
    head_seed: int
    embed_seed: int
    lam: float = 0.0

    @property
    def rows(self) -> int:
        return self.runs * self.rows_per_run


def train_shapes() -> dict:
    return {
        # 4 sequences x 2048 positions starting at t = 2052 (the last position
        # whose index sets coincide), with the Qwen3-1.7B hidden size and
        # vocabulary
        "qwen3-1.7b-8k": TrainShape("qwen3-1.7b-8k", 2048, 151936, 4, 2048, 2051, 0.25, seed=41,
                                    head_seed=141, embed_seed=241),
        "small": TrainShape("small", 2048, 151936, 2, 20, 2040, 0.5, seed=42, head_seed=142, embed_seed=242,
                            lam=0.001),
    }


def train_rows(sh: TrainShape):
    """pos, prev, tokens (x_t) and next tokens (x_{t+1}) of every row [N] int32.
    prev is the row of the previous position, -1 at the first row of a run
    whose position is 0 ... and also at the first row of a later stretch (its
    predecessor is not in the micro-batch)."""
    n = np.arange(sh.rows)
    run, j = n // sh.rows_per_run, n % sh.rows_per_run
    pos = (sh.first_pos + j).astype(np.int32)
    prev = np.where(j > 0, n - 1, -1).astype(np.int32)
    stream = (run.astype(_U64) << _U64(32))
    tok = (hash_at(sh.seed, TAG_TRAIN_TOK, stream + pos.astype(_U64)) % _U64(sh.vocab)).astype(np.int32)
    nxt = (hash_at(sh.seed, TAG_TRAIN_TOK, stream + pos.astype(_U64) + _U64(1)) % _U64(sh.vocab)).astype(np.int32)
    return pos, prev, tok, nxt


def train_differs(sh: TrainShape, pos: np.ndarray, sink: int = 4, window: int = 2048) -> np.ndarray:
    """Rows whose full-branch state is drawn independently of the local one."""
    u = uniform_at(sh.seed, TAG_TRAIN_SEL, np.arange(sh.rows))
    return (u < sh.differ_rate) & (np.asarray(pos) >= sink + window)


def train_hidden(sh: TrainShape, rows=None):
    """bf16 bits of h^L and h^F for `rows` (default: all) [len][D]."""
    rows = np.arange(sh.rows) if rows is None else np.asarray(rows, dtype=np.int64)
    pos, _, _, _ = train_rows(sh)
    D = sh.hidden
    idx = (rows[:, None] * D + np.arange(D)[None, :]).astype(_U64)
    hl = bf16_at(sh.seed, TAG_TRAIN_HL, idx)
    hf = hl.copy()
    dif = train_differs(sh, pos)[rows]
    if np.any(dif):
        hf[dif] = bf16_at(sh.seed, TAG_TRAIN_HF, idx[dif])
    return hl, hf


# --------------------------------------------------------------------------
# recurrent layers of a hybrid backbone (gated delta rule decode layers)
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class GdnShape:
    """Recurrent layers of a hybrid backbone: `layers` layers of `heads`
    heads (d_k = d_v = d), causal convolution of width `conv_width` over the
    3 H d channels of q | k | v.  `shared_layers` recurrent layers come
    before the first attention layer: both branches see the same inputs
    there."""
    layers: int
    batch: int
    heads: int
    d: int = 128
    conv_width: int = 4
    shared_layers: int = 3
    seed: int = 61

    @property
    def channels(self) -> int:
        return 3 * self.heads * self.d


GDN_MAX_B = 1024


def gdn_x(sh: GdnShape, layer: int, branch: int, step: int) -> np.ndarray:
    """bf16 bits of the q|k|v projection [B][C] of one layer, branch, step."""
    tag = TAG_GDN_XL if (branch == 0 or layer < sh.shared_layers) else TAG_GDN_XF
    C = sh.channels
    base = ((np.uint64(step) * np.uint64(sh.layers) + np.uint64(layer)) * np.uint64(GDN_MAX_B))
    idx = ((base + np.arange(sh.batch, dtype=_U64))[:, None] * _U64(C) + np.arange(C, dtype=_U64)[None, :])
    return bf16_at(sh.seed, tag, idx)


def gdn_gates(sh: GdnShape, layer: int, branch: int, step: int):
    """float32 alpha in [0.9, 1) and beta in [0.05, 0.95) [B][H]."""
    br = 0 if layer < sh.shared_layers else branch
    base = (((np.uint64(step) * np.uint64(sh.layers) + np.uint64(layer)) * _U64(2) + _U64(br)) * _U64(GDN_MAX_B))
    idx = (base + np.arange(sh.batch, dtype=_U64))[:, None] * _U64(2 * sh.heads) + np.arange(2 * sh.heads,
                                                                                              dtype=_U64)[None, :]
    u = uniform_at(sh.seed, TAG_GDN_GATE, idx)
    alpha = (0.9 + 0.1 * u[:, :sh.heads]).astype(np.float32)
    beta = (0.05 + 0.9 * u[:, sh.heads:]).astype(np.float32)
    return alpha, beta


def gdn_conv_weights(sh: GdnShape, layer: int) -> np.ndarray:
    """bf16 bits [C][W]: G's unit-variance values halved (exact in bf16)."""
    n = sh.channels * sh.conv_width
    idx = np.uint64(layer) * np.uint64(n) + np.arange(n, dtype=_U64)
    v = bf16_bits_to_f32(bf16_at(sh.seed, TAG_GDN_W, idx)) * np.float32(0.5)
    return f32_to_bf16_rne(v).reshape(sh.channels, sh.conv_width)


def gdn_initial_state(sh: GdnShape, layer: int, b: int):
    """fp32 recurrent state [H][d][d] (G's values / 4, exact) and bf16
    convolution state [W-1][C] of sequence b before the first step."""
    H, d, C = sh.heads, sh.d, sh.channels
    n = H * d * d
    base = (np.uint64(layer) * np.uint64(GDN_MAX_B) + np.uint64(b)) * np.uint64(n)
    S = bf16_bits_to_f32(bf16_at(sh.seed, TAG_GDN_S0, base + np.arange(n, dtype=_U64))) * np.float32(0.25)
    m = (sh.conv_width - 1) * C
    cb = (np.uint64(layer) * np.uint64(GDN_MAX_B) + np.uint64(b)) * np.uint64(m)
    conv = bf16_at(sh.seed, TAG_GDN_C0, cb + np.arange(m, dtype=_U64)).reshape(sh.conv_width - 1, C)
    return S.reshape(H, d, d), conv
