// Device-side generator G: fills KV caches and per-step inputs with the
// same bits as synth/gen.py (SplitMix64 stream keyed by (seed, tag), one
// 64-bit hash per two values, value = (sum of the four bytes of a 32-bit
// word - 510) * float32(1/sqrt(21845)) rounded to bf16, nearest-even).
// Holds none of the decode method's arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kMix1 = 0xBF58476D1CE4E5B9ull;
constexpr uint64_t kMix2 = 0x94D049BB133111EBull;
constexpr int kMaxB = 32;
constexpr int kPosBits = 18;
constexpr int kMaxNeedles = 4;

__host__ __device__ __forceinline__ uint64_t splitmix64(uint64_t z) {
  z += kGamma;
  z = (z ^ (z >> 30)) * kMix1;
  z = (z ^ (z >> 27)) * kMix2;
  return z ^ (z >> 31);
}

__host__ __device__ __forceinline__ uint64_t stream_key(uint64_t seed, uint64_t tag) {
  return splitmix64(seed * 256ull + tag);
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint16_t value_of(uint32_t w) {
  const int x = (int)(w & 0xFFu) + (int)((w >> 8) & 0xFFu) + (int)((w >> 16) & 0xFFu) + (int)(w >> 24) - 510;
  const float scale = __uint_as_float(0x3BDDB446u);  // float32(1/sqrt(21845))
  return bf16_rne(__fmul_rn((float)x, scale));
}

// 8 consecutive values starting at an even logical index -> one uint4
__device__ __forceinline__ uint4 eight_values(uint64_t key, uint64_t idx0) {
  uint32_t out[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint64_t h = splitmix64(key + (idx0 >> 1) + k);
    out[k] = (uint32_t)value_of((uint32_t)h) | ((uint32_t)value_of((uint32_t)(h >> 32)) << 16);
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

__device__ __forceinline__ uint4 needle_row8(uint64_t key11, int n, int d, int i0) {
  uint32_t out[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint16_t v2[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint64_t idx = (uint64_t)n * d + i0 + 2 * k + e;
      const uint64_t h = splitmix64(key11 + (idx >> 1));
      const uint32_t w = (uint32_t)(h >> (32 * (idx & 1)));
      v2[e] = (w & 1u) ? (uint16_t)0x3FC0 : (uint16_t)0xBFC0;  // +-1.5
    }
    out[k] = (uint32_t)v2[0] | ((uint32_t)v2[1] << 16);
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

struct CacheFill {
  uint16_t* dst;
  uint64_t key, key11;
  int L, B, Hkv, d;
  int64_t t_rows;        // positions generated per (l, b, g): max t0
  const int32_t* t0;     // [B] positions [0, t0[b]) are filled
  int64_t t_cap;         // contiguous row stride
  const int32_t* tables; // paged or null
  int max_blocks, log2_block;
  int64_t num_blocks;
  int n_needles;
  int needles[kMaxNeedles];
  int layer0;            // first layer index of this fill (layers [layer0, layer0 + L))
};

// one thread per 8 values; rows enumerated as (l, b, g, p)
__global__ void k_fill_cache(CacheFill F) {
  const int per_row = F.d / 8;
  const uint64_t total = (uint64_t)F.L * F.B * F.Hkv * F.t_rows * per_row;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (uint64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i % per_row);
    uint64_t r = i / per_row;
    const int64_t p = (int64_t)(r % F.t_rows);
    r /= F.t_rows;
    const int g = (int)(r % F.Hkv);
    r /= F.Hkv;
    const int b = (int)(r % F.B);
    const int l = (int)(r / F.B);
    if (p >= F.t0[b]) continue;
    const int lg = F.layer0 + l;
    const uint64_t idx0 =
        (((((uint64_t)lg * kMaxB + b) * F.Hkv + g) << kPosBits) + (uint64_t)p) * F.d + (uint64_t)c * 8;
    uint4 v = eight_values(F.key, idx0);
    for (int n = 0; n < F.n_needles; ++n)
      if (p == F.needles[n]) v = needle_row8(F.key11, n, F.d, c * 8);
    size_t off;
    if (F.tables == nullptr) {
      off = ((((size_t)l * F.B + b) * F.Hkv + g) * (size_t)F.t_cap + (size_t)p) * F.d;
    } else {
      const int32_t blk = F.tables[(size_t)b * F.max_blocks + (p >> F.log2_block)];
      if (blk < 0 || blk >= F.num_blocks) continue;
      off = (((((size_t)l * F.num_blocks + blk) * F.Hkv + g) << F.log2_block) |
             (size_t)(p & ((1 << F.log2_block) - 1))) * F.d;
    }
    *reinterpret_cast<uint4*>(F.dst + off + c * 8) = v;
  }
}

struct StepFill {
  uint16_t* dst[7];      // qL, qF, kL, vL, kF, vF  [L][B][H][d];  e [B][D]
  uint64_t key[7];       // stream keys of tags 3..9
  uint64_t key11;
  int L, B, Hq, Hkv, d, D;
  int layers_total;      // index-space layer count of the workload
  const int32_t* pos;    // step j = pos[0] - t0[0] (read on the device)
  const int32_t* t0;
  int n_needles;
};

// blockIdx.y = tensor (0..6); threads over 8-value chunks
__global__ void k_fill_step(StepFill F) {
  const int which = blockIdx.y;
  const int j = F.pos[0] - F.t0[0];
  const int heads = which < 2 ? F.Hq : F.Hkv;
  const uint64_t total = which == 6 ? (uint64_t)F.B * F.D / 8 : (uint64_t)F.L * F.B * heads * F.d / 8;
  const bool aligned = F.n_needles > 0 && (j % 8) == 0;
  const int needle = aligned ? (j / 8) % F.n_needles : 0;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (uint64_t)gridDim.x * blockDim.x) {
    uint4 v;
    if (which == 6) {
      const uint64_t b = (i * 8) / F.D, e = (i * 8) % F.D;
      v = eight_values(F.key[6], ((uint64_t)j * kMaxB + b) * F.D + e);
    } else {
      uint64_t r = i * 8;
      const int e = (int)(r % F.d);
      r /= F.d;
      const int h = (int)(r % heads);
      r /= heads;
      const int b = (int)(r % F.B);
      const int l = (int)(r / F.B);
      if (which < 2 && aligned) {
        v = needle_row8(F.key11, needle, F.d, e);
      } else {
        // layer 0: the full branch reuses the local branch's streams
        int kw = which;
        if (l == 0 && (which == 1 || which == 4 || which == 5)) kw = which == 1 ? 0 : which - 2;
        const uint64_t idx = ((((uint64_t)j * F.layers_total + l) * kMaxB + b) * heads + h) * F.d + e;
        v = eight_values(F.key[kw], idx);
      }
    }
    *reinterpret_cast<uint4*>(F.dst[which] + i * 8) = v;
  }
}

// Decoder matrices (synth/gen.py dec_matrix_bits): element e of tensor T is
// bf16(((m - 2^21) + 0.5) * s) with m the top 22 bits of the hash of the
// logical index (T << 40) + e; one thread per 8 elements.
__global__ void k_fill_dec(uint16_t* dst, int64_t n, uint64_t key, uint64_t base, uint32_t scale_bits) {
  const float s = __uint_as_float(scale_bits);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 8;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8; i < n; i += stride) {
    uint32_t out[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint16_t v2[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint64_t h = splitmix64(key + base + (uint64_t)(i + 2 * k + e));
        const int m = (int)(h >> 42) - (1 << 21);
        v2[e] = bf16_rne(__fmul_rn(__fadd_rn((float)m, 0.5f), s));
      }
      out[k] = (uint32_t)v2[0] | ((uint32_t)v2[1] << 16);
    }
    *reinterpret_cast<uint4*>(dst + i) = make_uint4(out[0], out[1], out[2], out[3]);
  }
}

}  // namespace

extern "C" {

// n elements of decoder matrix `tensor_id` (n a multiple of 8, dst 16-B aligned).
int synth_fill_dec_matrix(uint16_t* dst, int64_t n, uint64_t seed, uint64_t tensor_id, uint32_t scale_bits,
                          hipStream_t stream) {
  if (dst == nullptr || n < 0 || n % 8 != 0 || (reinterpret_cast<uintptr_t>(dst) & 15) != 0) return -1;
  if (n == 0) return 0;
  const int64_t threads = n / 8;
  int64_t blocks = (threads + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_fill_dec, dim3((unsigned)blocks), dim3(256), 0, stream, dst, n, stream_key(seed, 16),
                     tensor_id << 40, scale_bits);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}


// Fills layers [layer0, layer0 + L) of a KV cache (tag 1 = K with needles,
// tag 2 = V).  Contiguous: dst [L][B][Hkv][t_cap][d]; paged: dst
// [L][num_blocks][Hkv][2^log2_block][d] with tables [B][max_blocks].
int synth_fill_cache(uint16_t* dst, uint64_t seed, int tag, int layer0, int L, int B, int Hkv, int d,
                     int64_t t_rows, const int32_t* t0, int64_t t_cap, const int32_t* tables, int max_blocks,
                     int log2_block, int64_t num_blocks, int n_needles, const int32_t* needles_host,
                     hipStream_t stream) {
  if (dst == nullptr || t0 == nullptr || d % 8 != 0 || n_needles < 0 || n_needles > kMaxNeedles) return -1;
  CacheFill F;
  F.dst = dst;
  F.key = stream_key(seed, (uint64_t)tag);
  F.key11 = stream_key(seed, 11);
  F.L = L;
  F.B = B;
  F.Hkv = Hkv;
  F.d = d;
  F.t_rows = t_rows;
  F.t0 = t0;
  F.t_cap = t_cap;
  F.tables = tables;
  F.max_blocks = max_blocks;
  F.log2_block = log2_block;
  F.num_blocks = num_blocks;
  F.n_needles = tag == 1 ? n_needles : 0;
  for (int n = 0; n < kMaxNeedles; ++n) F.needles[n] = (n < n_needles) ? needles_host[n] : -1;
  F.layer0 = layer0;
  hipLaunchKernelGGL(k_fill_cache, dim3(65536), dim3(256), 0, stream, F);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// Per-step inputs of step j = pos[0] - t0[0] (read on the device): qL, qF
// [L][B][Hq][d]; kL, vL, kF, vF [L][B][Hkv][d]; e [B][D].
int synth_fill_step(uint16_t* qL, uint16_t* qF, uint16_t* kL, uint16_t* vL, uint16_t* kF, uint16_t* vF,
                    uint16_t* e, uint64_t seed, int L, int B, int Hq, int Hkv, int d, const int32_t* pos,
                    const int32_t* t0, int n_needles, hipStream_t stream) {
  if (!qL || !qF || !kL || !vL || !kF || !vF || !e || !pos || !t0 || d % 8 != 0) return -1;
  StepFill F;
  uint16_t* dsts[7] = {qL, qF, kL, vL, kF, vF, e};
  for (int i = 0; i < 7; ++i) {
    F.dst[i] = dsts[i];
    F.key[i] = stream_key(seed, (uint64_t)(3 + i));
  }
  F.key11 = stream_key(seed, 11);
  F.L = L;
  F.B = B;
  F.Hq = Hq;
  F.Hkv = Hkv;
  F.d = d;
  F.D = Hq * d;
  F.layers_total = L;
  F.pos = pos;
  F.t0 = t0;
  F.n_needles = n_needles;
  hipLaunchKernelGGL(k_fill_step, dim3(256, 7), dim3(256), 0, stream, F);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
