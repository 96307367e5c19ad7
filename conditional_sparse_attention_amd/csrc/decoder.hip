// Dense decoder backbone around the ODA path, for gfx950.
//
// The pages run ODA inside a dense Qwen3 backbone in BF16 and recompute the
// whole backbone in both branches [On-Demand Attention notes §2.3, §3.3].
// The layer computed here is the pre-norm decoder layer of that family
// (QK-norm, RoPE, SwiGLU MLP, tied LM head); oda_decoder.h states it and its
// rounding points.
//
// At decode batch sizes every projection is a skinny GEMM that streams its
// bf16 weights from HBM once (2 bytes per 2 B flop), so one kernel serves
// them all: v_mfma_f32_16x16x32_bf16 with A = 16 weight rows x 32 k and B = 32
// k x 16 sequences.  In lane l = 16q + i the instruction takes A[i][8q..8q+7]
// and B[8q..8q+7][i] (one 16-byte load each) and returns D[4q + r][i] in
// accumulator component r.  A workgroup of NW waves owns TW row tiles and one
// K slice; a wave takes 4 blocks of 32 k per pass and issues all its loads
// before its first MFMA.  RMSNorm is fused into the operand load (the bf16
// operand is gamma * x, the sum of squares is gathered from the same fp32
// registers and the 1/rms scale lands on the finished dot product); the
// residual add, SiLU(gate) * up and the LM head's per-block argmax are the
// epilogues.  Waves are summed in LDS, K slices through coherent partial
// tiles and a ticket, the last workgroup adding them in slice order.
#include <math.h>

#include "oda_decoder.h"
#include "oda_internal.h"

namespace oda {
namespace {

using f4v = __attribute__((ext_vector_type(4))) float;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kJB = 4;                                // 32-k blocks per wave pass (128 k)
constexpr int kWaveK = kJB * 32;
constexpr int kMaxCols = 32;
constexpr int kMaxSlices = 16;                        // K slices of one GEMM launch, at most

enum GemmMode { kQkv = 0, kOut = 1, kGateUp = 2, kDown = 3, kLogits = 4 };

struct GemmArgs {
  const uint16_t* W0;     // [N][K] (gate rows for kGateUp)
  const uint16_t* W1;     // up rows (kGateUp)
  const uint16_t* gamma;  // [K] norm gain (kQkv, kGateUp)
  const float* xf;        // fp32 rows [B][K] (kQkv, kGateUp)
  const uint16_t* xb;     // bf16 rows [B][K] (kOut, kDown); h_local (kLogits)
  const uint16_t* xb2;    // h_full (kLogits)
  const uint8_t* flag;    // kLogits: row source per sequence
  uint16_t* out_b;        // bf16 [B][N] (kQkv, kGateUp: N = pair count)
  float* out_f;           // fp32 residual [B][N], updated in place (kOut, kDown)
  float* cand_v;          // kLogits: [row blocks][B] maximum
  int32_t* cand_i;        //          and its row
  float* part;            // split-K partial tiles
  int32_t* tickets;
  const int32_t* skip;    // work-list count: the kernel does nothing when it is 0
  int32_t B, N, K;
  float eps;
};

__device__ __forceinline__ float bf16f(uint32_t h16) { return __uint_as_float(h16 << 16); }
__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }
__device__ __forceinline__ float comp(const f4v v, int r) { return v[r]; }
__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}
__device__ __forceinline__ void part_put(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float part_get(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int TW, int NG>
constexpr int part_stride() {
  return TW * NG * 4 * 64 + 64;
}

template <int MODE, int TW, int NW, int NG>
__global__ void __launch_bounds__(NW * 64) k_gemm16(GemmArgs A) {
  constexpr int NT = NW * 64, JB = kJB;
  constexpr int NV = TW * NG * 4;  // accumulator floats per lane
  constexpr int PMAIN = NV * 64;
  constexpr int PSZ = part_stride<TW, NG>();
  constexpr bool kNorm = MODE == kQkv || MODE == kGateUp;
  constexpr int HALF = TW / 2;
  constexpr int ROWS = MODE == kGateUp ? HALF * 16 : TW * 16;
  constexpr int VPR = NV < 8192 / NT ? NV : 8192 / NT;  // accumulator values per LDS round (32 KB)
  static_assert(NV % VPR == 0, "LDS rounds");
  __shared__ float red[NW * VPR * 64];
  __shared__ float tile[PMAIN];
  __shared__ float s_ss[kMaxCols];
  __shared__ int s_last;
  if (A.skip != nullptr && *A.skip == 0) return;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, lq = lane >> 4;
  const int rb = blockIdx.x, ks = blockIdx.y, nks = gridDim.y;
  const int B = A.B, K = A.K;
  const int kslice = K / nks;
  const int iters = kslice / (NW * kWaveK);

  const uint16_t* wrow[TW];
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    if (MODE == kGateUp) {
      wrow[t] = (t < HALF ? A.W0 : A.W1) + (size_t)(rb * ROWS + 16 * (t < HALF ? t : t - HALF) + li) * K;
    } else {
      wrow[t] = A.W0 + (size_t)(rb * ROWS + 16 * t + li) * K;
    }
  }
  // batch columns past B repeat column B-1 (a column only reaches its own
  // output column, and those outputs are never written)
  int col[NG];
  const uint16_t* xsrc[NG];
#pragma unroll
  for (int cg = 0; cg < NG; ++cg) {
    col[cg] = min(16 * cg + li, B - 1);
    if (MODE == kLogits) {
      xsrc[cg] = (A.flag[col[cg]] ? A.xb2 : A.xb) + (size_t)col[cg] * K;
    } else {
      xsrc[cg] = A.xb + (size_t)col[cg] * K;
    }
  }

  f4v acc[TW][NG];
  float ss[NG];
#pragma unroll
  for (int t = 0; t < TW; ++t)
#pragma unroll
    for (int cg = 0; cg < NG; ++cg) acc[t][cg] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int cg = 0; cg < NG; ++cg) ss[cg] = 0.0f;

  for (int it = 0; it < iters; ++it) {
    const int k0 = ks * kslice + (it * NW + wave) * (JB * 32) + 8 * lq;  // + 32 j
    // operands from L2 first, then every weight load; the fence keeps them
    // all in flight before the first MFMA
    float4 xa[kNorm ? NG : 1][kNorm ? JB : 1][2];
    uint4 xr[kNorm ? 1 : NG][kNorm ? 1 : JB];
    uint4 g[kNorm ? JB : 1];
    if (kNorm) {
#pragma unroll
      for (int j = 0; j < JB; ++j) g[j] = *reinterpret_cast<const uint4*>(A.gamma + k0 + 32 * j);
#pragma unroll
      for (int cg = 0; cg < NG; ++cg) {
        const float* xp = A.xf + (size_t)col[cg] * K + k0;
#pragma unroll
        for (int j = 0; j < JB; ++j) {
          xa[cg][j][0] = *reinterpret_cast<const float4*>(xp + 32 * j);
          xa[cg][j][1] = *reinterpret_cast<const float4*>(xp + 32 * j + 4);
        }
      }
    } else {
#pragma unroll
      for (int cg = 0; cg < NG; ++cg)
#pragma unroll
        for (int j = 0; j < JB; ++j) xr[cg][j] = *reinterpret_cast<const uint4*>(xsrc[cg] + k0 + 32 * j);
    }
    uint4 w[TW][JB];
#pragma unroll
    for (int t = 0; t < TW; ++t)
#pragma unroll
      for (int j = 0; j < JB; ++j) w[t][j] = *reinterpret_cast<const uint4*>(wrow[t] + k0 + 32 * j);
    __builtin_amdgcn_sched_barrier(0);

    bf16x8 xb8[NG][JB];
#pragma unroll
    for (int cg = 0; cg < NG; ++cg) {
#pragma unroll
      for (int j = 0; j < JB; ++j) {
        if (kNorm) {
          const float4 a = xa[cg][j][0], b = xa[cg][j][1];
          const uint4 gg = g[j];
          ss[cg] += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w + b.x * b.x + b.y * b.y + b.z * b.z + b.w * b.w;
          uint4 u;
          u.x = pack2(bf16f(gg.x & 0xFFFFu) * a.x, bf16f(gg.x >> 16) * a.y);
          u.y = pack2(bf16f(gg.y & 0xFFFFu) * a.z, bf16f(gg.y >> 16) * a.w);
          u.z = pack2(bf16f(gg.z & 0xFFFFu) * b.x, bf16f(gg.z >> 16) * b.y);
          u.w = pack2(bf16f(gg.w & 0xFFFFu) * b.z, bf16f(gg.w >> 16) * b.w);
          xb8[cg][j] = as_bf16x8(u);
        } else {
          xb8[cg][j] = as_bf16x8(xr[cg][j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < JB; ++j)
#pragma unroll
      for (int t = 0; t < TW; ++t)
#pragma unroll
        for (int cg = 0; cg < NG; ++cg)
          acc[t][cg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w[t][j]), xb8[cg][j], acc[t][cg], 0, 0, 0);
  }

  // ---- waves -> LDS tile (value index v = (t * NG + cg) * 4 + r, lane l), in
  // rounds of VPR values
#pragma unroll
  for (int r0 = 0; r0 < NV; r0 += VPR) {
#pragma unroll
    for (int v = 0; v < VPR; ++v) {
      const int vv = r0 + v;
      red[(wave * VPR + v) * 64 + lane] = comp(acc[vv / (NG * 4)][(vv / 4) % NG], vv % 4);
    }
    __syncthreads();
    for (int i = tid; i < VPR * 64; i += NT) {
      float s = 0.0f;
#pragma unroll
      for (int wv = 0; wv < NW; ++wv) s += red[wv * VPR * 64 + i];
      tile[r0 * 64 + i] = s;
    }
    __syncthreads();
  }
  if (kNorm) {
#pragma unroll
    for (int cg = 0; cg < NG; ++cg) red[(wave * NG + cg) * 64 + lane] = ss[cg];
    __syncthreads();
    if (tid < NG * 16) {
      const int cg = tid >> 4, i = tid & 15;
      float s = 0.0f;
      for (int wv = 0; wv < NW; ++wv)
#pragma unroll
        for (int q = 0; q < 4; ++q) s += red[(wv * NG + cg) * 64 + 16 * q + i];
      s_ss[tid] = s;
    }
    __syncthreads();
  }

  // ---- K slices: coherent partial tiles, the last workgroup adds them
  if (nks > 1) {
    const int rbg = rb;
    float* pb = A.part + (size_t)rbg * nks * PSZ;
    for (int i = tid; i < PMAIN; i += NT) part_put(pb + (size_t)ks * PSZ + i, tile[i]);
    if (kNorm && tid < NG * 16) part_put(pb + (size_t)ks * PSZ + PMAIN + tid, s_ss[tid]);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(A.tickets + rbg, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nks - 1;
    __syncthreads();
    if (!s_last) return;
    // every slice's partial in one batch of loads, then added in slice order
    for (int i = tid; i < PMAIN; i += NT) {
      float v[kMaxSlices];
#pragma unroll
      for (int sp = 0; sp < kMaxSlices; ++sp)
        if (sp < nks) v[sp] = part_get(pb + (size_t)sp * PSZ + i);
      float s = 0.0f;
#pragma unroll
      for (int sp = 0; sp < kMaxSlices; ++sp)
        if (sp < nks) s += v[sp];
      tile[i] = s;
    }
    if (kNorm && tid < NG * 16) {
      float v[kMaxSlices];
#pragma unroll
      for (int sp = 0; sp < kMaxSlices; ++sp)
        if (sp < nks) v[sp] = part_get(pb + (size_t)sp * PSZ + PMAIN + tid);
      float s = 0.0f;
#pragma unroll
      for (int sp = 0; sp < kMaxSlices; ++sp)
        if (sp < nks) s += v[sp];
      s_ss[tid] = s;
    }
    if (tid == 0) __hip_atomic_store(A.tickets + rbg, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
  }

  // ---- epilogue from the LDS tile
  if (MODE == kLogits) {
    if (tid < NG * 16 && tid < B) {
      const int c = tid, cg = c >> 4, ci = c & 15;
      float best = -INFINITY;
      int brow = 0;
      for (int row = 0; row < TW * 16; ++row) {
        const int t = row >> 4, q = (row >> 2) & 3, r = row & 3;
        const float v = tile[((t * NG + cg) * 4 + r) * 64 + 16 * q + ci];
        if (v > best) {
          best = v;
          brow = row;
        }
      }
      A.cand_v[(size_t)rb * B + c] = best;
      A.cand_i[(size_t)rb * B + c] = rb * ROWS + brow;
    }
    return;
  }
  constexpr int NOUT = MODE == kGateUp ? PMAIN / 2 : PMAIN;
  for (int i = tid; i < NOUT; i += NT) {
    const int v = i >> 6, l = i & 63;
    const int t = v / (NG * 4), cg = (v >> 2) % NG, r = v & 3;
    const int c = 16 * cg + (l & 15);
    if (c >= B) continue;
    const int n = rb * ROWS + 16 * t + 4 * (l >> 4) + r;
    const float y = tile[i];
    if (MODE == kQkv) {
      const float rs = rsqrtf(s_ss[c] / (float)K + A.eps);
      A.out_b[(size_t)c * A.N + n] = f32_to_bf16(rs * y);
    } else if (MODE == kGateUp) {
      const float rs = rsqrtf(s_ss[c] / (float)K + A.eps);
      const float gv = bf16_to_f32(f32_to_bf16(rs * y));
      const float uv = bf16_to_f32(f32_to_bf16(rs * tile[i + PMAIN / 2]));
      A.out_b[(size_t)c * A.N + n] = f32_to_bf16(silu(gv) * uv);
    } else {
      A.out_f[(size_t)c * A.N + n] += y;
    }
  }
}

// ---- per-head QK-norm + RoPE (the full branch); the v heads are copied.  grid (Hq + 2 Hkv, B), one wave.
struct RopeArgs {
  const uint16_t* qkv;   // [B][(Hq + 2 Hkv) d]
  const uint16_t* gq;    // [d]
  const uint16_t* gk;
  const int32_t* pos;
  uint16_t* q;           // [B][Hq][d]
  uint16_t* k;           // [B][Hkv][d]
  uint16_t* v;
  const int32_t* skip;
  int32_t Hq, Hkv;
  float eps;
  double theta;
};

__global__ void __launch_bounds__(64) k_qk_rope(RopeArgs A) {
  if (A.skip != nullptr && *A.skip == 0) return;
  constexpr int d = kHeadDim, half = kHeadDim / 2;
  const int h = blockIdx.x, b = blockIdx.y, i = threadIdx.x;  // pair (i, i + 64)
  const int nh = A.Hq + 2 * A.Hkv;
  const uint16_t* src = A.qkv + ((size_t)b * nh + h) * d;
  if (h >= A.Hq + A.Hkv) {
    uint16_t* dst = A.v + ((size_t)b * A.Hkv + (h - A.Hq - A.Hkv)) * d;
    dst[i] = src[i];
    dst[i + half] = src[i + half];
    return;
  }
  const float x1 = bf16_to_f32(src[i]), x2 = bf16_to_f32(src[i + half]);
  float s = x1 * x1 + x2 * x2;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
  const float rs = rsqrtf(s / (float)d + A.eps);
  const bool isq = h < A.Hq;
  const uint16_t* gm = isq ? A.gq : A.gk;
  const float y1 = bf16_to_f32(gm[i]) * x1 * rs, y2 = bf16_to_f32(gm[i + half]) * x2 * rs;
  // angle in double: positions reach 1e5 and more, past fp32's resolution
  const double ang = (double)A.pos[b] * pow(A.theta, -2.0 * (double)i / (double)d);
  const float c = (float)cos(ang), sn = (float)sin(ang);
  uint16_t* dst = isq ? A.q + ((size_t)b * A.Hq + h) * d : A.k + ((size_t)b * A.Hkv + (h - A.Hq)) * d;
  dst[i] = f32_to_bf16(y1 * c - y2 * sn);
  dst[i + half] = f32_to_bf16(y2 * c + y1 * sn);
}

// ---- the step's RoPE table: (cos, sin) of pos_b * theta^(-2i/d) for i < d/2,
// per sequence, read by the local attention kernel's QK-norm + RoPE.  The angle is
// formed in double: positions reach 1e5 and more, past fp32's resolution.
// grid (B), d/2 threads.
__global__ void __launch_bounds__(64) k_rope_table(const int32_t* pos, double theta, float* cs) {
  constexpr int half = kHeadDim / 2;
  const int b = blockIdx.x, i = threadIdx.x;
  const double ang = (double)pos[b] * pow(theta, -2.0 * (double)i / (double)kHeadDim);
  float* t = cs + ((size_t)b * half + i) * 2;
  t[0] = (float)cos(ang);
  t[1] = (float)sin(ang);
}

// ---- token embedding: x rows (fp32) and the head's E(x_t) (bf16).  grid (B)
__global__ void __launch_bounds__(256) k_embed(const uint16_t* E, const int32_t* tokens, float* xl, float* xf,
                                               uint16_t* emb, int32_t* err, int D, int V) {
  const int b = blockIdx.x;
  int tok = tokens[b];
  if (tok < 0 || tok >= V) {
    if (threadIdx.x == 0 && err != nullptr) atomicOr(err, ODA_ERR_TOKEN);
    tok = 0;
  }
  const uint16_t* row = E + (size_t)tok * D;
  for (int i = threadIdx.x; i < D; i += 256) {
    const uint16_t v = row[i];
    const float f = bf16_to_f32(v);
    if (xl != nullptr) xl[(size_t)b * D + i] = f;
    if (xf != nullptr) xf[(size_t)b * D + i] = f;
    emb[(size_t)b * D + i] = v;
  }
}

// ---- final RMSNorm to the step's hidden state.  grid (B)
__global__ void __launch_bounds__(256) k_final_norm(const uint16_t* gamma, const float* x, uint16_t* h,
                                                    const int32_t* skip, int D, float eps) {
  if (skip != nullptr && *skip == 0) return;
  __shared__ float s_part[4];
  const int b = blockIdx.x, tid = threadIdx.x;
  const float* xr = x + (size_t)b * D;
  float s = 0.0f;
  for (int i = tid; i < D; i += 256) s += xr[i] * xr[i];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
  if ((tid & 63) == 0) s_part[tid >> 6] = s;
  __syncthreads();
  const float rs = rsqrtf((s_part[0] + s_part[1] + s_part[2] + s_part[3]) / (float)D + eps);
  for (int i = tid; i < D; i += 256) h[(size_t)b * D + i] = f32_to_bf16(bf16_to_f32(gamma[i]) * xr[i] * rs);
}

// ---- argmax over the LM head's row-block candidates.  grid (B)
__global__ void __launch_bounds__(256) k_argmax(const float* cand_v, const int32_t* cand_i, int nrb, int B,
                                                int32_t* tokens, float* max_logit) {
  __shared__ float s_v[256];
  __shared__ int s_i[256];
  const int b = blockIdx.x, tid = threadIdx.x;
  float best = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int r = tid; r < nrb; r += 256) {
    const float v = cand_v[(size_t)r * B + b];
    const int i = cand_i[(size_t)r * B + b];
    if (v > best || (v == best && i < bi)) {
      best = v;
      bi = i;
    }
  }
  s_v[tid] = best;
  s_i[tid] = bi;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (tid < w) {
      const float v = s_v[tid + w];
      const int i = s_i[tid + w];
      if (v > s_v[tid] || (v == s_v[tid] && i < s_i[tid])) {
        s_v[tid] = v;
        s_i[tid] = i;
      }
    }
    __syncthreads();
  }
  if (tid == 0) {
    tokens[b] = s_i[0] == 0x7FFFFFFF ? 0 : s_i[0];
    if (max_logit != nullptr) max_logit[b] = s_v[0];
  }
}

// ------------------------------------------------------------------ host
struct DecDerived {
  int B, D, Hq, Hkv, d, I, V, L;
  int nqkv;           // (Hq + 2 Hkv) d
  int64_t offs[ODA_DEC_NTENSORS + 1];
};

bool dec_derive(const oda_dec_dims* dd, DecDerived* o, int* st) {
  if (dd == nullptr) {
    *st = ODA_E_NULL;
    return false;
  }
  if (!dims_valid(&dd->attn, st)) return false;
  const oda_dims& a = dd->attn;
  o->B = a.batch;
  o->D = a.hidden;
  o->Hq = a.num_q_heads;
  o->Hkv = a.num_kv_heads;
  o->d = a.head_dim;
  o->I = dd->inter;
  o->V = dd->vocab;
  o->L = a.num_layers;
  o->nqkv = (o->Hq + 2 * o->Hkv) * o->d;
  if (o->I <= 0 || o->V <= 0 || !(dd->eps > 0.0f) || !(dd->rope_theta > 1.0f)) {
    *st = ODA_E_DIMS;
    return false;
  }
  if (o->D % 1024 != 0 || o->I % 1024 != 0 || o->V % 64 != 0 ||
      o->nqkv % 16 != 0 || o->B > kMaxCols) {
    *st = ODA_E_UNSUPPORTED;
    return false;
  }
  const int64_t D = o->D, d = o->d, I = o->I;
  const int64_t sizes[ODA_DEC_NTENSORS] = {D, (int64_t)o->nqkv * D, d, d, D * o->Hq * d, D, I * D, I * D, D * I};
  int64_t at = 0;
  for (int i = 0; i < ODA_DEC_NTENSORS; ++i) {
    o->offs[i] = at;
    at += sizes[i];
  }
  o->offs[ODA_DEC_NTENSORS] = at;
  *st = ODA_OK;
  return true;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct DecWs {
  size_t qkv, act, part, tickets, cand_v, cand_i, rope, total;
};

// Shape of one GEMM launch: row tiles per workgroup, waves per workgroup,
// row blocks and K slices.  The QKV and output projections use 16-row tiles
// and 16 waves where K splits into 16 shares of 128 (else 8 waves, several
// passes each), each wave loading its whole share at once, and a single K
// slice: 256 and 128 workgroups at D = 2048, no cross-workgroup hand-off.
// The LM head has rows enough for 64-row tiles of 4 waves.
struct GemmShape {
  int tw, nw, nrb, nks;
};
// RMSNorm-fused modes hold the fp32 operand too: with two column groups
// (B > 16) they run 8 waves inside the 1024-thread register budget.
int waves_for(int K, bool norm_two_groups) { return K % (16 * kWaveK) == 0 && !norm_two_groups ? 16 : 8; }
GemmShape shape_qkv(const DecDerived& g) { return {1, waves_for(g.D, g.B > 16), g.nqkv / 16, 1}; }
GemmShape shape_out(const DecDerived& g) { return {1, waves_for(g.Hq * g.d, false), g.D / 16, 1}; }
// Gate/up holds x, the gains and both weight tiles (117 VGPRs at 16 waves):
// one 16-wave workgroup per CU, so its I / 16 workgroups (384 at I = 6144)
// would run in two rounds.  At 8 waves, two passes each, two workgroups fit
// per CU and one round holds them (measured 1-2% faster per decoder step).
GemmShape shape_gateup(const DecDerived& g) { return {2, 8, g.I / 16, 1}; }
// Down (K = I): 8 waves and I / 1024 K slices (6 at I = 6144) keep more
// workgroups loading at once than 16 waves and half the slices (measured
// 0.5% faster per step).
GemmShape shape_down(const DecDerived& g) { return {1, 8, g.D / 16, g.I / (8 * kWaveK)}; }
GemmShape shape_logits(const DecDerived& g) { return {4, 4, g.V / 64, 1}; }

DecWs dec_ws(const DecDerived& g) {
  const GemmShape s4[4] = {shape_qkv(g), shape_out(g), shape_gateup(g), shape_down(g)};
  size_t part = 0, tick = 0;
  for (int i = 0; i < 4; ++i) {
    const size_t psz = (size_t)s4[i].tw * 2 * 4 * 64 + 64;  // two column groups: the largest tile
    const size_t n = s4[i].nks > 1 ? (size_t)s4[i].nrb * s4[i].nks * psz : 0;
    if (n > part) part = n;
    if ((size_t)s4[i].nrb > tick) tick = s4[i].nrb;
  }
  DecWs w;
  size_t at = 0;
  w.tickets = at;
  at = align256(at + tick * sizeof(int32_t));
  w.qkv = at;
  at = align256(at + (size_t)g.B * g.nqkv * 2);
  w.act = at;
  at = align256(at + (size_t)g.B * g.I * 2);
  w.part = at;
  at = align256(at + part * sizeof(float));
  w.cand_v = at;
  at = align256(at + (size_t)(g.V / 64) * g.B * sizeof(float));
  w.cand_i = at;
  at = align256(at + (size_t)(g.V / 64) * g.B * sizeof(int32_t));
  w.rope = at;
  at = align256(at + (size_t)g.B * kHeadDim * sizeof(float));
  w.total = at;
  return w;
}

template <int MODE, int TW, int NW>
int launch_gemm_nw(const GemmArgs& a, GemmShape s, hipStream_t st) {
  const dim3 grid(s.nrb, s.nks);
  constexpr bool kNorm = MODE == kQkv || MODE == kGateUp;
  if (a.B <= 16) {
    hipLaunchKernelGGL((k_gemm16<MODE, TW, NW, 1>), grid, dim3(NW * 64), 0, st, a);
  } else if constexpr (!(kNorm && NW == 16)) {  // those run 8 waves at B > 16 (register budget)
    hipLaunchKernelGGL((k_gemm16<MODE, TW, NW, 2>), grid, dim3(NW * 64), 0, st, a);
  } else {
    return ODA_E_UNSUPPORTED;
  }
  return ODA_OK;
}

template <int MODE, int TW>
int launch_gemm(const GemmArgs& a, GemmShape s, hipStream_t st) {
  if (s.tw != TW || s.nks > kMaxSlices || a.K % (s.nks * s.nw * kWaveK) != 0 || a.K / s.nks < s.nw * kWaveK)
    return ODA_E_UNSUPPORTED;
  int rc;
  if constexpr (MODE == kLogits) {
    if (s.nw != 4) return ODA_E_UNSUPPORTED;
    rc = launch_gemm_nw<MODE, TW, 4>(a, s, st);
  } else {
    if (s.nw == 8)
      rc = launch_gemm_nw<MODE, TW, 8>(a, s, st);
    else if (s.nw == 16)
      rc = launch_gemm_nw<MODE, TW, 16>(a, s, st);
    else
      return ODA_E_UNSUPPORTED;
  }
  if (rc != ODA_OK) return rc;
  return hipGetLastError() == hipSuccess ? ODA_OK : ODA_E_LAUNCH;
}

const int32_t* worklist_count(const oda_dims* a, void* attn_ws) {
  const WsLayout L = ws_layout(a);
  return reinterpret_cast<const int32_t*>(static_cast<char*>(attn_ws) + L.worklist);
}

}  // namespace
}  // namespace oda

using namespace oda;

extern "C" {

int64_t oda_dec_layer_numel(const oda_dec_dims* dims) {
  DecDerived g;
  int st;
  if (!dec_derive(dims, &g, &st)) return -1;
  return g.offs[ODA_DEC_NTENSORS];
}

int oda_dec_layer_offsets(const oda_dec_dims* dims, int64_t* offsets) {
  DecDerived g;
  int st;
  if (offsets == nullptr) return ODA_E_NULL;
  if (!dec_derive(dims, &g, &st)) return st;
  for (int i = 0; i <= ODA_DEC_NTENSORS; ++i) offsets[i] = g.offs[i];
  return ODA_OK;
}

size_t oda_dec_workspace_bytes(const oda_dec_dims* dims) {
  DecDerived g;
  int st;
  if (!dec_derive(dims, &g, &st)) return 0;
  return dec_ws(g).total;
}

int oda_dec_workspace_init(const oda_dec_dims* dims, void* dws, size_t dws_bytes, hipStream_t stream) {
  DecDerived g;
  int st;
  if (!dec_derive(dims, &g, &st)) return st;
  if (dws == nullptr) return ODA_E_NULL;
  const DecWs w = dec_ws(g);
  if (dws_bytes < w.total) return ODA_E_WORKSPACE;
  return launch_fill_zero(static_cast<int32_t*>(dws), w.qkv / sizeof(int32_t), stream);
}

int oda_dec_embed(const oda_dec_dims* dims, const oda_bf16* embed, const int32_t* tokens, float* x_local,
                  float* x_full, oda_bf16* emb, void* attn_ws, size_t attn_ws_bytes, hipStream_t stream) {
  DecDerived g;
  int st;
  if (!dec_derive(dims, &g, &st)) return st;
  if (embed == nullptr || tokens == nullptr || emb == nullptr) return ODA_E_NULL;
  int32_t* err = nullptr;
  if (attn_ws != nullptr) {
    const WsLayout L = ws_layout(&dims->attn);
    if (attn_ws_bytes < L.total) return ODA_E_WORKSPACE;
    err = reinterpret_cast<int32_t*>(static_cast<char*>(attn_ws) + L.header);
  }
  hipLaunchKernelGGL(k_embed, dim3(g.B), dim3(256), 0, stream, embed, tokens, x_local, x_full, emb, err, g.D, g.V);
  return hipGetLastError() == hipSuccess ? ODA_OK : ODA_E_LAUNCH;
}

int oda_dec_layer(const oda_dec_dims* dims, int32_t layer, int32_t branch, const oda_bf16* w_layer,
                  const oda_kv* kv, const int32_t* pos, float* x, oda_bf16* q, oda_bf16* k_cur, oda_bf16* v_cur,
                  oda_bf16* o, void* attn_ws, size_t attn_ws_bytes, void* dws, size_t dws_bytes,
                  hipStream_t stream) {
  DecDerived g;
  int st;
  if (!dec_derive(dims, &g, &st)) return st;
  if (branch != ODA_DEC_LOCAL && branch != ODA_DEC_FULL) return ODA_E_DIMS;
  if (layer < 0 || layer >= g.L) return ODA_E_LAYER;
  if (w_layer == nullptr || kv == nullptr || pos == nullptr || x == nullptr || q == nullptr ||
      k_cur == nullptr || v_cur == nullptr || o == nullptr || attn_ws == nullptr || dws == nullptr)
    return ODA_E_NULL;
  const WsLayout AL = ws_layout(&dims->attn);
  const DecWs W = dec_ws(g);
  if (attn_ws_bytes < AL.total || dws_bytes < W.total) return ODA_E_WORKSPACE;
  char* dw = static_cast<char*>(dws);
  uint16_t* qkv = reinterpret_cast<uint16_t*>(dw + W.qkv);
  uint16_t* act = reinterpret_cast<uint16_t*>(dw + W.act);
  float* part = reinterpret_cast<float*>(dw + W.part);
  int32_t* tickets = reinterpret_cast<int32_t*>(dw + W.tickets);
  const int32_t* skip = branch == ODA_DEC_FULL ? worklist_count(&dims->attn, attn_ws) : nullptr;
  const uint16_t* wl = w_layer;

  GemmArgs a{};
  a.part = part;
  a.tickets = tickets;
  a.skip = skip;
  a.B = g.B;
  a.eps = dims->eps;
  // q, k, v projections (RMSNorm fused)
  a.W0 = wl + g.offs[1];
  a.gamma = wl + g.offs[0];
  a.xf = x;
  a.out_b = qkv;
  a.N = g.nqkv;
  a.K = g.D;
  if ((st = launch_gemm<kQkv, 1>(a, shape_qkv(g), stream)) != ODA_OK) return st;
  // attention of the branch (the ODA path).  The local branch runs the
  // attention in decoder mode: its kernel applies the QK-norm and RoPE to the
  // raw q / k rows and stages the current key / value, from the step's RoPE
  // table, which layer 0 writes.  The full branch's persistent kernel walks
  // several units per workgroup, each of which would redo that work, so it
  // keeps a separate QK-norm + RoPE launch.
  if (branch == ODA_DEC_LOCAL) {
    float* rope = reinterpret_cast<float*>(dw + W.rope);
    if (layer == 0) {
      hipLaunchKernelGGL(k_rope_table, dim3(g.B), dim3(kHeadDim / 2), 0, stream, pos, (double)dims->rope_theta, rope);
      if (hipGetLastError() != hipSuccess) return ODA_E_LAUNCH;
    }
    st = decoder_local_attn(&dims->attn, layer, kv, pos, qkv, wl + g.offs[2], wl + g.offs[3], rope, dims->eps, k_cur,
                            v_cur, o, attn_ws, attn_ws_bytes, stream);
  } else {
    RopeArgs r{};
    r.qkv = qkv;
    r.gq = wl + g.offs[2];
    r.gk = wl + g.offs[3];
    r.pos = pos;
    r.q = q;
    r.k = k_cur;
    r.v = v_cur;
    r.skip = skip;
    r.Hq = g.Hq;
    r.Hkv = g.Hkv;
    r.eps = dims->eps;
    r.theta = (double)dims->rope_theta;
    hipLaunchKernelGGL(k_qk_rope, dim3(g.Hq + 2 * g.Hkv, g.B), dim3(64), 0, stream, r);
    if (hipGetLastError() != hipSuccess) return ODA_E_LAUNCH;
    st = oda_full_attn_if(&dims->attn, layer, kv, pos, q, k_cur, v_cur, o, nullptr, attn_ws, attn_ws_bytes, stream);
  }
  if (st != ODA_OK) return st;
  // output projection + residual
  a.W0 = wl + g.offs[4];
  a.gamma = nullptr;
  a.xf = nullptr;
  a.xb = o;
  a.out_b = nullptr;
  a.out_f = x;
  a.N = g.D;
  a.K = g.Hq * g.d;
  if ((st = launch_gemm<kOut, 1>(a, shape_out(g), stream)) != ODA_OK) return st;
  // gate / up (RMSNorm fused) -> SiLU(g) * u
  a.W0 = wl + g.offs[6];
  a.W1 = wl + g.offs[7];
  a.gamma = wl + g.offs[5];
  a.xf = x;
  a.xb = nullptr;
  a.out_b = act;
  a.out_f = nullptr;
  a.N = g.I;
  a.K = g.D;
  if ((st = launch_gemm<kGateUp, 2>(a, shape_gateup(g), stream)) != ODA_OK) return st;
  // down projection + residual
  a.W0 = wl + g.offs[8];
  a.W1 = nullptr;
  a.gamma = nullptr;
  a.xf = nullptr;
  a.xb = act;
  a.out_b = nullptr;
  a.out_f = x;
  a.N = g.D;
  a.K = g.I;
  return launch_gemm<kDown, 1>(a, shape_down(g), stream);
}

int oda_dec_final_norm(const oda_dec_dims* dims, int32_t branch, const oda_bf16* gamma_f, const float* x,
                       oda_bf16* h, void* attn_ws, size_t attn_ws_bytes, hipStream_t stream) {
  DecDerived g;
  int st;
  if (!dec_derive(dims, &g, &st)) return st;
  if (branch != ODA_DEC_LOCAL && branch != ODA_DEC_FULL) return ODA_E_DIMS;
  if (gamma_f == nullptr || x == nullptr || h == nullptr) return ODA_E_NULL;
  const int32_t* skip = nullptr;
  if (branch == ODA_DEC_FULL) {
    if (attn_ws == nullptr) return ODA_E_NULL;
    if (attn_ws_bytes < ws_layout(&dims->attn).total) return ODA_E_WORKSPACE;
    skip = worklist_count(&dims->attn, attn_ws);
  }
  hipLaunchKernelGGL(k_final_norm, dim3(g.B), dim3(256), 0, stream, gamma_f, x, h, skip, g.D, dims->eps);
  return hipGetLastError() == hipSuccess ? ODA_OK : ODA_E_LAUNCH;
}

int oda_dec_next_token(const oda_dec_dims* dims, const oda_bf16* embed, const oda_bf16* h_local,
                       const oda_bf16* h_full, const uint8_t* flag, int32_t* tokens, float* max_logit, void* dws,
                       size_t dws_bytes, hipStream_t stream) {
  DecDerived g;
  int st;
  if (!dec_derive(dims, &g, &st)) return st;
  if (embed == nullptr || h_local == nullptr || h_full == nullptr || flag == nullptr || tokens == nullptr ||
      dws == nullptr)
    return ODA_E_NULL;
  const DecWs W = dec_ws(g);
  if (dws_bytes < W.total) return ODA_E_WORKSPACE;
  char* dw = static_cast<char*>(dws);
  GemmArgs a{};
  a.W0 = embed;
  a.xb = h_local;
  a.xb2 = h_full;
  a.flag = flag;
  a.cand_v = reinterpret_cast<float*>(dw + W.cand_v);
  a.cand_i = reinterpret_cast<int32_t*>(dw + W.cand_i);
  a.B = g.B;
  a.N = g.V;
  a.K = g.D;
  a.eps = dims->eps;
  if ((st = launch_gemm<kLogits, 4>(a, shape_logits(g), stream)) != ODA_OK) return st;
  hipLaunchKernelGGL(k_argmax, dim3(g.B), dim3(256), 0, stream, a.cand_v, a.cand_i, g.V / 64, g.B, tokens,
                     max_logit);
  return hipGetLastError() == hipSuccess ? ODA_OK : ODA_E_LAUNCH;
}

}  // extern "C"
