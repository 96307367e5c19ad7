// Recall head R_psi, branch rule and full-branch work list, for gfx950.
//
// q_t = R_psi(h_{t-1}, E(x_t), h_t^L)  [On-Demand Attention notes §2.2,
// equation for q_t and the architecture paragraph], fp32 weights and math:
//   a, b, c  = silu(W_s rmsnorm(x_s) + c_s)               three towers, D -> 1024
//   u        = W_I [a,b,c,ab,ac,bc,|a-b|,|a-c|,|b-c|] + c_I + (a + b + c)
//   u       += W_down(silu(W_gate r) * (W_up r)), r = rmsnorm(u)    (x2)
//   q        = w_o . rmsnorm(u) + c_o
// then the rule of §2.3: full when q > theta or q is not finite, unless the
// caller forces the branch; then the compacted full-branch work list.
//
// At decode batch sizes every layer is a skinny matrix-vector product that
// streams its fp32 weights once from HBM (4 bytes per 2*B flops), so the
// kernels are bandwidth-shaped GEMVs.  One wave owns R output rows: its 64
// lanes hold the rows' weights in registers (16-byte loads, all issued at
// once), then sweep every batch row against them, so the weights are read
// from HBM exactly once whatever the batch; the batch inputs come from L2.
// The batch inputs of a layer (a few KB per sequence) are copied once per
// workgroup into LDS with direct-to-LDS loads issued right after the
// weights, so every batch row arrives in one memory round trip instead of
// one per row; biases and residual operands are loaded before any store.
// The dot products are reduced inside the wave (DPP row sums + readlane).
// RMSNorm scales are folded in after the dot product (W (gamma*x) / rms(x)),
// the sum of squares gathered in the same pass; the interaction vector is
// formed on the fly from the tower outputs.
#include "head_internal.h"

namespace oda {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr float kEps = 1e-6f;

__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }
__device__ __forceinline__ float dot4(const float4 a, const float4 b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}
__device__ __forceinline__ float4 mul4(const float4 a, const float4 b) {
  return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w);
}
__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 ldbf4(const uint16_t* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  return make_float4(bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y));
}

// Copies the first n 16-byte chunks of `src` into `dst` (LDS) with
// direct-to-LDS loads, chunk c by thread c % kThreads: the LDS address of a
// wave's load is its first lane's chunk, each lane writing 16 bytes after the
// previous lane's.  The caller waits (stage_wait) before reading.
template <int MAXC>
__device__ __forceinline__ void stage_lds(const void* src, int n, void* dst) {
  const int tid = threadIdx.x, lane = tid & 63;
  const uint4* g = static_cast<const uint4*>(src);
  uint4* l = static_cast<uint4*>(dst);
#pragma unroll
  for (int j = 0; j < MAXC; ++j) {
    const int c = j * kThreads + tid;
    if (c < n) __builtin_amdgcn_global_load_lds(g + c, l + (c - lane), 16, 0, 0);
  }
}
// Every load of the workgroup has landed (the staged rows included), then
// the staged LDS is visible to all waves.
__device__ __forceinline__ void stage_wait() {
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ------------------------------------------------------------------ towers
struct TowerArgs {
  const float* w;  // blob
  int64_t off_gamma[3], off_W[3], off_c[3];
  const uint16_t* x[3];  // h_prev, emb, h_local  [B][D] bf16
  float* out;            // towers [3][B][T]
  int B;
};

// KI = D / 256 float4 per lane per row; R rows per wave; NBM >= B.
// grid (T / (4R), 3 towers)
template <int KI, int R, int NBM>
__global__ void __launch_bounds__(kThreads) k_tower(TowerArgs A) {
  constexpr int D = KI * 256;
  constexpr int CPR = D / 8;  // 16-byte chunks of one bf16 input row
  __shared__ uint4 s_x[NBM * CPR];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tw = blockIdx.y;
  const int n0 = (blockIdx.x * kWaves + wave) * R;
  const float* W = A.w + A.off_W[tw] + (size_t)n0 * D + lane * 4;
  const float* gam = A.w + A.off_gamma[tw] + lane * 4;
  float4 w[R][KI];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < KI; ++i) w[r][i] = ld4(W + (size_t)r * D + 256 * i);
  float4 g[KI];
#pragma unroll
  for (int i = 0; i < KI; ++i) g[i] = ld4(gam + 256 * i);
  const float* cb = A.w + A.off_c[tw] + n0;
  float cbv[R];
#pragma unroll
  for (int r = 0; r < R; ++r) cbv[r] = cb[r];
  stage_lds<(NBM * CPR + kThreads - 1) / kThreads>(A.x[tw], A.B * CPR, s_x);
  stage_wait();
  const uint2* sx = reinterpret_cast<const uint2*>(s_x);
  float acc[R][NBM], ss[NBM];
#pragma unroll
  for (int b = 0; b < NBM; ++b) {
    ss[b] = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r][b] = 0.0f;
    if (b < A.B) {
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        const uint2 raw = sx[(b * D + 256 * i) / 4 + lane];
        const float4 xv = make_float4(bf16lo(raw.x), bf16hi(raw.x), bf16lo(raw.y), bf16hi(raw.y));
        const float4 in = mul4(xv, g[i]);
        ss[b] += dot4(xv, xv);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][b] += dot4(w[r][i], in);
      }
    }
  }
#pragma unroll
  for (int b = 0; b < NBM; ++b) {
    if (b < A.B) {
      const float inv = rsqrtf(wave_sum64(ss[b]) / (float)D + kEps);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float v = wave_sum64(acc[r][b]);
        if (lane == 0) A.out[((size_t)tw * A.B + b) * kTower + n0 + r] = silu(v * inv + cbv[r]);
      }
    }
  }
}

// ------------------------------------------------------------- interaction
struct InteractArgs {
  const float* W;       // W_I [T][9T]
  const float* bias;    // c_I
  const float* towers;  // [3][B][T]
  float* out;           // u0 [B][T]
  int B;
};

__device__ __forceinline__ float4 seg_value(int seg, const float4 a, const float4 b, const float4 c) {
  switch (seg) {
    case 0: return a;
    case 1: return b;
    case 2: return c;
    case 3: return mul4(a, b);
    case 4: return mul4(a, c);
    case 5: return mul4(b, c);
    case 6: return make_float4(fabsf(a.x - b.x), fabsf(a.y - b.y), fabsf(a.z - b.z), fabsf(a.w - b.w));
    case 7: return make_float4(fabsf(a.x - c.x), fabsf(a.y - c.y), fabsf(a.z - c.z), fabsf(a.w - c.w));
    default: return make_float4(fabsf(b.x - c.x), fabsf(b.y - c.y), fabsf(b.z - c.z), fabsf(b.w - c.w));
  }
}

// One wave per output row.  The lane's 36 float4 of the 9216-long row are
// loaded at once (chunk q holds element q*256 + 4*lane of each of the 9
// segments), so one (a, b, c) float4 per batch row and chunk serves all 9
// segment values of that chunk.  grid (T / 4)
template <int NBM>
__global__ void __launch_bounds__(kThreads) k_interact(InteractArgs A) {
  __shared__ float4 s_t[3 * NBM * kTower / 4];  // towers [3][B][T]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = blockIdx.x * kWaves + wave;
  const float* W = A.W + (size_t)n * (9 * kTower) + lane * 4;
  float4 w[4][9];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int s = 0; s < 9; ++s) w[q][s] = ld4(W + s * kTower + q * 256);
  const float cI = A.bias[n];
  stage_lds<(3 * NBM * kTower / 4 + kThreads - 1) / kThreads>(A.towers, 3 * A.B * kTower / 4, s_t);
  stage_wait();
  const float* st = reinterpret_cast<const float*>(s_t);
  const int B = A.B;
  float acc[NBM];
#pragma unroll
  for (int b = 0; b < NBM; ++b) {
    acc[b] = 0.0f;
    if (b < B) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = q * 64 + lane;  // float4 index of element q*256 + 4*lane
        const float4 av = s_t[b * (kTower / 4) + e];
        const float4 bv = s_t[(B + b) * (kTower / 4) + e];
        const float4 cv = s_t[(2 * B + b) * (kTower / 4) + e];
#pragma unroll
        for (int s = 0; s < 9; ++s) acc[b] += dot4(w[q][s], seg_value(s, av, bv, cv));
      }
    }
  }
#pragma unroll
  for (int b = 0; b < NBM; ++b) {
    if (b < B) {
      const float v = wave_sum64(acc[b]);
      if (lane == 0) {
        const float resid = st[b * kTower + n] + st[(B + b) * kTower + n] + st[(2 * B + b) * kTower + n];
        A.out[(size_t)b * kTower + n] = v + cI + resid;
      }
    }
  }
}

// ----------------------------------------------------------- gated FFN
struct GateUpArgs {
  const float* gamma;  // [T]
  const float* Wg;     // [F][T]
  const float* Wu;     // [F][T]
  const float* u;      // [B][T]
  float* hdn;          // [B][F]
  int B;
};

// One wave per R (gate, up) row pairs, K = T = 1024 (4 float4 per lane).
// grid (F / (4R))
template <int R, int NBM>
__global__ void __launch_bounds__(kThreads) k_gateup(GateUpArgs A) {
  constexpr int KI = kTower / 256;
  __shared__ float4 s_u[NBM * kTower / 4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = (blockIdx.x * kWaves + wave) * R;
  float4 wg[R][KI], wu[R][KI], g[KI];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      wg[r][i] = ld4(A.Wg + (size_t)(n0 + r) * kTower + 256 * i + lane * 4);
      wu[r][i] = ld4(A.Wu + (size_t)(n0 + r) * kTower + 256 * i + lane * 4);
    }
#pragma unroll
  for (int i = 0; i < KI; ++i) g[i] = ld4(A.gamma + 256 * i + lane * 4);
  stage_lds<(NBM * kTower / 4 + kThreads - 1) / kThreads>(A.u, A.B * kTower / 4, s_u);
  stage_wait();
  float ag[R][NBM], au[R][NBM], ss[NBM];
#pragma unroll
  for (int b = 0; b < NBM; ++b) {
    ss[b] = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) ag[r][b] = au[r][b] = 0.0f;
    if (b < A.B) {
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        const float4 xv = s_u[b * (kTower / 4) + 64 * i + lane];
        const float4 in = mul4(xv, g[i]);
        ss[b] += dot4(xv, xv);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          ag[r][b] += dot4(wg[r][i], in);
          au[r][b] += dot4(wu[r][i], in);
        }
      }
    }
  }
#pragma unroll
  for (int b = 0; b < NBM; ++b) {
    if (b < A.B) {
      const float inv = rsqrtf(wave_sum64(ss[b]) / (float)kTower + kEps);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float gv = wave_sum64(ag[r][b]) * inv;
        const float uv = wave_sum64(au[r][b]) * inv;
        if (lane == 0) A.hdn[(size_t)b * kFfn + n0 + r] = silu(gv) * uv;
      }
    }
  }
}

struct DownArgs {
  const float* Wd;   // [T][F]
  const float* hdn;  // [B][F]
  const float* u;    // [B][T] residual input
  float* out;        // [B][T]
  int B;
};

// One wave per output row, K = F = 2048 (8 float4 per lane).  grid (T / 4)
template <int NBM>
__global__ void __launch_bounds__(kThreads) k_down(DownArgs A) {
  constexpr int KI = kFfn / 256;
  __shared__ float4 s_h[NBM * kFfn / 4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = blockIdx.x * kWaves + wave;
  float4 w[KI];
#pragma unroll
  for (int i = 0; i < KI; ++i) w[i] = ld4(A.Wd + (size_t)n * kFfn + 256 * i + lane * 4);
  // residual inputs of this row, one per batch row (lane b)
  const float resid = lane < A.B ? A.u[(size_t)lane * kTower + n] : 0.0f;
  stage_lds<(NBM * kFfn / 4 + kThreads - 1) / kThreads>(A.hdn, A.B * kFfn / 4, s_h);
  stage_wait();
  float acc[NBM];
#pragma unroll
  for (int b = 0; b < NBM; ++b) {
    acc[b] = 0.0f;
    if (b < A.B) {
#pragma unroll
      for (int i = 0; i < KI; ++i) acc[b] += dot4(w[i], s_h[b * (kFfn / 4) + 64 * i + lane]);
    }
  }
#pragma unroll
  for (int b = 0; b < NBM; ++b) {
    if (b < A.B) {
      const float v = wave_sum64(acc[b]);
      const float r = __shfl(resid, b, 64);
      if (lane == 0) A.out[(size_t)b * kTower + n] = r + v;
    }
  }
}

// --------------------------------------------------- output, rule, work list
struct OutArgs {
  const float* gamma;  // [T]
  const float* w;      // [T]
  const float* c;      // [1]
  const float* u;      // [B][T]
  float theta;
  const int8_t* force;
  const int32_t* pos;
  float* score;
  uint8_t* flag;
  int32_t* worklist;  // count, items
  int B, Hkv;
};

// The rule wave's per-sequence values are exchanged through LDS: lane
// b < kMaxBatch writes its entry, then every lane reads the whole table with
// wave-uniform addresses (broadcast reads, issued back to back), so each
// reduction costs one LDS round trip instead of a chain of cross-lane
// shuffles.  Lanes of one wave run their LDS accesses in order; the
// wavefront-scope fence keeps the compiler from moving the reads above the
// writes.
struct RuleLds {
  int t[kMaxBatch];    // t = pos + 1 of a flagged sequence, else 0
  int4 p[kMaxBatch];   // (na, nb, ua, ub): both candidate cuts and their unit lengths
  int2 w[kMaxBatch];   // (nsplit, unit length) of the chosen cut, 0 when unflagged
};
__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

// Lane b < B of one wave (B <= 32) holds sequence b's flag f and position:
// its split count under the policy stated in oda.h, which depends on every
// flagged lane (their number, their keys together, and the cost of the two
// candidate cuts summed or maximised over the batch).  Integer sums, maxima
// and minima: the same in any order.
__device__ __forceinline__ int split_count(bool f, int pos, int lane, int B, int hkv, RuleLds* L) {
  const bool on = f && lane < B;
  const int nflag = __popcll(__ballot(on));
  const int t = pos + 1;
  if (lane < kMaxBatch) L->t[lane] = on ? t : 0;
  wave_lds_fence();
  int64_t total = 0;
#pragma unroll
  for (int o = 0; o < kMaxBatch; o += 4) {
    const int4 v = *reinterpret_cast<const int4*>(&L->t[o]);
    total += (int64_t)v.x + v.y + v.z + v.w;
  }
  const int na = on ? full_nsplit_round(t, nflag, hkv, total) : 0;
  const int nb = on ? full_nsplit_rounds(t, hkv, total) : 0;
  const int ua = na > 0 ? (t + na - 1) / na : 0;
  const int ub = nb > 0 ? (t + nb - 1) / nb : 0;
  if (lane < kMaxBatch) L->p[lane] = make_int4(na, nb, ua, ub);
  wave_lds_fence();
  int4 tab[kMaxBatch];
#pragma unroll
  for (int o = 0; o < kMaxBatch; ++o) tab[o] = L->p[o];  // all reads in flight together
  int sa = 0, sb = 0;  // at most 32 x 32 splits
  int long_a = 0, long_b = 0, short_a = 0x7FFFFFFF, short_b = 0x7FFFFFFF;
#pragma unroll
  for (int o = 0; o < kMaxBatch; ++o) {
    const int4 v = tab[o];
    sa += v.x;
    sb += v.y;
    long_a = max(long_a, v.z);
    long_b = max(long_b, v.w);
    // a flagged entry has both counts >= 1; unflagged entries hold zeros
    short_a = min(short_a, v.x > 0 ? v.z : 0x7FFFFFFF);
    short_b = min(short_b, v.y > 0 ? v.w : 0x7FFFFFFF);
  }
  const int64_t cost_a = full_split_cost((int64_t)sa * hkv, long_a, short_a, total, hkv);
  const int64_t cost_b = full_split_cost((int64_t)sb * hkv, long_b, short_b, total, hkv);
  return cost_b < cost_a ? nb : na;
}

// The compacted work list in the policy's order: flagged sequences by
// descending unit length ceil(t / nsplit) (ties by ascending b), each with
// its items (b << 20) | (nsplit << 10) | split for split = 0 .. nsplit-1.
// Lanes < B of one wave (B <= 32) hold cnt = nsplit (0 when unflagged) and
// t = pos + 1.  A flagged lane's items start after those of every flagged
// sequence ordered before it, so each lane sums those counts over the
// broadcast table and writes its items there; lane 0 writes the total.
__device__ __forceinline__ void write_worklist(int cnt, int t, int lane, int B, RuleLds* L, int32_t* worklist) {
  const int unit = cnt > 0 ? (t + cnt - 1) / cnt : 0;
  if (lane < kMaxBatch) L->w[lane] = make_int2(lane < B ? cnt : 0, unit);
  wave_lds_fence();
  int2 tab[kMaxBatch];
#pragma unroll
  for (int o = 0; o < kMaxBatch; o += 2) {  // all reads in flight together
    const int4 v = *reinterpret_cast<const int4*>(&L->w[o]);
    tab[o] = make_int2(v.x, v.y);
    tab[o + 1] = make_int2(v.z, v.w);
  }
  int start = 0, total = 0;
#pragma unroll
  for (int o = 0; o < kMaxBatch; ++o) {
    const int c = tab[o].x, u = tab[o].y;  // (nsplit, unit length) of sequence o
    const bool before = c > 0 && (u > unit || (u == unit && o < lane));
    total += c;
    start += before ? c : 0;
  }
  if (lane == 0) worklist[0] = total;
  if (lane < B && cnt > 0) {
    for (int s = 0; s < cnt; ++s) worklist[1 + start + s] = full_item(lane, cnt, s);
  }
}

// One block: wave w scores sequences w, w+4, ...; wave 0 then applies the
// rule and writes the compacted work list (exclusive scan of flag * nsplit).
__global__ void __launch_bounds__(kThreads) k_out_rule(OutArgs A) {
  __shared__ float s_q[kMaxBatch];
  __shared__ RuleLds s_rule;
  __shared__ float4 s_u[kMaxBatch * kTower / 4];
  constexpr int KI = kTower / 256;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int B = A.B;
  float4 wg[KI];
#pragma unroll
  for (int i = 0; i < KI; ++i) wg[i] = mul4(ld4(A.w + 256 * i + lane * 4), ld4(A.gamma + 256 * i + lane * 4));
  const float c = A.c[0];
  // the rule's operands, loaded before the scores exist (wave 0, lane b)
  const int fo = wave == 0 && lane < B && A.force != nullptr ? (int)A.force[lane] : -1;
  const int pos = wave == 0 && lane < B ? A.pos[lane] : 0;
  stage_lds<(kMaxBatch * kTower / 4 + kThreads - 1) / kThreads>(A.u, B * kTower / 4, s_u);
  stage_wait();
  for (int b = wave; b < B; b += kWaves) {
    float d = 0.0f, ss = 0.0f;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const float4 x = s_u[b * (kTower / 4) + 64 * i + lane];
      d += dot4(wg[i], x);
      ss += dot4(x, x);
    }
    d = wave_sum64(d);
    ss = wave_sum64(ss);
    if (lane == 0) s_q[b] = d * rsqrtf(ss / (float)kTower + kEps) + c;
  }
  __syncthreads();
  if (wave != 0) return;
  int f = 0;
  if (lane < B) {
    const float q = s_q[lane];
    A.score[lane] = q;
    f = fo >= 0 ? (fo != 0) : ((q > A.theta) || !isfinite(q));
    A.flag[lane] = (uint8_t)f;
  }
  const int cnt = split_count(f != 0, pos, lane, B, A.Hkv, &s_rule);
  write_worklist(cnt, pos + 1, lane, B, &s_rule, A.worklist);
}

__global__ void __launch_bounds__(64) k_worklist(const uint8_t* flag, const int32_t* pos, int32_t* worklist, int B,
                                                 int hkv) {
  __shared__ RuleLds s_rule;
  const int lane = threadIdx.x;
  const bool f = lane < B && flag[lane] != 0;
  const int p = lane < B ? pos[lane] : 0;
  const int cnt = split_count(f, p, lane, B, hkv, &s_rule);
  write_worklist(cnt, p + 1, lane, B, &s_rule, worklist);
}

// ------------------------------------------------ dense batches: fp32 MFMA
// From five sequences on, the same layers run faster as skinny GEMMs on the
// matrix cores: Y[n][col] = sum_k W[n][k] X[col][k] with
// v_mfma_f32_16x16x4f32, A = 16 weight rows x 4 k, B = 4 k x 16 batch
// columns.  In lane l = 16q + i the instruction takes A[i][q] and B[q][i] and
// returns D[4q + r][i] in accumulator component r.
//
// A workgroup owns TW row tiles (16 rows each) and one of KSPLIT slices of K;
// each of its NW waves takes JB blocks of 16 k: lane (i, q) loads the float4
// at k_j + 4q of weight row i of every tile and of batch column i, so one
// load instruction reads 64 contiguous bytes of 16 rows, and sub-step (j, c)
// pairs component c of the lane's j-th float4 on both operands (any fixed
// pairing of k between A and B gives the same sum).  In the dense layers the
// blocks are 4 consecutive ones (k_j = k0 + 16j); in the interaction they are
// the 9 segments at one position (k_j = 1024 j + p), so a lane reads a, b and
// c once and forms all nine segment values from them.  Every operand is
// consumed straight from the load: the RMSNorm gain is applied to X as it
// arrives and the sum of squares is gathered from the same registers (the
// 1/rms scale is applied to the finished dot product).
// The waves of a workgroup are summed through LDS, the KSPLIT workgroups of a
// row block through coherent partial tiles: the last to take the row block's
// ticket adds them in split order (deterministic) and applies the layer's
// epilogue.
using f4v = __attribute__((ext_vector_type(4))) float;

enum DenseMode { kTowerMode = 0, kInterMode = 1, kGateUpMode = 2, kDownMode = 3 };

struct DenseArgs {
  const float* W[3];      // weights [N][K]: one per tower; gate, up for the FFN
  const float* gamma[3];  // RMSNorm gains [K]
  const float* bias[3];   // [N]
  const uint16_t* xb[3];  // bf16 tower inputs [B][K]
  const float* xf;        // fp32 input [B][K]; the towers [3][B][T] for the interaction
  const float* resid;     // [B][T] residual of the down projection
  float* out[3];          // [B][N] per tower / layer output
  float* part;
  int32_t* tickets;
  int B;
};

__device__ __forceinline__ void part_put(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float part_get(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float comp(const float4 v, int c) {
  return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
}
__device__ __forceinline__ float f4v_comp(const f4v v, int r) { return v[r]; }
__device__ __forceinline__ float4 as_f4(const uint4 u) {
  return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
}

template <int TW, int NG>
constexpr int dense_part_stride() {
  return TW * NG * 4 * 64 + 64;  // accumulator tile, then one sum of squares per column
}

template <int MODE>
constexpr int dense_jb() {
  return MODE == kInterMode ? 9 : 4;
}

template <int MODE, int K, int TW, int NW, int NG, int KSPLIT>
__global__ void __launch_bounds__(NW * 64) k_dense(DenseArgs A) {
  constexpr int JB = dense_jb<MODE>();    // 16-k blocks per wave
  static_assert(K == KSPLIT * NW * JB * 16, "K slices");
  constexpr int NT = NW * 64;
  constexpr int NV = TW * NG * 4;         // accumulator floats per lane
  constexpr int PMAIN = NV * 64;
  constexpr int PSZ = dense_part_stride<TW, NG>();
  constexpr bool kNorm = MODE == kTowerMode || MODE == kGateUpMode;
  constexpr int HALF = TW / 2;            // gate tiles of the FFN pairs
  constexpr int ROWS = MODE == kGateUpMode ? HALF * 16 : TW * 16;
  constexpr int VPR = NV < 128 / NW ? NV : 128 / NW;  // values per LDS round (32 KB)
  __shared__ float red[NW * VPR * 64];
  __shared__ float s_inv[32];
  __shared__ int s_last;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, lq = lane >> 4;
  const int rb = blockIdx.x, ks = blockIdx.y, z = blockIdx.z;
  const int B = A.B;
  // k of this lane's float4 in block j: k0 + kstep * j
  constexpr int kstep = MODE == kInterMode ? kTower : 16;
  const int k0 = (MODE == kInterMode ? (ks * NW + wave) * 16 : (ks * NW + wave) * 64) + 4 * lq;

  // Batch columns past B repeat column B-1: a column of B only reaches the
  // same column of the result, and those outputs are never written.
  // Loads go out first (batch operands from L2, then every weight load from
  // HBM), the scheduler is fenced so none of them slides behind arithmetic,
  // and the operand transforms wait only for the batch loads.
  constexpr int XR = MODE == kInterMode ? 3 : 4;  // loads per column group
  uint4 xr[NG][XR];
  float4 g[4];
  if (kNorm) {
#pragma unroll
    for (int j = 0; j < 4; ++j) g[j] = ld4(A.gamma[z] + k0 + 16 * j);
  }
#pragma unroll
  for (int cg = 0; cg < NG; ++cg) {
    const int col = min(16 * cg + li, B - 1);
    if (MODE == kTowerMode) {
      const uint16_t* xp = A.xb[z] + (size_t)col * K + k0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint2 v = *reinterpret_cast<const uint2*>(xp + 16 * j);
        xr[cg][j] = make_uint4(v.x, v.y, 0u, 0u);
      }
    } else if (MODE == kInterMode) {
      const float* ta = A.xf + (size_t)col * kTower + k0;
#pragma unroll
      for (int tw = 0; tw < 3; ++tw) xr[cg][tw] = *reinterpret_cast<const uint4*>(ta + (size_t)tw * B * kTower);
    } else {
      const float* xp = A.xf + (size_t)col * K + k0;
#pragma unroll
      for (int j = 0; j < 4; ++j) xr[cg][j] = *reinterpret_cast<const uint4*>(xp + 16 * j);
    }
  }
  float4 w[TW][JB];
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    const float* Wt;
    int row;
    if (MODE == kGateUpMode) {
      Wt = A.W[t < HALF ? 0 : 1];
      row = rb * ROWS + 16 * (t < HALF ? t : t - HALF) + li;
    } else {
      Wt = A.W[z];
      row = rb * ROWS + 16 * t + li;
    }
    const float* wp = Wt + (size_t)row * K + k0;
#pragma unroll
    for (int j = 0; j < JB; ++j) w[t][j] = ld4(wp + kstep * j);
  }
  __builtin_amdgcn_sched_barrier(0);

  float4 x[NG][JB];
  float ss[NG];
#pragma unroll
  for (int cg = 0; cg < NG; ++cg) {
    if (MODE == kTowerMode) {
#pragma unroll
      for (int j = 0; j < JB; ++j)
        x[cg][j] = make_float4(bf16lo(xr[cg][j].x), bf16hi(xr[cg][j].x), bf16lo(xr[cg][j].y), bf16hi(xr[cg][j].y));
    } else if (MODE == kInterMode) {
      // [a, b, c, ab, ac, bc, |a-b|, |a-c|, |b-c|]
      const float4 a = as_f4(xr[cg][0]), b = as_f4(xr[cg][1]), c = as_f4(xr[cg][2]);
#pragma unroll
      for (int j = 0; j < JB; ++j) x[cg][j] = seg_value(j, a, b, c);
    } else {
#pragma unroll
      for (int j = 0; j < JB; ++j) x[cg][j] = as_f4(xr[cg][j]);
    }
    ss[cg] = 0.0f;
    if (kNorm) {
#pragma unroll
      for (int j = 0; j < JB; ++j) {
        ss[cg] += dot4(x[cg][j], x[cg][j]);
        x[cg][j] = mul4(x[cg][j], g[j]);
      }
    }
  }

  f4v acc[TW][NG];
#pragma unroll
  for (int t = 0; t < TW; ++t)
#pragma unroll
    for (int cg = 0; cg < NG; ++cg) acc[t][cg] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < JB; ++j)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int t = 0; t < TW; ++t)
#pragma unroll
        for (int cg = 0; cg < NG; ++cg)
          acc[t][cg] = __builtin_amdgcn_mfma_f32_16x16x4f32(comp(w[t][j], c), comp(x[cg][j], c), acc[t][cg], 0, 0, 0);

  // ---- sum the waves (LDS), store this workgroup's partial tile
  const int rbg = z * gridDim.x + rb;
  float* part = A.part + ((size_t)rbg * KSPLIT + ks) * PSZ;
#pragma unroll
  for (int r0 = 0; r0 < NV; r0 += VPR) {
#pragma unroll
    for (int v = 0; v < VPR; ++v) {
      const int vv = r0 + v;
      red[(wave * VPR + v) * 64 + lane] = f4v_comp(acc[vv / (NG * 4)][(vv / 4) % NG], vv % 4);
    }
    __syncthreads();
    for (int i = tid; i < VPR * 64; i += NT) {
      float sum = 0.0f;
#pragma unroll
      for (int wv = 0; wv < NW; ++wv) sum += red[wv * VPR * 64 + i];
      part_put(part + r0 * 64 + i, sum);
    }
    __syncthreads();
  }
  if (kNorm) {
#pragma unroll
    for (int cg = 0; cg < NG; ++cg) red[(wave * NG + cg) * 64 + lane] = ss[cg];
    __syncthreads();
    if (tid < NG * 16) {
      const int cg = tid >> 4, i = tid & 15;
      float sum = 0.0f;
      for (int wv = 0; wv < NW; ++wv)
#pragma unroll
        for (int q = 0; q < 4; ++q) sum += red[(wv * NG + cg) * 64 + 16 * q + i];
      part_put(part + PMAIN + tid, sum);
    }
  }

  // ---- hand-off: the last workgroup of the row block finishes it.  The
  // partial tiles were stored with agent-scope atomic stores, which gfx950
  // issues with the device-scope cache policy (coherent across the XCDs);
  // s_waitcnt vmcnt(0) waits for their acknowledgement (gfx9 counts stores in
  // vmcnt), the barrier makes that hold for every wave, and only then is the
  // returning agent-scope ticket taken.  The workgroup that completes the set
  // uses the returned value before it issues its agent-scope partial loads,
  // so every earlier workgroup's acknowledged stores precede them.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(A.tickets + rbg, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == KSPLIT - 1;
  __syncthreads();
  if (!s_last) return;

  const float* pb = A.part + (size_t)rbg * KSPLIT * PSZ;
  constexpr int NOUT = MODE == kGateUpMode ? PMAIN / 2 : PMAIN;
  static_assert(NOUT % NT == 0, "outputs per thread");
  constexpr int NO = NOUT / NT;
  constexpr int NSUM = MODE == kGateUpMode ? 2 : 1;
  // every partial this thread needs (sums of squares included) in one batch
  // of loads, then added in split order
  float sq[KSPLIT];
  if (kNorm && tid < NG * 16) {
#pragma unroll
    for (int sp = 0; sp < KSPLIT; ++sp) sq[sp] = part_get(pb + (size_t)sp * PSZ + PMAIN + tid);
  }
  float pv[NO][NSUM][KSPLIT];
#pragma unroll
  for (int o = 0; o < NO; ++o)
#pragma unroll
    for (int h = 0; h < NSUM; ++h)
#pragma unroll
      for (int sp = 0; sp < KSPLIT; ++sp)
        pv[o][h][sp] = part_get(pb + (size_t)sp * PSZ + h * (PMAIN / 2) + tid + o * NT);
  // the epilogue's bias and residual operands, in the same batch of loads
  float ea[NO], eb[NO], ec[NO], ed[NO];
#pragma unroll
  for (int o = 0; o < NO; ++o) {
    const int i = tid + o * NT;
    const int v = i >> 6, l = i & 63;
    const int t = v / (NG * 4), cg = (v >> 2) % NG, r = v & 3;
    const int col = 16 * cg + (l & 15);
    const int n = rb * ROWS + 16 * t + 4 * (l >> 4) + r;
    ea[o] = eb[o] = ec[o] = ed[o] = 0.0f;
    if (col < B) {
      if (MODE == kTowerMode) {
        ea[o] = A.bias[z][n];
      } else if (MODE == kInterMode) {
        const float* ta = A.xf + (size_t)col * kTower + n;
        ea[o] = ta[0];
        eb[o] = ta[(size_t)B * kTower];
        ec[o] = ta[(size_t)2 * B * kTower];
        ed[o] = A.bias[0][n];
      } else if (MODE == kDownMode) {
        ea[o] = A.resid[(size_t)col * kTower + n];
      }
    }
  }
  if (kNorm) {
    if (tid < NG * 16) {
      float sum = 0.0f;
#pragma unroll
      for (int sp = 0; sp < KSPLIT; ++sp) sum += sq[sp];
      s_inv[tid] = rsqrtf(sum / (float)K + kEps);
    }
    __syncthreads();
  }
#pragma unroll
  for (int o = 0; o < NO; ++o) {
    const int i = tid + o * NT;
    const int v = i >> 6, l = i & 63;
    const int t = v / (NG * 4), cg = (v >> 2) % NG, r = v & 3;
    const int col = 16 * cg + (l & 15);
    const int n = rb * ROWS + 16 * t + 4 * (l >> 4) + r;
    float y = 0.0f;
#pragma unroll
    for (int sp = 0; sp < KSPLIT; ++sp) y += pv[o][0][sp];
    if (col >= B) continue;
    if (MODE == kTowerMode) {
      A.out[z][(size_t)col * kTower + n] = silu(y * s_inv[col] + ea[o]);
    } else if (MODE == kInterMode) {
      A.out[0][(size_t)col * kTower + n] = y + ed[o] + (ea[o] + eb[o] + ec[o]);
    } else if (MODE == kGateUpMode) {
      float yu = 0.0f;
#pragma unroll
      for (int sp = 0; sp < KSPLIT; ++sp) yu += pv[o][NSUM - 1][sp];
      const float inv = s_inv[col];
      A.out[0][(size_t)col * kFfn + n] = silu(y * inv) * (yu * inv);
    } else {
      A.out[0][(size_t)col * kTower + n] = ea[o] + y;
    }
  }
  if (tid == 0) __hip_atomic_store(A.tickets + rbg, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Shapes of the dense layers: tiles per wave, waves per workgroup, K slices.
// K = KSPLIT * NW * 64 (the interaction: KSPLIT * NW * 16 positions of its 9
// segments); each keeps a few hundred workgroups in flight.
struct DenseShape {
  int tw, nw, ksplit, rowblocks, z;
};
DenseShape tower_shape(int D) {
  return D == 4096 ? DenseShape{4, 8, 8, kTower / 64, 3} : D == 2048 ? DenseShape{4, 4, 8, kTower / 64, 3}
                                                                     : DenseShape{4, 4, 4, kTower / 64, 3};
}
constexpr DenseShape kInterShape{2, 8, 8, kTower / 32, 1};
constexpr DenseShape kGateUpShape{4, 4, 4, kFfn / 32, 1};
constexpr DenseShape kDownShape{2, 4, 8, kTower / 32, 1};

size_t shape_part_floats(const DenseShape& s, int ng) {
  return (size_t)s.z * s.rowblocks * s.ksplit * (s.tw * ng * 4 * 64 + 64);
}

template <int NG>
int launch_dense_t(const HeadParams& p, const int64_t* offs, hipStream_t s) {
  const int B = p.B;
  const dim3 blk256(256), blk512(512);
  DenseArgs ta{};
  for (int t = 0; t < 3; ++t) {
    ta.gamma[t] = p.w + offs[3 * t + 0];
    ta.W[t] = p.w + offs[3 * t + 1];
    ta.bias[t] = p.w + offs[3 * t + 2];
    ta.out[t] = p.act.towers + (size_t)t * B * kTower;
  }
  ta.xb[0] = p.h_prev;
  ta.xb[1] = p.emb;
  ta.xb[2] = p.h_local;
  ta.part = p.act.part;
  ta.tickets = p.tickets;
  ta.B = B;
  const DenseShape ts = tower_shape(p.D);
  const dim3 tgrid(ts.rowblocks, ts.ksplit, 3);
  switch (p.D) {
    case 1024: hipLaunchKernelGGL((k_dense<kTowerMode, 1024, 4, 4, NG, 4>), tgrid, blk256, 0, s, ta); break;
    case 2048: hipLaunchKernelGGL((k_dense<kTowerMode, 2048, 4, 4, NG, 8>), tgrid, blk256, 0, s, ta); break;
    case 4096: hipLaunchKernelGGL((k_dense<kTowerMode, 4096, 4, 8, NG, 8>), tgrid, blk512, 0, s, ta); break;
    default: return ODA_E_UNSUPPORTED;
  }

  DenseArgs ia{};
  ia.W[0] = p.w + offs[9];
  ia.bias[0] = p.w + offs[10];
  ia.xf = p.act.towers;
  ia.out[0] = p.act.u0;
  ia.part = p.act.part;
  ia.tickets = p.tickets;
  ia.B = B;
  hipLaunchKernelGGL((k_dense<kInterMode, 9 * kTower, 2, 8, NG, 8>),
                     dim3(kInterShape.rowblocks, kInterShape.ksplit), blk512, 0, s, ia);

  const float* u_in = p.act.u0;
  float* u_out[2] = {p.act.u1, p.act.u2};
  for (int b = 0; b < 2; ++b) {
    const int base = 11 + 4 * b;
    DenseArgs ga{};
    ga.gamma[0] = p.w + offs[base + 0];
    ga.W[0] = p.w + offs[base + 1];
    ga.W[1] = p.w + offs[base + 2];
    ga.xf = u_in;
    ga.out[0] = p.act.hdn;
    ga.part = p.act.part;
    ga.tickets = p.tickets;
    ga.B = B;
    hipLaunchKernelGGL((k_dense<kGateUpMode, kTower, 4, 4, NG, 4>),
                       dim3(kGateUpShape.rowblocks, kGateUpShape.ksplit), blk256, 0, s, ga);
    DenseArgs da{};
    da.W[0] = p.w + offs[base + 3];
    da.xf = p.act.hdn;
    da.resid = u_in;
    da.out[0] = u_out[b];
    da.part = p.act.part;
    da.tickets = p.tickets;
    da.B = B;
    hipLaunchKernelGGL((k_dense<kDownMode, kFfn, 2, 4, NG, 8>), dim3(kDownShape.rowblocks, kDownShape.ksplit),
                       blk256, 0, s, da);
    u_in = u_out[b];
  }

  OutArgs oa;
  oa.gamma = p.w + offs[19];
  oa.w = p.w + offs[20];
  oa.c = p.w + offs[21];
  oa.u = u_in;
  oa.theta = p.theta;
  oa.force = p.force;
  oa.pos = p.pos;
  oa.score = p.score;
  oa.flag = p.flag;
  oa.worklist = p.worklist;
  oa.B = B;
  oa.Hkv = p.Hkv;
  hipLaunchKernelGGL(k_out_rule, dim3(1), dim3(kThreads), 0, s, oa);
  return hipGetLastError() == hipSuccess ? ODA_OK : ODA_E_LAUNCH;
}

int nbm_of(int B) { return B > 16 ? 32 : B > 8 ? 16 : B > 4 ? 8 : B > 2 ? 4 : B > 1 ? 2 : 1; }

template <int NBM>
int launch_head_t(const HeadParams& p, const int64_t* offs, hipStream_t s) {
  const int B = p.B;
#ifndef ODA_TOWER_ROWS
#define ODA_TOWER_ROWS 1
#endif
  constexpr int R = NBM <= 8 ? ODA_TOWER_ROWS : 1;  // rows per wave: fewer when many batch accumulators are live
  TowerArgs ta;
  ta.w = p.w;
  for (int t = 0; t < 3; ++t) {
    ta.off_gamma[t] = offs[3 * t + 0];
    ta.off_W[t] = offs[3 * t + 1];
    ta.off_c[t] = offs[3 * t + 2];
  }
  ta.x[0] = p.h_prev;
  ta.x[1] = p.emb;
  ta.x[2] = p.h_local;
  ta.out = p.act.towers;
  ta.B = B;
  const dim3 tgrid(kTower / (kWaves * R), 3);
  switch (p.D) {
    case 1024: hipLaunchKernelGGL((k_tower<4, R, NBM>), tgrid, dim3(kThreads), 0, s, ta); break;
    case 2048: hipLaunchKernelGGL((k_tower<8, R, NBM>), tgrid, dim3(kThreads), 0, s, ta); break;
    case 4096: hipLaunchKernelGGL((k_tower<16, 1, NBM>), dim3(kTower / kWaves, 3), dim3(kThreads), 0, s, ta); break;
    default: return ODA_E_UNSUPPORTED;
  }

  InteractArgs ia;
  ia.W = p.w + offs[9];
  ia.bias = p.w + offs[10];
  ia.towers = p.act.towers;
  ia.out = p.act.u0;
  ia.B = B;
  hipLaunchKernelGGL(k_interact<NBM>, dim3(kTower / kWaves), dim3(kThreads), 0, s, ia);

  const float* u_in = p.act.u0;
  float* u_out[2] = {p.act.u1, p.act.u2};
  for (int blk = 0; blk < 2; ++blk) {
    const int base = 11 + 4 * blk;
    GateUpArgs ga;
    ga.gamma = p.w + offs[base + 0];
    ga.Wg = p.w + offs[base + 1];
    ga.Wu = p.w + offs[base + 2];
    ga.u = u_in;
    ga.hdn = p.act.hdn;
    ga.B = B;
    hipLaunchKernelGGL((k_gateup<R, NBM>), dim3(kFfn / (kWaves * R)), dim3(kThreads), 0, s, ga);
    DownArgs da;
    da.Wd = p.w + offs[base + 3];
    da.hdn = p.act.hdn;
    da.u = u_in;
    da.out = u_out[blk];
    da.B = B;
    hipLaunchKernelGGL(k_down<NBM>, dim3(kTower / kWaves), dim3(kThreads), 0, s, da);
    u_in = u_out[blk];
  }

  OutArgs oa;
  oa.gamma = p.w + offs[19];
  oa.w = p.w + offs[20];
  oa.c = p.w + offs[21];
  oa.u = u_in;
  oa.theta = p.theta;
  oa.force = p.force;
  oa.pos = p.pos;
  oa.score = p.score;
  oa.flag = p.flag;
  oa.worklist = p.worklist;
  oa.B = B;
  oa.Hkv = p.Hkv;
  hipLaunchKernelGGL(k_out_rule, dim3(1), dim3(kThreads), 0, s, oa);
  return hipGetLastError() == hipSuccess ? ODA_OK : ODA_E_LAUNCH;
}

}  // namespace

size_t dense_head_part_floats(int B, int D) {
  const int ng = B > 16 ? 2 : 1;
  size_t m = shape_part_floats(tower_shape(D), ng);
  const DenseShape others[3] = {kInterShape, kGateUpShape, kDownShape};
  for (const DenseShape& s : others) {
    const size_t n = shape_part_floats(s, ng);
    if (n > m) m = n;
  }
  return m;
}

// offs: host array of the ODA_HEAD_NTENSORS+1 tensor offsets (oda_head_offsets order)
int launch_worklist(const uint8_t* flag, const int32_t* pos, int32_t* worklist, int B, int Hkv, hipStream_t s) {
  hipLaunchKernelGGL(k_worklist, dim3(1), dim3(64), 0, s, flag, pos, worklist, B, Hkv);
  return hipGetLastError() == hipSuccess ? ODA_OK : ODA_E_LAUNCH;
}

int launch_recall_head(const HeadParams& p, const int64_t* offs, hipStream_t s) {
  if (p.B >= kHeadDenseMin) return p.B > 16 ? launch_dense_t<2>(p, offs, s) : launch_dense_t<1>(p, offs, s);
  switch (nbm_of(p.B)) {
    case 1: return launch_head_t<1>(p, offs, s);
    case 2: return launch_head_t<2>(p, offs, s);
    case 4: return launch_head_t<4>(p, offs, s);
    default: return launch_head_t<8>(p, offs, s);
  }
}

}  // namespace oda
