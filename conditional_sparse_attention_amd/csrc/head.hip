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
// The dot products are reduced inside the wave (DPP row sums + readlane),
// with no LDS and no barrier.  RMSNorm scales are folded in after the dot
// product (W (gamma*x) / rms(x)), the sum of squares gathered in the same
// pass; the interaction vector is formed on the fly from the tower outputs.
#include "oda_internal.h"

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
  float acc[R][NBM], ss[NBM];
  const uint16_t* x = A.x[tw] + lane * 4;
#pragma unroll
  for (int b = 0; b < NBM; ++b) {
    ss[b] = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r][b] = 0.0f;
    if (b < A.B) {
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        const float4 xv = ldbf4(x + (size_t)b * D + 256 * i);
        const float4 in = mul4(xv, g[i]);
        ss[b] += dot4(xv, xv);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][b] += dot4(w[r][i], in);
      }
    }
  }
  const float* cb = A.w + A.off_c[tw] + n0;
#pragma unroll
  for (int b = 0; b < NBM; ++b) {
    if (b < A.B) {
      const float inv = rsqrtf(wave_sum64(ss[b]) / (float)D + kEps);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float v = wave_sum64(acc[r][b]);
        if (lane == 0) A.out[((size_t)tw * A.B + b) * kTower + n0 + r] = silu(v * inv + cb[r]);
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
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = blockIdx.x * kWaves + wave;
  const float* W = A.W + (size_t)n * (9 * kTower) + lane * 4;
  float4 w[4][9];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int s = 0; s < 9; ++s) w[q][s] = ld4(W + s * kTower + q * 256);
  float acc[NBM];
#pragma unroll
  for (int b = 0; b < NBM; ++b) {
    acc[b] = 0.0f;
    if (b < A.B) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = q * 256 + lane * 4;
        const float4 av = ld4(A.towers + (size_t)b * kTower + e);
        const float4 bv = ld4(A.towers + ((size_t)A.B + b) * kTower + e);
        const float4 cv = ld4(A.towers + ((size_t)2 * A.B + b) * kTower + e);
#pragma unroll
        for (int s = 0; s < 9; ++s) acc[b] += dot4(w[q][s], seg_value(s, av, bv, cv));
      }
    }
  }
  const float cI = A.bias[n];
#pragma unroll
  for (int b = 0; b < NBM; ++b) {
    if (b < A.B) {
      const float v = wave_sum64(acc[b]);
      if (lane == 0) {
        const float resid = A.towers[(size_t)b * kTower + n] + A.towers[((size_t)A.B + b) * kTower + n] +
                            A.towers[((size_t)2 * A.B + b) * kTower + n];
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
  float ag[R][NBM], au[R][NBM], ss[NBM];
#pragma unroll
  for (int b = 0; b < NBM; ++b) {
    ss[b] = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) ag[r][b] = au[r][b] = 0.0f;
    if (b < A.B) {
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        const float4 xv = ld4(A.u + (size_t)b * kTower + 256 * i + lane * 4);
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
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = blockIdx.x * kWaves + wave;
  float4 w[KI];
#pragma unroll
  for (int i = 0; i < KI; ++i) w[i] = ld4(A.Wd + (size_t)n * kFfn + 256 * i + lane * 4);
  float acc[NBM];
#pragma unroll
  for (int b = 0; b < NBM; ++b) {
    acc[b] = 0.0f;
    if (b < A.B) {
#pragma unroll
      for (int i = 0; i < KI; ++i) acc[b] += dot4(w[i], ld4(A.hdn + (size_t)b * kFfn + 256 * i + lane * 4));
    }
  }
#pragma unroll
  for (int b = 0; b < NBM; ++b) {
    if (b < A.B) {
      const float v = wave_sum64(acc[b]);
      if (lane == 0) {
        const size_t o = (size_t)b * kTower + n;
        A.out[o] = A.u[o] + v;
      }
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
  int B;
};

// Exclusive scan of the per-sequence split counts (lanes < B of one wave,
// B <= 32) and the compacted items (b << 20) | split, b ascending.
__device__ __forceinline__ void write_worklist(int cnt, int lane, int B, int* s_start, const int* s_count,
                                               int32_t* worklist) {
  int incl = cnt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  if (lane < B) s_start[lane] = incl - cnt;
  if (lane == B - 1) worklist[0] = incl;
  __builtin_amdgcn_wave_barrier();
  for (int i = lane; i < B * kFullMaxSplits; i += 64) {
    const int b = i / kFullMaxSplits, s = i % kFullMaxSplits;
    if (s < s_count[b]) worklist[1 + s_start[b] + s] = (b << 20) | s;
  }
}

// One block: wave w scores sequences w, w+4, ...; wave 0 then applies the
// rule and writes the compacted work list (exclusive scan of flag * nsplit).
__global__ void __launch_bounds__(kThreads) k_out_rule(OutArgs A) {
  __shared__ float s_q[kMaxBatch];
  __shared__ int s_start[kMaxBatch + 1];
  __shared__ int s_count[kMaxBatch];
  constexpr int KI = kTower / 256;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float4 wg[KI];
#pragma unroll
  for (int i = 0; i < KI; ++i) wg[i] = mul4(ld4(A.w + 256 * i + lane * 4), ld4(A.gamma + 256 * i + lane * 4));
  for (int b = wave; b < A.B; b += kWaves) {
    float d = 0.0f, ss = 0.0f;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const float4 x = ld4(A.u + (size_t)b * kTower + 256 * i + lane * 4);
      d += dot4(wg[i], x);
      ss += dot4(x, x);
    }
    d = wave_sum64(d);
    ss = wave_sum64(ss);
    if (lane == 0) s_q[b] = d * rsqrtf(ss / (float)kTower + kEps) + A.c[0];
  }
  __syncthreads();
  if (wave != 0) return;
  int cnt = 0;
  if (lane < A.B) {
    const float q = s_q[lane];
    A.score[lane] = q;
    const int fo = A.force != nullptr ? (int)A.force[lane] : -1;
    const int f = fo >= 0 ? (fo != 0) : ((q > A.theta) || !isfinite(q));
    A.flag[lane] = (uint8_t)f;
    cnt = f ? full_nsplit(A.pos[lane] + 1) : 0;
    s_count[lane] = cnt;
  }
  write_worklist(cnt, lane, A.B, s_start, s_count, A.worklist);
}

__global__ void __launch_bounds__(64) k_worklist(const uint8_t* flag, const int32_t* pos, int32_t* worklist, int B) {
  __shared__ int s_start[kMaxBatch + 1];
  __shared__ int s_count[kMaxBatch];
  const int lane = threadIdx.x;
  int cnt = 0;
  if (lane < B) {
    cnt = flag[lane] ? full_nsplit(pos[lane] + 1) : 0;
    s_count[lane] = cnt;
  }
  write_worklist(cnt, lane, B, s_start, s_count, worklist);
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
  hipLaunchKernelGGL(k_out_rule, dim3(1), dim3(kThreads), 0, s, oa);
  return hipGetLastError() == hipSuccess ? ODA_OK : ODA_E_LAUNCH;
}

}  // namespace

// offs: host array of the ODA_HEAD_NTENSORS+1 tensor offsets (oda_head_offsets order)
int launch_worklist(const uint8_t* flag, const int32_t* pos, int32_t* worklist, int B, hipStream_t s) {
  hipLaunchKernelGGL(k_worklist, dim3(1), dim3(64), 0, s, flag, pos, worklist, B);
  return hipGetLastError() == hipSuccess ? ODA_OK : ODA_E_LAUNCH;
}

int launch_recall_head(const HeadParams& p, const int64_t* offs, hipStream_t s) {
  switch (nbm_of(p.B)) {
    case 1: return launch_head_t<1>(p, offs, s);
    case 2: return launch_head_t<2>(p, offs, s);
    case 4: return launch_head_t<4>(p, offs, s);
    case 8: return launch_head_t<8>(p, offs, s);
    case 16: return launch_head_t<16>(p, offs, s);
    default: return launch_head_t<32>(p, offs, s);
  }
}

}  // namespace oda
