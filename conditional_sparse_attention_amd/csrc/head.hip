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
// kernels are bandwidth-shaped GEMVs: a workgroup owns 4 output rows, its
// 256 lanes walk the reduction dimension with 16-byte weight loads, every
// batch row is accumulated from the same weight registers, and RMSNorm
// scales are folded in after the dot product (W (gamma*x) / rms(x)), with
// the sum of squares gathered in the same pass.  The interaction vector is
// never materialised: each lane forms its 4 elements from the tower outputs
// on the fly.  Batches above 8 rows are processed in tiles of 8.
#include "oda_internal.h"

namespace oda {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 4;       // output rows per workgroup
constexpr int kMaxNB = 8;      // batch rows per tile
constexpr float kEps = 1e-6f;

__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// Reduce NV per-thread values over the 256-thread block; result in red[0..NV).
template <int NV>
__device__ __forceinline__ void block_sum(float (&v)[NV], float* red /* [4][NV] */) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const float s = wave_sum(v[i]);
    if (lane == 0) red[wave * NV + i] = s;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < NV; i += kThreads) {
    red[4 * NV + i] = red[i] + red[NV + i] + red[2 * NV + i] + red[3 * NV + i];
  }
  __syncthreads();
}

__device__ __forceinline__ float4 load_bf16x4(const uint16_t* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  return make_float4(bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y));
}
__device__ __forceinline__ float dot4(const float4 a, const float4 b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

struct TowerArgs {
  const float* w;      // blob
  int64_t off_gamma[3], off_W[3], off_c[3];
  const uint16_t* x[3];  // h_prev, emb, h_local  [B][D]
  float* out;            // towers [3][B][T]
  int B, D;
};

// grid (T / kRows, 3 towers, batch tiles)
template <int NB>
__global__ void __launch_bounds__(kThreads) k_tower(TowerArgs A) {
  __shared__ float red[5 * (kRows * NB + NB)];
  const int tw = blockIdx.y;
  const int n0 = blockIdx.x * kRows;
  const int b0 = blockIdx.z * kMaxNB;
  const int nb = min(NB, A.B - b0);
  const float* W = A.w + A.off_W[tw];
  const float* gamma = A.w + A.off_gamma[tw];
  const uint16_t* x = A.x[tw] + (size_t)b0 * A.D;
  float acc[kRows * NB + NB];
#pragma unroll
  for (int i = 0; i < kRows * NB + NB; ++i) acc[i] = 0.0f;
  for (int k = threadIdx.x * 4; k < A.D; k += kThreads * 4) {
    float4 w[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) w[r] = *reinterpret_cast<const float4*>(W + (size_t)(n0 + r) * A.D + k);
    const float4 gm = *reinterpret_cast<const float4*>(gamma + k);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b < nb) {
        const float4 xv = load_bf16x4(x + (size_t)b * A.D + k);
        const float4 in = make_float4(xv.x * gm.x, xv.y * gm.y, xv.z * gm.z, xv.w * gm.w);
#pragma unroll
        for (int r = 0; r < kRows; ++r) acc[r * NB + b] += dot4(w[r], in);
        acc[kRows * NB + b] += dot4(xv, xv);
      }
    }
  }
  block_sum<kRows * NB + NB>(acc, red);
  const float* tot = red + 4 * (kRows * NB + NB);
  if (threadIdx.x < kRows * NB) {
    const int r = threadIdx.x / NB, b = threadIdx.x % NB;
    if (b < nb) {
      const float inv = rsqrtf(tot[kRows * NB + b] / (float)A.D + kEps);
      const float c = A.w[A.off_c[tw] + n0 + r];
      A.out[((size_t)tw * A.B + b0 + b) * kTower + n0 + r] = silu(tot[r * NB + b] * inv + c);
    }
  }
}

struct InteractArgs {
  const float* W;      // W_I [T][9T]
  const float* bias;   // c_I
  const float* towers; // [3][B][T]
  float* out;          // u0 [B][T]
  int B;
};

__device__ __forceinline__ float4 seg_value(int seg, const float4 a, const float4 b, const float4 c) {
  switch (seg) {
    case 0: return a;
    case 1: return b;
    case 2: return c;
    case 3: return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w);
    case 4: return make_float4(a.x * c.x, a.y * c.y, a.z * c.z, a.w * c.w);
    case 5: return make_float4(b.x * c.x, b.y * c.y, b.z * c.z, b.w * c.w);
    case 6: return make_float4(fabsf(a.x - b.x), fabsf(a.y - b.y), fabsf(a.z - b.z), fabsf(a.w - b.w));
    case 7: return make_float4(fabsf(a.x - c.x), fabsf(a.y - c.y), fabsf(a.z - c.z), fabsf(a.w - c.w));
    default: return make_float4(fabsf(b.x - c.x), fabsf(b.y - c.y), fabsf(b.z - c.z), fabsf(b.w - c.w));
  }
}

// grid (T / kRows, 1, batch tiles); one loop iteration per interaction segment
template <int NB>
__global__ void __launch_bounds__(kThreads) k_interact(InteractArgs A) {
  __shared__ float red[5 * kRows * NB];
  const int n0 = blockIdx.x * kRows;
  const int b0 = blockIdx.z * kMaxNB;
  const int nb = min(NB, A.B - b0);
  const float* ta = A.towers + (size_t)b0 * kTower;
  const float* tb = A.towers + ((size_t)A.B + b0) * kTower;
  const float* tc = A.towers + ((size_t)2 * A.B + b0) * kTower;
  const int i4 = threadIdx.x * 4;  // element inside the segment (T = 1024 = 256 lanes * 4)
  float acc[kRows * NB];
#pragma unroll
  for (int i = 0; i < kRows * NB; ++i) acc[i] = 0.0f;
  float4 av[NB], bv[NB], cv[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (b < nb) {
      av[b] = *reinterpret_cast<const float4*>(ta + (size_t)b * kTower + i4);
      bv[b] = *reinterpret_cast<const float4*>(tb + (size_t)b * kTower + i4);
      cv[b] = *reinterpret_cast<const float4*>(tc + (size_t)b * kTower + i4);
    } else {
      av[b] = bv[b] = cv[b] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  for (int seg = 0; seg < 9; ++seg) {
    float4 w[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r)
      w[r] = *reinterpret_cast<const float4*>(A.W + (size_t)(n0 + r) * (9 * kTower) + seg * kTower + i4);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float4 in = seg_value(seg, av[b], bv[b], cv[b]);
#pragma unroll
      for (int r = 0; r < kRows; ++r) acc[r * NB + b] += dot4(w[r], in);
    }
  }
  block_sum<kRows * NB>(acc, red);
  const float* tot = red + 4 * kRows * NB;
  if (threadIdx.x < kRows * NB) {
    const int r = threadIdx.x / NB, b = threadIdx.x % NB;
    if (b < nb) {
      const int n = n0 + r;
      const size_t o = (size_t)(b0 + b) * kTower + n;
      const float resid = ta[(size_t)b * kTower + n] + tb[(size_t)b * kTower + n] + tc[(size_t)b * kTower + n];
      A.out[o] = tot[r * NB + b] + A.bias[n] + resid;
    }
  }
}

struct GateUpArgs {
  const float* gamma;  // [T]
  const float* Wg;     // [F][T]
  const float* Wu;     // [F][T]
  const float* u;      // [B][T]
  float* hdn;          // [B][F]
  int B;
};

// grid (F / (kRows/2), 1, batch tiles): rows n0, n0+1 of both gate and up
template <int NB>
__global__ void __launch_bounds__(kThreads) k_gateup(GateUpArgs A) {
  constexpr int NP = kRows / 2;  // (gate, up) pairs per block
  __shared__ float red[5 * (kRows * NB + NB)];
  const int n0 = blockIdx.x * NP;
  const int b0 = blockIdx.z * kMaxNB;
  const int nb = min(NB, A.B - b0);
  const float* u = A.u + (size_t)b0 * kTower;
  float acc[kRows * NB + NB];
#pragma unroll
  for (int i = 0; i < kRows * NB + NB; ++i) acc[i] = 0.0f;
  const int k = threadIdx.x * 4;  // T = 1024 = one pass
  float4 w[kRows];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    w[2 * p] = *reinterpret_cast<const float4*>(A.Wg + (size_t)(n0 + p) * kTower + k);
    w[2 * p + 1] = *reinterpret_cast<const float4*>(A.Wu + (size_t)(n0 + p) * kTower + k);
  }
  const float4 gm = *reinterpret_cast<const float4*>(A.gamma + k);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (b < nb) {
      const float4 xv = *reinterpret_cast<const float4*>(u + (size_t)b * kTower + k);
      const float4 in = make_float4(xv.x * gm.x, xv.y * gm.y, xv.z * gm.z, xv.w * gm.w);
#pragma unroll
      for (int r = 0; r < kRows; ++r) acc[r * NB + b] += dot4(w[r], in);
      acc[kRows * NB + b] += dot4(xv, xv);
    }
  }
  block_sum<kRows * NB + NB>(acc, red);
  const float* tot = red + 4 * (kRows * NB + NB);
  if (threadIdx.x < NP * NB) {
    const int p = threadIdx.x / NB, b = threadIdx.x % NB;
    if (b < nb) {
      const float inv = rsqrtf(tot[kRows * NB + b] / (float)kTower + kEps);
      const float g = tot[(2 * p) * NB + b] * inv;
      const float up = tot[(2 * p + 1) * NB + b] * inv;
      A.hdn[(size_t)(b0 + b) * kFfn + n0 + p] = silu(g) * up;
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

template <int NB>
__global__ void __launch_bounds__(kThreads) k_down(DownArgs A) {
  __shared__ float red[5 * kRows * NB];
  const int n0 = blockIdx.x * kRows;
  const int b0 = blockIdx.z * kMaxNB;
  const int nb = min(NB, A.B - b0);
  const float* h = A.hdn + (size_t)b0 * kFfn;
  float acc[kRows * NB];
#pragma unroll
  for (int i = 0; i < kRows * NB; ++i) acc[i] = 0.0f;
  for (int k = threadIdx.x * 4; k < kFfn; k += kThreads * 4) {
    float4 w[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) w[r] = *reinterpret_cast<const float4*>(A.Wd + (size_t)(n0 + r) * kFfn + k);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b < nb) {
        const float4 in = *reinterpret_cast<const float4*>(h + (size_t)b * kFfn + k);
#pragma unroll
        for (int r = 0; r < kRows; ++r) acc[r * NB + b] += dot4(w[r], in);
      }
    }
  }
  block_sum<kRows * NB>(acc, red);
  const float* tot = red + 4 * kRows * NB;
  if (threadIdx.x < kRows * NB) {
    const int r = threadIdx.x / NB, b = threadIdx.x % NB;
    if (b < nb) {
      const size_t o = (size_t)(b0 + b) * kTower + n0 + r;
      A.out[o] = A.u[o] + tot[r * NB + b];
    }
  }
}

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
  int32_t* worklist;   // count, items
  int B;
};

// One block: q for every sequence, the rule, and the work list.
__global__ void __launch_bounds__(kThreads) k_out_rule(OutArgs A) {
  __shared__ float red[5 * 2 * kMaxBatch];
  __shared__ int counts[kMaxBatch];
  __shared__ int starts[kMaxBatch + 1];
  const int k = threadIdx.x * 4;
  const float4 gm = *reinterpret_cast<const float4*>(A.gamma + k);
  const float4 wv = *reinterpret_cast<const float4*>(A.w + k);
  const float4 wg = make_float4(wv.x * gm.x, wv.y * gm.y, wv.z * gm.z, wv.w * gm.w);
  float acc[2 * kMaxBatch];
#pragma unroll
  for (int b = 0; b < kMaxBatch; ++b) {
    if (b < A.B) {
      const float4 x = *reinterpret_cast<const float4*>(A.u + (size_t)b * kTower + k);
      acc[b] = dot4(wg, x);
      acc[kMaxBatch + b] = dot4(x, x);
    } else {
      acc[b] = 0.0f;
      acc[kMaxBatch + b] = 0.0f;
    }
  }
  block_sum<2 * kMaxBatch>(acc, red);
  const float* tot = red + 4 * 2 * kMaxBatch;
  if (threadIdx.x < A.B) {
    const int b = threadIdx.x;
    const float inv = rsqrtf(tot[kMaxBatch + b] / (float)kTower + kEps);
    const float q = tot[b] * inv + A.c[0];
    A.score[b] = q;
    int f;
    const int fo = A.force != nullptr ? (int)A.force[b] : -1;
    if (fo >= 0) {
      f = fo != 0;
    } else {
      f = (q > A.theta) || !isfinite(q);
    }
    A.flag[b] = (uint8_t)f;
    counts[b] = f ? full_nsplit(A.pos[b] + 1) : 0;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int s = 0;
    for (int b = 0; b < A.B; ++b) {
      starts[b] = s;
      s += counts[b];
    }
    starts[A.B] = s;
    A.worklist[0] = s;
  }
  __syncthreads();
  // each sequence writes its own items; lanes stride over (b, split)
  for (int i = threadIdx.x; i < A.B * kFullMaxSplits; i += kThreads) {
    const int b = i / kFullMaxSplits, s = i % kFullMaxSplits;
    if (s < counts[b]) A.worklist[1 + starts[b] + s] = (b << 20) | s;
  }
}

// smallest tile width in {1, 2, 4, 8} that holds min(B, 8) rows
int nb_of(int B) { return B > 4 ? 8 : (B > 2 ? 4 : (B > 1 ? 2 : 1)); }

#define ODA_NB_DISPATCH(KERNEL, GRID, ARGS, B, S)                                         \
  do {                                                                                   \
    const int nb_ = nb_of(B);                                                            \
    if (nb_ == 8) hipLaunchKernelGGL(KERNEL<8>, GRID, dim3(kThreads), 0, S, ARGS);       \
    else if (nb_ == 4) hipLaunchKernelGGL(KERNEL<4>, GRID, dim3(kThreads), 0, S, ARGS);  \
    else if (nb_ == 2) hipLaunchKernelGGL(KERNEL<2>, GRID, dim3(kThreads), 0, S, ARGS);  \
    else hipLaunchKernelGGL(KERNEL<1>, GRID, dim3(kThreads), 0, S, ARGS);                \
  } while (0)

}  // namespace

// offs: host array of the ODA_HEAD_NTENSORS+1 tensor offsets (oda_head_offsets order)
int launch_recall_head(const HeadParams& p, const int64_t* offs, hipStream_t s) {
  const int B = p.B;
  // tiles of 8 rows; a batch of B uses ceil(B/8) tiles (kernels guard b < B)
  const int tiles = (B + kMaxNB - 1) / kMaxNB;
  const int nbB = B > kMaxNB ? kMaxNB : B;

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
  ta.D = p.D;
  ODA_NB_DISPATCH(k_tower, dim3(kTower / kRows, 3, tiles), ta, nbB, s);

  InteractArgs ia;
  ia.W = p.w + offs[9];
  ia.bias = p.w + offs[10];
  ia.towers = p.act.towers;
  ia.out = p.act.u0;
  ia.B = B;
  ODA_NB_DISPATCH(k_interact, dim3(kTower / kRows, 1, tiles), ia, nbB, s);

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
    ODA_NB_DISPATCH(k_gateup, dim3(kFfn / (kRows / 2), 1, tiles), ga, nbB, s);
    DownArgs da;
    da.Wd = p.w + offs[base + 3];
    da.hdn = p.act.hdn;
    da.u = u_in;
    da.out = u_out[blk];
    da.B = B;
    ODA_NB_DISPATCH(k_down, dim3(kTower / kRows, 1, tiles), da, nbB, s);
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

}  // namespace oda
