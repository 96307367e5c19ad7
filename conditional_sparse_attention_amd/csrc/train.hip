// One recall-head training step for gfx950: labels from the two branches'
// final hidden states through the tied LM head, then forward, Huber loss and
// backward of the fp32 recall head [On-Demand Attention notes §2.1 gain g;
// §2.2 d, y, loss, paired supervision].  oda_train.h states what is computed.
//
// Labels.  The log-sum-exp over the vocabulary of E h for 2N hidden rows is a
// dense bf16 contraction (2 N V D multiply-adds): k_lse tiles it 256 rows x
// 256 vocabulary rows per workgroup of eight waves (128 x 64 each) on
// v_mfma_f32_16x16x32_bf16 (lane 16q + i takes A[i][8q..8q+7] and
// B[8q..8q+7][i], returns D[4q + r][i]), K staged through LDS 64 at a time,
// and reduces its tile to a (max, sum of exp) pair per row, never writing
// logits.  Each XCD owns one slice of the
// vocabulary and walks it for groups of row blocks, so E streams through
// every L2 a few times and the hidden rows stay cache-resident.  k_lse_fin
// merges the pairs in tile order.
//
// Head.  Forward and backward are fp32 GEMMs over the N rows (about 6 P N
// flops for P parameters) on v_mfma_f32_16x16x4_f32 (lane 16q + i takes
// A[i][q] and B[q][i]).  One kernel, k_sgemm, serves every product: a
// 128 x 128 tile per workgroup of four waves (64 x 64 each), K staged
// through LDS 16 at a time with both operands stored k-contiguous, so that a
// lane's 16-byte LDS read holds A[i][4q..4q+3]: MFMA number j of a stage then
// sums over k = 4q + j, and the four together cover the stage's 16 k.
// Operands are row-major with either index contiguous (weights [out][in] for
// the forward and data gradients, activations [rows][features] read
// transposed for the weight gradients).  Weight gradients split K (the rows)
// over workgroups into partial tiles summed in split order.  Norms, the
// interaction, SwiGLU, the loss and their backward passes are row kernels;
// bias and gain gradients are column sums over rows in fixed order, so the
// whole step is deterministic.
#include <math.h>
#include <string.h>

#include <algorithm>

#include "oda_train.h"
#include "oda_internal.h"

namespace oda {
namespace {

using f4v = __attribute__((ext_vector_type(4))) float;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float kEps = 1e-6f;         // RMSNorm epsilon of the head
constexpr int kMaxRows = 65536;
constexpr int kXcds = 8;              // gfx950: workgroups are dealt to 8 XCDs in turn
constexpr int kColChunks = 256;       // at most this many row chunks in a column sum

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float sigm(float x) { return 1.0f / (1.0f + expf(-x)); }

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  return x;
}

// Sum over a 256-thread block in a fixed order; every thread gets the result.
__device__ __forceinline__ float block_sum256(float x, float* red) {
  x = row16_sum(x);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  x = (r0 + r1) + (r2 + r3);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

__device__ __forceinline__ void raise_err(int32_t* err, int bit) {
  if (err != nullptr) atomicOr(err, bit);
}

// ===========================================================================
// fp32 GEMM: C[M][N] = sum_k A(m, k) B(k, n)
// ===========================================================================
constexpr int kBM = 128, kBN = 128, kBK = 16, kLdk = kBK + 4;  // 80-byte LDS rows: conflict-free b128 reads

enum Epi { kStore = 0, kBiasSilu = 1, kAdd = 2 };

struct Sg {
  const float* A;       // A(m, k) = A[m * lda + k] (AK) or A[k * lda + m]
  const float* B;       // B(k, n) = B[n * ldb + k] (BK) or B[k * ldb + n]
  float* C;             // C[m * ldc + n]; split z adds z * split_stride
  int64_t lda, ldb, ldc, split_stride;
  int32_t M, N, K, kchunk;
  const float* bias;    // [N] (kBiasSilu; optional for kAdd)
  float* C2;            // kBiasSilu: SiLU of C
  const float* R;       // kAdd: residual, same layout as C
};

// Global -> registers for one operand tile: 128 rows (m or n) x 16 k.
template <bool KC>
__device__ __forceinline__ void sg_fetch(const float* __restrict__ X, int64_t ld, int rows, int r0, int k0, int kend,
                                         int tid, float4 (&v)[2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + 256 * i;
    if (KC) {
      const int r = r0 + (idx >> 2), k = k0 + 4 * (idx & 3);
      v[i] = (r < rows && k < kend) ? *reinterpret_cast<const float4*>(X + (size_t)r * ld + k)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
      const int k = k0 + (idx >> 5), r = r0 + 4 * (idx & 31);
      v[i] = (k < kend && r < rows) ? *reinterpret_cast<const float4*>(X + (size_t)k * ld + r)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
}

// Registers -> LDS.  A k-contiguous operand is stored as S[row][k] (row
// stride kLdk), a row-contiguous one as S[k][row] (row stride kLdr): both
// as 16-byte stores, and both read without bank conflicts by sg_frag.
constexpr int kLdr = kBM + 4;
constexpr int kTileFloats = kBM * kLdk > kBK * kLdr ? kBM * kLdk : kBK * kLdr;

template <bool KC>
__device__ __forceinline__ void sg_put(float* S, int tid, const float4 (&v)[2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + 256 * i;
    if (KC) {
      *reinterpret_cast<float4*>(&S[(idx >> 2) * kLdk + 4 * (idx & 3)]) = v[i];
    } else {
      *reinterpret_cast<float4*>(&S[(idx >> 5) * kLdr + 4 * (idx & 31)]) = v[i];
    }
  }
}

// The four values lane (q, i) feeds MFMA number j = 0..3 of a stage for the
// 16 rows starting at r0: element (r0 + i, k = 4q + j).
template <bool KC>
__device__ __forceinline__ f4v sg_frag(const float* S, int r0, int li, int lq) {
  if (KC) return *reinterpret_cast<const f4v*>(&S[(r0 + li) * kLdk + 4 * lq]);
  f4v v;
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = S[(4 * lq + j) * kLdr + r0 + li];
  return v;
}

template <bool AK, bool BK, int EPI>
__global__ void __launch_bounds__(256) k_sgemm(Sg g) {
  __shared__ __attribute__((aligned(16))) float As[2][kTileFloats];
  __shared__ __attribute__((aligned(16))) float Bs[2][kTileFloats];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, li = lane & 15, lq = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * kBN, m0 = blockIdx.y * kBM, z = blockIdx.z;
  const int kbeg = z * g.kchunk;
  const int kend = min(g.K, kbeg + g.kchunk);
  const int nst = (kend - kbeg + kBK - 1) / kBK;

  f4v acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f4v{0.f, 0.f, 0.f, 0.f};

  float4 ra[2], rb[2];
  sg_fetch<AK>(g.A, g.lda, g.M, m0, kbeg, kend, tid, ra);
  sg_fetch<BK>(g.B, g.ldb, g.N, n0, kbeg, kend, tid, rb);
  sg_put<AK>(As[0], tid, ra);
  sg_put<BK>(Bs[0], tid, rb);
  __syncthreads();
  for (int s = 0; s < nst; ++s) {
    const int cur = s & 1;
    const bool more = s + 1 < nst;
    if (more) {
      sg_fetch<AK>(g.A, g.lda, g.M, m0, kbeg + (s + 1) * kBK, kend, tid, ra);
      sg_fetch<BK>(g.B, g.ldb, g.N, n0, kbeg + (s + 1) * kBK, kend, tid, rb);
    }
    f4v a[4], b[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      a[t] = sg_frag<AK>(As[cur], wm * 64 + t * 16, li, lq);
      b[t] = sg_frag<BK>(Bs[cur], wn * 64 + t * 16, li, lq);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[mt][j], b[nt][j], acc[mt][nt], 0, 0, 0);
    if (more) {
      sg_put<AK>(As[cur ^ 1], tid, ra);
      sg_put<BK>(Bs[cur ^ 1], tid, rb);
    }
    __syncthreads();
  }

#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * 64 + mt * 16 + 4 * lq + r;
        const int n = n0 + wn * 64 + nt * 16 + li;
        if (m < g.M && n < g.N) {
          const float v = acc[mt][nt][r];
          const size_t o = (size_t)m * g.ldc + n;
          if (EPI == kStore) {
            g.C[(size_t)z * g.split_stride + o] = v;
          } else if (EPI == kBiasSilu) {
            const float pre = v + g.bias[n];
            g.C[o] = pre;
            g.C2[o] = pre * sigm(pre);
          } else {
            g.C[o] = v + (g.bias != nullptr ? g.bias[n] : 0.0f) + g.R[o];
          }
        }
      }
}

// out[i] = sum over z of part[z * stride + i], z ascending.
__global__ void __launch_bounds__(256) k_split_sum(const float* __restrict__ part, int splits, int64_t stride,
                                                   int64_t n4, float* __restrict__ out) {
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    float4 s = reinterpret_cast<const float4*>(part)[i];
    for (int z = 1; z < splits; ++z) {
      const float4 v = reinterpret_cast<const float4*>(part + z * stride)[i];
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    reinterpret_cast<float4*>(out)[i] = s;
  }
}

// ===========================================================================
// row kernels of the head
// ===========================================================================
struct RowArgs {
  // tower inputs
  const uint16_t* E;
  const uint16_t* hL;
  const uint16_t* hF;
  const int32_t* tokens;
  const int32_t* prev;
  const float* gain;
  const float* gamma[3];
  float* xhat;     // [3][N][D]
  float* xn;       // [3][N][D]
  int32_t* err;
  int32_t N, D, V;
  float lambda;
};

// Per row: the three tower inputs (h_prev chosen from the previous row's
// gain, E[x_t], h^L), their RMS-normalised values and gamma-scaled values.
__global__ void __launch_bounds__(256) k_tower_in(RowArgs a) {
  __shared__ float red[4];
  const int n = blockIdx.x, D = a.D, N = a.N;
  const uint16_t* src[3];
  int p = a.prev[n];
  if (p >= N || p < -1) {
    if (threadIdx.x == 0) raise_err(a.err, ODA_ERR_ROW);
    p = -1;
  }
  if (p < 0) {
    src[0] = nullptr;
  } else {
    const float d = a.gain[p] - a.lambda;
    src[0] = ((!isfinite(d) || d > 0.0f) ? a.hF : a.hL) + (size_t)p * D;
  }
  const int tok = a.tokens[n];
  if (tok < 0 || tok >= a.V) {
    if (threadIdx.x == 0) raise_err(a.err, ODA_ERR_TOKEN);
    src[1] = nullptr;
  } else {
    src[1] = a.E + (size_t)tok * D;
  }
  src[2] = a.hL + (size_t)n * D;
  for (int s = 0; s < 3; ++s) {
    float ss = 0.0f;
    for (int i = threadIdx.x; i < D; i += 256) {
      const float x = src[s] != nullptr ? bf16_to_f32(src[s][i]) : 0.0f;
      ss += x * x;
    }
    const float inv = rsqrtf(block_sum256(ss, red) / (float)D + kEps);
    float* xh = a.xhat + ((size_t)s * N + n) * D;
    float* xg = a.xn + ((size_t)s * N + n) * D;
    for (int i = threadIdx.x; i < D; i += 256) {
      const float x = src[s] != nullptr ? bf16_to_f32(src[s][i]) : 0.0f;
      const float h = x * inv;
      xh[i] = h;
      xg[i] = h * a.gamma[s][i];
    }
  }
}

// Z = [a, b, c, ab, ac, bc, |a-b|, |a-c|, |b-c|] and S = a + b + c.
__global__ void __launch_bounds__(256) k_interact(const float* __restrict__ act, float* __restrict__ Z,
                                                  float* __restrict__ S, int N) {
  constexpr int T = kTower;
  const int i = blockIdx.x * 256 + threadIdx.x, n = blockIdx.y;
  const size_t o = (size_t)n * T + i;
  const float a = act[o], b = act[(size_t)N * T + o], c = act[2 * (size_t)N * T + o];
  float* z = Z + (size_t)n * 9 * T + i;
  z[0] = a;
  z[T] = b;
  z[2 * T] = c;
  z[3 * T] = a * b;
  z[4 * T] = a * c;
  z[5 * T] = b * c;
  z[6 * T] = fabsf(a - b);
  z[7 * T] = fabsf(a - c);
  z[8 * T] = fabsf(b - c);
  S[o] = (a + b) + c;
}

// uhat = u / rms(u), r = gamma * uhat (width T).
__global__ void __launch_bounds__(256) k_rownorm(const float* __restrict__ u, const float* __restrict__ gamma,
                                                 float* __restrict__ uhat, float* __restrict__ r) {
  __shared__ float red[4];
  constexpr int T = kTower;
  const size_t base = (size_t)blockIdx.x * T;
  float v[T / 256];
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < T / 256; ++j) {
    v[j] = u[base + threadIdx.x + 256 * j];
    ss += v[j] * v[j];
  }
  const float inv = rsqrtf(block_sum256(ss, red) / (float)T + kEps);
#pragma unroll
  for (int j = 0; j < T / 256; ++j) {
    const int i = threadIdx.x + 256 * j;
    const float h = v[j] * inv;
    uhat[base + i] = h;
    r[base + i] = h * gamma[i];
  }
}

// M = SiLU(G) * U from GU = [G | U] (rows of width 2F).
__global__ void __launch_bounds__(256) k_swiglu(const float* __restrict__ GU, float* __restrict__ M) {
  constexpr int F = kFfn;
  const int i = blockIdx.x * 256 + threadIdx.x;
  const size_t n = blockIdx.y;
  const float G = GU[n * 2 * F + i], U = GU[n * 2 * F + F + i];
  M[n * F + i] = G * sigm(G) * U;
}

__global__ void __launch_bounds__(256) k_count_valid(const uint8_t* __restrict__ valid, int N, int32_t* out) {
  __shared__ float red[4];
  float c = 0.0f;
  for (int n = threadIdx.x; n < N; n += 256) c += valid[n] != 0 ? 1.0f : 0.0f;
  c = block_sum256(c, red);
  if (threadIdx.x == 0) *out = (int32_t)c;
}

struct OutArgs {
  const float* u2;
  const float* gamma_o;
  const float* w_o;
  const float* c_o;
  const float* label;
  const uint8_t* valid;
  const int32_t* nvalid;
  float* uhat_o;
  float* on;
  float* score;
  float* hub;
  float* dq;
  float* du;
};

// Output norm and projection, the row's Huber term and dL/dq, and the
// gradient of the loss with respect to u2 through the output norm.
__global__ void __launch_bounds__(256) k_head_out(OutArgs a) {
  __shared__ float red[4];
  constexpr int T = kTower, J = T / 256;
  const int n = blockIdx.x;
  const size_t base = (size_t)n * T;
  float u[J], on[J];
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    u[j] = a.u2[base + threadIdx.x + 256 * j];
    ss += u[j] * u[j];
  }
  const float inv = rsqrtf(block_sum256(ss, red) / (float)T + kEps);
  float dot = 0.0f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = threadIdx.x + 256 * j;
    const float h = u[j] * inv;
    on[j] = h * a.gamma_o[i];
    a.uhat_o[base + i] = h;
    a.on[base + i] = on[j];
    dot += on[j] * a.w_o[i];
  }
  const float q = block_sum256(dot, red) + a.c_o[0];
  const int nv = *a.nvalid;
  const bool use = a.valid[n] != 0 && nv > 0;
  const float r = q - a.label[n];
  const float hub = use ? (fabsf(r) <= 1.0f ? 0.5f * r * r : fabsf(r) - 0.5f) : 0.0f;
  const float dq = use ? fminf(fmaxf(r, -1.0f), 1.0f) / (float)nv : 0.0f;
  if (threadIdx.x == 0) {
    a.score[n] = q;
    a.hub[n] = hub;
    a.dq[n] = dq;
  }
  // dL/d on = dq * w_o; through on = gamma * u * inv
  float sg = 0.0f;
  float gd[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = threadIdx.x + 256 * j;
    gd[j] = a.gamma_o[i] * dq * a.w_o[i];
    sg += gd[j] * u[j];
  }
  sg = block_sum256(sg, red);
  const float c = inv * inv * inv * sg / (float)T;
#pragma unroll
  for (int j = 0; j < J; ++j) a.du[base + threadIdx.x + 256 * j] = gd[j] * inv - u[j] * c;
}

// loss = sum of Huber terms / |valid|; the output-bias gradient = sum of dq.
__global__ void __launch_bounds__(256) k_loss(const float* __restrict__ hub, const float* __restrict__ dq, int N,
                                              const int32_t* nvalid, float* loss, float* grad_c_o) {
  __shared__ float red[4];
  float h = 0.0f, d = 0.0f;
  for (int n = threadIdx.x; n < N; n += 256) {
    h += hub[n];
    d += dq[n];
  }
  h = block_sum256(h, red);
  d = block_sum256(d, red);
  if (threadIdx.x == 0) {
    const int nv = *nvalid;
    *loss = nv > 0 ? h / (float)nv : 0.0f;
    *grad_c_o = d;
  }
}

// dG = dM U SiLU'(G), dU = dM SiLU(G)  ->  dGU = [dG | dU].
__global__ void __launch_bounds__(256) k_swiglu_bwd(const float* __restrict__ GU, const float* __restrict__ dM,
                                                    float* __restrict__ dGU) {
  constexpr int F = kFfn;
  const int i = blockIdx.x * 256 + threadIdx.x;
  const size_t n = blockIdx.y;
  const float G = GU[n * 2 * F + i], U = GU[n * 2 * F + F + i], d = dM[n * F + i];
  const float s = sigm(G);
  dGU[n * 2 * F + i] = d * U * (s * (1.0f + G * (1.0f - s)));
  dGU[n * 2 * F + F + i] = d * G * s;
}

// du += d(norm)/du applied to dr, for r = gamma * u / rms(u) (width T).
__global__ void __launch_bounds__(256) k_rownorm_bwd(const float* __restrict__ dr, const float* __restrict__ u,
                                                     const float* __restrict__ gamma, float* __restrict__ du) {
  __shared__ float red[4];
  constexpr int T = kTower, J = T / 256;
  const size_t base = (size_t)blockIdx.x * T;
  float uv[J], gd[J];
  float ss = 0.0f, sg = 0.0f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = threadIdx.x + 256 * j;
    uv[j] = u[base + i];
    gd[j] = gamma[i] * dr[base + i];
    ss += uv[j] * uv[j];
    sg += gd[j] * uv[j];
  }
  const float inv = rsqrtf(block_sum256(ss, red) / (float)T + kEps);
  sg = block_sum256(sg, red);
  const float c = inv * inv * inv * sg / (float)T;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const size_t o = base + threadIdx.x + 256 * j;
    du[o] += gd[j] * inv - uv[j] * c;
  }
}

__device__ __forceinline__ float sgnf(float x) { return (float)(x > 0.0f) - (float)(x < 0.0f); }

// From dZ and du0 (the residual a + b + c): the tower outputs' gradients,
// then through SiLU to the tower pre-activations.
__global__ void __launch_bounds__(256) k_interact_bwd(const float* __restrict__ du, const float* __restrict__ dZ,
                                                      const float* __restrict__ act, const float* __restrict__ pre,
                                                      float* __restrict__ dpre, int N) {
  constexpr int T = kTower;
  const int i = blockIdx.x * 256 + threadIdx.x, n = blockIdx.y;
  const size_t o = (size_t)n * T + i, NT = (size_t)N * T;
  const float a = act[o], b = act[NT + o], c = act[2 * NT + o];
  const float* z = dZ + (size_t)n * 9 * T + i;
  const float s_ab = sgnf(a - b), s_ac = sgnf(a - c), s_bc = sgnf(b - c);
  const float d0 = du[o];
  const float da = d0 + z[0] + z[3 * T] * b + z[4 * T] * c + z[6 * T] * s_ab + z[7 * T] * s_ac;
  const float db = d0 + z[T] + z[3 * T] * a + z[5 * T] * c - z[6 * T] * s_ab + z[8 * T] * s_bc;
  const float dc = d0 + z[2 * T] + z[4 * T] * a + z[5 * T] * b - z[7 * T] * s_ac - z[8 * T] * s_bc;
  const float dt[3] = {da, db, dc};
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    const float p = pre[s * NT + o];
    const float sg = sigm(p);
    dpre[s * NT + o] = dt[s] * (sg * (1.0f + p * (1.0f - sg)));
  }
}

// part[chunk][j] = sum over the chunk's rows of A[n][j] (* B[n][j]) (* rs[n]).
__global__ void __launch_bounds__(256) k_colsum_part(const float* __restrict__ A, const float* __restrict__ B,
                                                     const float* __restrict__ rs, int rows, int cols,
                                                     float* __restrict__ part) {
  const int j = blockIdx.x * 256 + threadIdx.x, c = blockIdx.y, nc = gridDim.y;
  if (j >= cols) return;
  const int n0 = (int)((int64_t)rows * c / nc), n1 = (int)((int64_t)rows * (c + 1) / nc);
  float s = 0.0f;
  for (int n = n0; n < n1; ++n) {
    float v = A[(size_t)n * cols + j];
    if (B != nullptr) v *= B[(size_t)n * cols + j];
    if (rs != nullptr) v *= rs[n];
    s += v;
  }
  part[(size_t)c * cols + j] = s;
}

// out[j] = sum over chunks of part[c][j] (* post[j]); four threads per
// column take the chunks c = 4 i + t in order, then add their sums in t order.
__global__ void __launch_bounds__(256) k_colsum_fin(const float* __restrict__ part, int chunks, int cols,
                                                    const float* __restrict__ post, float* __restrict__ out) {
  const int j = blockIdx.x * 64 + (threadIdx.x >> 2), t = threadIdx.x & 3;
  float s = 0.0f;
  if (j < cols)
    for (int c = t; c < chunks; c += 4) s += part[(size_t)c * cols + j];
  const int base = threadIdx.x & ~3;
  const float s0 = __shfl(s, base, 64), s1 = __shfl(s, base + 1, 64), s2 = __shfl(s, base + 2, 64),
              s3 = __shfl(s, base + 3, 64);
  if (t == 0 && j < cols) {
    const float v = (s0 + s1) + (s2 + s3);
    out[j] = post != nullptr ? v * post[j] : v;
  }
}

// ===========================================================================
// labels: log-sum-exp of E h over the vocabulary for 2N rows
// ===========================================================================
constexpr int kLBM = 256, kLBN = 256, kLBK = 64, kLLd = kLBK + 8;  // 144-byte LDS rows: conflict-free b128 reads
constexpr int kLThreads = 512;                                       // 8 waves, 2 x 4, each 128 rows x 64 columns
constexpr int kLGroup = 16;                                          // row blocks walked together per XCD

struct LseArgs {
  const uint16_t* E;       // [V][D]
  const uint16_t* hL;      // rows 0 .. N-1
  const uint16_t* hF;      // rows N .. 2N-1
  const int32_t* tok;      // next_tok, resolved: -1 or a vocabulary row
  float2* part;            // [ntiles][R] (max, sum of exp) per vocabulary tile
  float* tgt;              // [R] logit of the reference token
  int32_t N, D, V, R, rblocks, ntiles;
  int32_t per_xcd;         // workgroup slots per XCD
};

__device__ __forceinline__ const uint16_t* lse_row(const LseArgs& a, int r) {
  return r < a.N ? a.hL + (size_t)r * a.D : a.hF + (size_t)(r - a.N) * a.D;
}

// One stage: 256 hidden rows and 256 vocabulary rows of 64 k each, four
// 16-byte pieces per thread and operand (rows idx / 8 + 64 j).  Named fields
// rather than arrays keep the pieces in registers.  Rows past the ends are
// clamped to the last row rather than skipped: their logits land in rows
// that are never written and in columns the epilogue masks, and
// unconditional loads keep the compiler's wait counts exact.
struct LseStage {
  uint4 a0, a1, a2, a3, b0, b1, b2, b3;
};

__device__ __forceinline__ uint4 lse_ld(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ LseStage lse_fetch(const LseArgs& a, int r0, int v0, int k0, int tid) {
  const int row = tid >> 3, kk = k0 + 8 * (tid & 7);
  const int rm = a.R - 1, vm = a.V - 1;
  const uint16_t* E = a.E + kk;
  const size_t D = a.D;
  LseStage st;
  st.a0 = lse_ld(lse_row(a, min(r0 + row, rm)) + kk);
  st.a1 = lse_ld(lse_row(a, min(r0 + row + 64, rm)) + kk);
  st.a2 = lse_ld(lse_row(a, min(r0 + row + 128, rm)) + kk);
  st.a3 = lse_ld(lse_row(a, min(r0 + row + 192, rm)) + kk);
  st.b0 = lse_ld(E + (size_t)min(v0 + row, vm) * D);
  st.b1 = lse_ld(E + (size_t)min(v0 + row + 64, vm) * D);
  st.b2 = lse_ld(E + (size_t)min(v0 + row + 128, vm) * D);
  st.b3 = lse_ld(E + (size_t)min(v0 + row + 192, vm) * D);
  return st;
}

__device__ __forceinline__ void lse_put(uint16_t (*As)[kLLd], uint16_t (*Bs)[kLLd], int tid, const LseStage& st) {
  const int row = tid >> 3, c = 8 * (tid & 7);
  *reinterpret_cast<uint4*>(&As[row][c]) = st.a0;
  *reinterpret_cast<uint4*>(&As[row + 64][c]) = st.a1;
  *reinterpret_cast<uint4*>(&As[row + 128][c]) = st.a2;
  *reinterpret_cast<uint4*>(&As[row + 192][c]) = st.a3;
  *reinterpret_cast<uint4*>(&Bs[row][c]) = st.b0;
  *reinterpret_cast<uint4*>(&Bs[row + 64][c]) = st.b1;
  *reinterpret_cast<uint4*>(&Bs[row + 128][c]) = st.b2;
  *reinterpret_cast<uint4*>(&Bs[row + 192][c]) = st.b3;
}

// One stage of a wave's 128 x 64 block: two 32-k steps of 8 x 4 MFMAs.  The
// scheduling groups issue the B and first A fragments, then interleave one
// LDS read with every two MFMAs (6% faster than leaving the order to the
// compiler, measured).
__device__ __forceinline__ void lse_mma(const uint16_t (*As)[kLLd], const uint16_t (*Bs)[kLLd], int wm, int wn,
                                        int li, int lq, f4v (&acc)[8][4]) {
#pragma unroll
  for (int kk = 0; kk < kLBK / 32; ++kk) {
    bf16x8 bv[4], av[8];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      bv[t] = __builtin_bit_cast(bf16x8,
                                 *reinterpret_cast<const uint4*>(&Bs[wn * 64 + t * 16 + li][32 * kk + 8 * lq]));
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
      av[mt] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(&As[wm * 128 + mt * 16 + li][32 * kk + 8 * lq]));
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt], bv[nt], acc[mt][nt], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);
#pragma unroll
    for (int i = 0; i < 7; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  }
}

__global__ void __launch_bounds__(kLThreads) k_lse(LseArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kLBM][kLLd];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kLBN][kLLd];
  __shared__ int s_tok[kLBM];
  __shared__ float s_m[4][kLBM], s_s[4][kLBM];

  // workgroup -> (row block, vocabulary tile): XCD x owns tiles
  // [x ntiles / 8, (x + 1) ntiles / 8) and walks them for kLGroup row blocks
  // at a time
  const int xcd = blockIdx.x % kXcds, k = blockIdx.x / kXcds;
  const int t_lo = (int)((int64_t)a.ntiles * xcd / kXcds), t_hi = (int)((int64_t)a.ntiles * (xcd + 1) / kXcds);
  const int nt_x = t_hi - t_lo;
  if (nt_x == 0 || k >= nt_x * a.rblocks) return;
  const int grp = k / (kLGroup * nt_x), rem = k % (kLGroup * nt_x);
  const int gcnt = min(kLGroup, a.rblocks - grp * kLGroup);
  const int tile = t_lo + rem / gcnt, rb = grp * kLGroup + rem % gcnt;
  const int r0 = rb * kLBM, v0 = tile * kLBN;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, li = lane & 15, lq = lane >> 4;
  const int wm = wave >> 2, wn = wave & 3;
  if (tid < kLBM) {
    const int r = r0 + tid;
    s_tok[tid] = r < a.R ? a.tok[r < a.N ? r : r - a.N] : -1;
  }

  f4v acc[8][4];
#pragma unroll
  for (int x = 0; x < 8; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f4v{0.f, 0.f, 0.f, 0.f};

  // K stages of 64, double-buffered in LDS: the next stage's loads are in
  // flight during a stage's 64 MFMAs per wave
  const int nst = a.D / kLBK;
  LseStage g = lse_fetch(a, r0, v0, 0, tid);
  lse_put(As[0], Bs[0], tid, g);
  __syncthreads();
  for (int s = 0; s < nst; ++s) {
    const int cur = s & 1;
    const bool more = s + 1 < nst;
    if (more) g = lse_fetch(a, r0, v0, (s + 1) * kLBK, tid);
    lse_mma(As[cur], Bs[cur], wm, wn, li, lq, acc);
    if (more) lse_put(As[cur ^ 1], Bs[cur ^ 1], tid, g);
    __syncthreads();
  }

  // per row: max and sum of exp over this tile's columns (< V), the
  // reference token's logit where it falls in the tile
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rl = wm * 128 + mt * 16 + 4 * lq + r;
      float mx = -INFINITY;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int col = v0 + wn * 64 + nt * 16 + li;
        if (col < a.V) mx = fmaxf(mx, acc[mt][nt][r]);
      }
      mx = row16_max(mx);
      float sm = 0.0f;
      const int tk = s_tok[rl];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int col = v0 + wn * 64 + nt * 16 + li;
        if (col < a.V) sm += expf(acc[mt][nt][r] - mx);
        if (col == tk && r0 + rl < a.R) a.tgt[r0 + rl] = acc[mt][nt][r];
      }
      sm = row16_sum(sm);
      if (li == 0) {
        s_m[wn][rl] = mx;
        s_s[wn][rl] = sm;
      }
    }
  __syncthreads();
  if (tid < kLBM && r0 + tid < a.R) {
    float M = s_m[0][tid];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, s_m[w][tid]);
    float S = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (s_m[w][tid] != -INFINITY) S += s_s[w][tid] * expf(s_m[w][tid] - M);
    a.part[(size_t)tile * a.R + r0 + tid] = make_float2(M, S);
  }
}

// next_tok -> -1 or a vocabulary row (ODA_ERR_TOKEN for ids outside the vocabulary)
__global__ void __launch_bounds__(256) k_resolve_tok(const int32_t* __restrict__ next_tok, int N, int V,
                                                     int32_t* __restrict__ out, int32_t* err) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  int t = next_tok[n];
  if (t != -1 && (t < 0 || t >= V)) {
    raise_err(err, ODA_ERR_TOKEN);
    t = -1;
  }
  out[n] = t;
}

// Per row: merge the tiles' pairs in tile order (four interleaved streams,
// then the four in order) into lse.
__global__ void __launch_bounds__(256) k_lse_fin(const float2* __restrict__ part, int ntiles, int R,
                                                 float* __restrict__ lse) {
  const int r = blockIdx.x * 64 + (threadIdx.x >> 2), j = threadIdx.x & 3;
  float M = -INFINITY, S = 0.0f;
  if (r < R) {
    for (int t = j; t < ntiles; t += 4) {
      const float2 p = part[(size_t)t * R + r];
      if (p.x > M) {
        S = S * expf(M - p.x) + p.y;
        M = p.x;
      } else {
        S += p.y * expf(p.x - M);
      }
    }
  }
  // combine lanes j = 0..3 of the row in order
  float Ms[4], Ss[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    Ms[q] = __shfl(M, (threadIdx.x & ~3) + q, 64);
    Ss[q] = __shfl(S, (threadIdx.x & ~3) + q, 64);
  }
  if (j == 0 && r < R) {
    float MM = Ms[0];
    for (int q = 1; q < 4; ++q) MM = fmaxf(MM, Ms[q]);
    float SS = 0.0f;
    for (int q = 0; q < 4; ++q)
      if (Ms[q] != -INFINITY) SS += Ss[q] * expf(Ms[q] - MM);
    lse[r] = MM + logf(SS);
  }
}

__global__ void __launch_bounds__(256) k_labels(const float* __restrict__ lse, const float* __restrict__ tgt,
                                                const int32_t* __restrict__ tok, const int32_t* __restrict__ pos,
                                                int N, int sw, float lambda, float* __restrict__ gain,
                                                float* __restrict__ label, uint8_t* __restrict__ valid) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  float g = 0.0f, y = 0.0f;
  uint8_t v = 0;
  if (tok[n] >= 0) {
    g = (tgt[N + n] - lse[N + n]) - (tgt[n] - lse[n]);
    if (isfinite(g)) {
      const float d = g - lambda;
      y = d > 0.0f ? log1pf(d) : (d < 0.0f ? -log1pf(-d) : 0.0f);
      v = pos[n] >= sw ? 1 : 0;
    }
  }
  gain[n] = g;
  label[n] = y;
  valid[n] = v;
}

// ===========================================================================
// host side
// ===========================================================================
size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

int lse_tiles(int V) { return (V + kLBN - 1) / kLBN; }

// Weight-gradient GEMMs (K = rows) split K so that about 512 workgroups run.
int wgrad_splits(int M, int N, int K) {
  const int tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  int s = (512 + tiles - 1) / tiles;
  const int cap = K / 512 > 1 ? K / 512 : 1;
  return s < cap ? s : cap;
}

struct TrainWs {
  size_t header;    // int32[64]: [0] error bits, [16] valid-row count
  size_t tok;       // int32[N] resolved next tokens
  size_t lse_part;  // float2[ntiles][2N]
  size_t tgt, lse;  // float[2N]
  size_t xhat, xn;  // float[3][N][D]
  size_t pre, act;  // float[3][N][T]
  size_t Z;         // float[N][9T] (dZ in the backward pass)
  size_t S, u0, u1, u2, uh1, r1, uh2, r2, uho, on, du, dr;  // float[N][T]
  size_t GU1, GU2, dGU;      // float[N][2F]
  size_t M1, M2, dM;         // float[N][F]
  size_t dpre;               // float[3][N][T]
  size_t dxn;                // float[N][D]
  size_t hub, dq;            // float[N]
  size_t split;              // split-K partials
  size_t colpart;            // float[kColChunks][max(D, T)]
  size_t total;
};

size_t split_floats(int N, int D) {
  const int T = kTower, F = kFfn;
  const int shapes[4][2] = {{T, F}, {2 * F, T}, {T, 9 * T}, {T, D}};
  size_t m = 0;
  for (auto& s : shapes) {
    const int z = wgrad_splits(s[0], s[1], N);
    if (z > 1) m = std::max(m, (size_t)z * s[0] * s[1]);
  }
  return m;
}

TrainWs train_ws(int N, int D, int V) {
  const size_t T = kTower, F = kFfn, n = N, R = 2 * n;
  TrainWs w;
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t o = at;
    at += al256(bytes);
    return o;
  };
  w.header = take(256);
  w.tok = take(n * 4);
  w.lse_part = take((size_t)lse_tiles(V) * R * 8);
  w.tgt = take(R * 4);
  w.lse = take(R * 4);
  w.xhat = take(3 * n * D * 4);
  w.xn = take(3 * n * D * 4);
  w.pre = take(3 * n * T * 4);
  w.act = take(3 * n * T * 4);
  w.Z = take(n * 9 * T * 4);
  size_t* rowT[] = {&w.S, &w.u0, &w.u1, &w.u2, &w.uh1, &w.r1, &w.uh2, &w.r2, &w.uho, &w.on, &w.du, &w.dr};
  for (size_t* p : rowT) *p = take(n * T * 4);
  w.GU1 = take(n * 2 * F * 4);
  w.GU2 = take(n * 2 * F * 4);
  w.dGU = take(n * 2 * F * 4);
  w.M1 = take(n * F * 4);
  w.M2 = take(n * F * 4);
  w.dM = take(n * F * 4);
  w.dpre = take(3 * n * T * 4);
  w.dxn = take(n * D * 4);
  w.hub = take(n * 4);
  w.dq = take(n * 4);
  w.split = take(split_floats(N, D) * 4 + 16);
  w.colpart = take((size_t)kColChunks * std::max((size_t)D, T) * 4);
  w.total = at;
  return w;
}

bool train_dims_ok(const oda_train_dims* d) {
  return d != nullptr && d->rows >= 1 && d->rows <= kMaxRows && d->hidden >= 256 && d->hidden % 256 == 0 &&
         d->hidden <= 16384 && d->vocab >= 1 && d->sink >= 0 && d->window >= 1 && d->lambda >= 0.0f &&
         isfinite(d->lambda);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

template <bool AK, bool BK, int EPI>
int sgemm(Sg g, int splits, float* split_buf, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0 || g.K <= 0) return ODA_OK;
  int kc = (g.K + splits - 1) / splits;
  kc = (kc + kBK - 1) / kBK * kBK;
  splits = (g.K + kc - 1) / kc;
  g.kchunk = kc;
  float* dst = g.C;
  // split partials are summed into a contiguous destination (a gradient tensor)
  if (splits > 1 && (EPI != kStore || g.ldc != g.N || ((int64_t)g.M * g.N) % 4 != 0)) return ODA_E_UNSUPPORTED;
  if (splits > 1) {
    g.C = split_buf;
    g.ldc = g.N;
    g.split_stride = (int64_t)g.M * g.N;
  }
  dim3 grid((g.N + kBN - 1) / kBN, (g.M + kBM - 1) / kBM, splits);
  hipLaunchKernelGGL((k_sgemm<AK, BK, EPI>), grid, dim3(256), 0, st, g);
  if (splits > 1) {
    const int64_t n4 = (int64_t)g.M * g.N / 4;
    const int blocks = (int)std::min<int64_t>((n4 + 255) / 256, 4096);
    hipLaunchKernelGGL(k_split_sum, dim3(blocks), dim3(256), 0, st, split_buf, splits, g.split_stride, n4, dst);
  }
  return ODA_OK;
}

Sg sg(const float* A, int64_t lda, const float* B, int64_t ldb, float* C, int64_t ldc, int M, int N, int K) {
  Sg g;
  memset(&g, 0, sizeof(g));
  g.A = A;
  g.lda = lda;
  g.B = B;
  g.ldb = ldb;
  g.C = C;
  g.ldc = ldc;
  g.M = M;
  g.N = N;
  g.K = K;
  return g;
}

void colsum(const float* A, const float* B, const float* rs, int rows, int cols, const float* post, float* out,
            float* part, hipStream_t st) {
  const int chunks = std::max(1, std::min(kColChunks, rows / 32));
  dim3 g1((cols + 255) / 256, chunks);
  hipLaunchKernelGGL(k_colsum_part, g1, dim3(256), 0, st, A, B, rs, rows, cols, part);
  hipLaunchKernelGGL(k_colsum_fin, dim3((cols + 63) / 64), dim3(256), 0, st, part, chunks, cols, post, out);
}

}  // namespace
}  // namespace oda

using namespace oda;

extern "C" {

size_t oda_train_workspace_bytes(const oda_train_dims* dims) {
  if (!train_dims_ok(dims)) return 0;
  return train_ws(dims->rows, dims->hidden, dims->vocab).total;
}

int oda_train_workspace_init(const oda_train_dims* dims, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (dims == nullptr || ws == nullptr) return ODA_E_NULL;
  if (!train_dims_ok(dims)) return ODA_E_DIMS;
  if (ws_bytes < train_ws(dims->rows, dims->hidden, dims->vocab).total) return ODA_E_WORKSPACE;
  return launch_fill_zero(static_cast<int32_t*>(ws), 64, stream);
}

int oda_train_labels(const oda_train_dims* dims, const oda_bf16* lm_head, const oda_bf16* h_local,
                     const oda_bf16* h_full, const int32_t* next_tok, const int32_t* pos, float* gain, float* label,
                     uint8_t* valid, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (dims == nullptr || lm_head == nullptr || h_local == nullptr || h_full == nullptr || next_tok == nullptr ||
      pos == nullptr || gain == nullptr || label == nullptr || valid == nullptr || ws == nullptr)
    return ODA_E_NULL;
  if (!train_dims_ok(dims)) return ODA_E_DIMS;
  if (!aligned16(lm_head) || !aligned16(h_local) || !aligned16(h_full)) return ODA_E_DIMS;
  const int N = dims->rows, D = dims->hidden, V = dims->vocab;
  const TrainWs W = train_ws(N, D, V);
  if (ws_bytes < W.total) return ODA_E_WORKSPACE;
  char* b = static_cast<char*>(ws);
  int32_t* err = reinterpret_cast<int32_t*>(b + W.header);
  int32_t* tok = reinterpret_cast<int32_t*>(b + W.tok);
  float* tgt = reinterpret_cast<float*>(b + W.tgt);
  float* lse = reinterpret_cast<float*>(b + W.lse);
  hipLaunchKernelGGL(k_resolve_tok, dim3((N + 255) / 256), dim3(256), 0, stream, next_tok, N, V, tok, err);
  LseArgs a;
  a.E = lm_head;
  a.hL = h_local;
  a.hF = h_full;
  a.tok = tok;
  a.part = reinterpret_cast<float2*>(b + W.lse_part);
  a.tgt = tgt;
  a.N = N;
  a.D = D;
  a.V = V;
  a.R = 2 * N;
  a.rblocks = (2 * N + kLBM - 1) / kLBM;
  a.ntiles = lse_tiles(V);
  a.per_xcd = 0;
  for (int x = 0; x < kXcds; ++x) {
    const int t_lo = (int)((int64_t)a.ntiles * x / kXcds), t_hi = (int)((int64_t)a.ntiles * (x + 1) / kXcds);
    a.per_xcd = std::max(a.per_xcd, (t_hi - t_lo) * a.rblocks);
  }
  hipLaunchKernelGGL(k_lse, dim3(a.per_xcd * kXcds), dim3(kLThreads), 0, stream, a);
  hipLaunchKernelGGL(k_lse_fin, dim3((2 * N + 63) / 64), dim3(256), 0, stream, a.part, a.ntiles, 2 * N, lse);
  hipLaunchKernelGGL(k_labels, dim3((N + 255) / 256), dim3(256), 0, stream, lse, tgt, tok, pos, N,
                     dims->sink + dims->window, dims->lambda, gain, label, valid);
  return hipGetLastError() == hipSuccess ? ODA_OK : ODA_E_LAUNCH;
}

int oda_train_head_step(const oda_train_dims* dims, const float* head_w, const oda_bf16* lm_head,
                        const oda_bf16* h_local, const oda_bf16* h_full, const int32_t* tokens, const int32_t* prev,
                        const float* gain, const float* label, const uint8_t* valid, float* score, float* loss,
                        float* grad, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (dims == nullptr || head_w == nullptr || lm_head == nullptr || h_local == nullptr || h_full == nullptr ||
      tokens == nullptr || prev == nullptr || gain == nullptr || label == nullptr || valid == nullptr ||
      score == nullptr || loss == nullptr || grad == nullptr || ws == nullptr)
    return ODA_E_NULL;
  if (!train_dims_ok(dims)) return ODA_E_DIMS;
  if (!aligned16(head_w) || !aligned16(grad)) return ODA_E_DIMS;
  const int N = dims->rows, D = dims->hidden, V = dims->vocab;
  constexpr int T = kTower, F = kFfn;
  const TrainWs W = train_ws(N, D, V);
  if (ws_bytes < W.total) return ODA_E_WORKSPACE;
  int64_t off[ODA_HEAD_NTENSORS + 1];
  if (oda_head_offsets(D, off) != ODA_OK) return ODA_E_DIMS;
  char* b = static_cast<char*>(ws);
  auto fp = [&](size_t o) { return reinterpret_cast<float*>(b + o); };
  int32_t* hdr = reinterpret_cast<int32_t*>(b + W.header);
  int32_t* nvalid = hdr + 16;
  float* split = fp(W.split);
  float* colp = fp(W.colpart);
  const size_t NT = (size_t)N * T, ND = (size_t)N * D;
  auto Wt = [&](int i) { return head_w + off[i]; };
  auto Gt = [&](int i) { return grad + off[i]; };
  // packed tensor indices (oda.h): tower s at 3s (gamma), 3s+1 (W), 3s+2 (c);
  // W_I 9, c_I 10; ffn k (1, 2) at 11 + 4(k-1): gamma, Wg, Wu, Wd; out 19, 20, 21
  int st = ODA_OK;

  // ---- forward ----
  RowArgs ra;
  ra.E = lm_head;
  ra.hL = h_local;
  ra.hF = h_full;
  ra.tokens = tokens;
  ra.prev = prev;
  ra.gain = gain;
  for (int s = 0; s < 3; ++s) ra.gamma[s] = Wt(3 * s);
  ra.xhat = fp(W.xhat);
  ra.xn = fp(W.xn);
  ra.err = hdr;
  ra.N = N;
  ra.D = D;
  ra.V = V;
  ra.lambda = dims->lambda;
  hipLaunchKernelGGL(k_tower_in, dim3(N), dim3(256), 0, stream, ra);
  for (int s = 0; s < 3 && st == ODA_OK; ++s) {
    Sg g = sg(fp(W.xn) + s * ND, D, Wt(3 * s + 1), D, fp(W.pre) + s * NT, T, N, T, D);
    g.bias = Wt(3 * s + 2);
    g.C2 = fp(W.act) + s * NT;
    st = sgemm<true, true, kBiasSilu>(g, 1, split, stream);
  }
  hipLaunchKernelGGL(k_interact, dim3(T / 256, N), dim3(256), 0, stream, fp(W.act), fp(W.Z), fp(W.S), N);
  {
    Sg g = sg(fp(W.Z), 9 * T, Wt(9), 9 * T, fp(W.u0), T, N, T, 9 * T);
    g.bias = Wt(10);
    g.R = fp(W.S);
    if (st == ODA_OK) st = sgemm<true, true, kAdd>(g, 1, split, stream);
  }
  const size_t uin[2] = {W.u0, W.u1}, uout[2] = {W.u1, W.u2}, uh[2] = {W.uh1, W.uh2}, rr[2] = {W.r1, W.r2};
  const size_t GU[2] = {W.GU1, W.GU2}, MM[2] = {W.M1, W.M2};
  for (int k = 0; k < 2 && st == ODA_OK; ++k) {
    const int t0 = 11 + 4 * k;
    hipLaunchKernelGGL(k_rownorm, dim3(N), dim3(256), 0, stream, fp(uin[k]), Wt(t0), fp(uh[k]), fp(rr[k]));
    st = sgemm<true, true, kStore>(sg(fp(rr[k]), T, Wt(t0 + 1), T, fp(GU[k]), 2 * F, N, 2 * F, T), 1, split, stream);
    hipLaunchKernelGGL(k_swiglu, dim3(F / 256, N), dim3(256), 0, stream, fp(GU[k]), fp(MM[k]));
    Sg g = sg(fp(MM[k]), F, Wt(t0 + 3), F, fp(uout[k]), T, N, T, F);
    g.R = fp(uin[k]);
    if (st == ODA_OK) st = sgemm<true, true, kAdd>(g, 1, split, stream);
  }
  hipLaunchKernelGGL(k_count_valid, dim3(1), dim3(256), 0, stream, valid, N, nvalid);
  OutArgs oa;
  oa.u2 = fp(W.u2);
  oa.gamma_o = Wt(19);
  oa.w_o = Wt(20);
  oa.c_o = Wt(21);
  oa.label = label;
  oa.valid = valid;
  oa.nvalid = nvalid;
  oa.uhat_o = fp(W.uho);
  oa.on = fp(W.on);
  oa.score = score;
  oa.hub = fp(W.hub);
  oa.dq = fp(W.dq);
  oa.du = fp(W.du);
  hipLaunchKernelGGL(k_head_out, dim3(N), dim3(256), 0, stream, oa);
  hipLaunchKernelGGL(k_loss, dim3(1), dim3(256), 0, stream, fp(W.hub), fp(W.dq), N, nvalid, loss, Gt(21));
  // output norm and projection: dw_o = sum dq on, dgamma_o = w_o * sum dq uhat_o
  colsum(fp(W.on), nullptr, fp(W.dq), N, T, nullptr, Gt(20), colp, stream);
  colsum(fp(W.uho), nullptr, fp(W.dq), N, T, Wt(20), Gt(19), colp, stream);

  // ---- backward through the two gated FFN blocks (du holds dL/du_out) ----
  for (int k = 1; k >= 0 && st == ODA_OK; --k) {
    const int t0 = 11 + 4 * k;
    // dWd = du^T M
    st = sgemm<false, false, kStore>(sg(fp(W.du), T, fp(MM[k]), F, Gt(t0 + 3), F, T, F, N),
                                     wgrad_splits(T, F, N), split, stream);
    // dM = du Wd
    if (st == ODA_OK)
      st = sgemm<true, false, kStore>(sg(fp(W.du), T, Wt(t0 + 3), F, fp(W.dM), F, N, F, T), 1, split, stream);
    hipLaunchKernelGGL(k_swiglu_bwd, dim3(F / 256, N), dim3(256), 0, stream, fp(GU[k]), fp(W.dM), fp(W.dGU));
    // d[Wg; Wu] = dGU^T r
    if (st == ODA_OK)
      st = sgemm<false, false, kStore>(sg(fp(W.dGU), 2 * F, fp(rr[k]), T, Gt(t0 + 1), T, 2 * F, T, N),
                                       wgrad_splits(2 * F, T, N), split, stream);
    // dr = dGU [Wg; Wu]
    if (st == ODA_OK)
      st = sgemm<true, false, kStore>(sg(fp(W.dGU), 2 * F, Wt(t0 + 1), T, fp(W.dr), T, N, T, 2 * F), 1, split,
                                      stream);
    // dgamma_k = sum dr uhat; du += norm backward of dr
    colsum(fp(W.dr), fp(uh[k]), nullptr, N, T, nullptr, Gt(t0), colp, stream);
    hipLaunchKernelGGL(k_rownorm_bwd, dim3(N), dim3(256), 0, stream, fp(W.dr), fp(uin[k]), Wt(t0), fp(W.du));
  }

  // ---- interaction (du now holds dL/du0) ----
  if (st == ODA_OK)
    st = sgemm<false, false, kStore>(sg(fp(W.du), T, fp(W.Z), 9 * T, Gt(9), 9 * T, T, 9 * T, N),
                                     wgrad_splits(T, 9 * T, N), split, stream);
  colsum(fp(W.du), nullptr, nullptr, N, T, nullptr, Gt(10), colp, stream);
  if (st == ODA_OK)
    st = sgemm<true, false, kStore>(sg(fp(W.du), T, Wt(9), 9 * T, fp(W.Z), 9 * T, N, 9 * T, T), 1, split, stream);
  hipLaunchKernelGGL(k_interact_bwd, dim3(T / 256, N), dim3(256), 0, stream, fp(W.du), fp(W.Z), fp(W.act),
                     fp(W.pre), fp(W.dpre), N);

  // ---- towers ----
  for (int s = 0; s < 3 && st == ODA_OK; ++s) {
    const float* dpre = fp(W.dpre) + s * NT;
    st = sgemm<false, false, kStore>(sg(dpre, T, fp(W.xn) + s * ND, D, Gt(3 * s + 1), D, T, D, N),
                                     wgrad_splits(T, D, N), split, stream);
    colsum(dpre, nullptr, nullptr, N, T, nullptr, Gt(3 * s + 2), colp, stream);
    if (st == ODA_OK)
      st = sgemm<true, false, kStore>(sg(dpre, T, Wt(3 * s + 1), D, fp(W.dxn), D, N, D, T), 1, split, stream);
    colsum(fp(W.dxn), fp(W.xhat) + s * ND, nullptr, N, D, nullptr, Gt(3 * s), colp, stream);
  }
  if (st != ODA_OK) return st;
  return hipGetLastError() == hipSuccess ? ODA_OK : ODA_E_LAUNCH;
}

}  // extern "C"
