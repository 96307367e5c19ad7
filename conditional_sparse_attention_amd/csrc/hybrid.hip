// Recurrent layers of a hybrid backbone around the ODA path, for gfx950: one
// gated delta rule decode step per (sequence, head), and the transaction
// that keeps both branches on the same pre-step state [On-Demand Attention
// notes §2.3 state commit, §3.3].  oda_hybrid.h states the layer and the
// slot scheme.
//
// A step is HBM-bound: each (sequence, head) reads its 128 x 128 fp32 state
// (64 KB) from the committed slot and writes the updated one to the branch's
// slot, 2 x 64 KB per head and layer, plus a few hundred bytes of inputs.
// The grid is (4 row blocks, H, B).  A workgroup loads its channels'
// convolution inputs, then issues the loads of its 32 state rows, rebuilds
// the head's q^, k^, v in LDS while those are in flight (convolution, SiLU;
// the row block 0 workgroup also writes the new convolution state; every
// wave reduces the two L2 norms itself), then updates the rows: 16 lanes per
// row, 8 floats per lane, the row's two dot products summed over the 16
// lanes with DPP row operations.  The commit moves a per-sequence slot index; no state is
// copied.
#include <math.h>

#include "oda_hybrid.h"
#include "oda_internal.h"

namespace oda {
namespace {

constexpr int kD = 128;          // d_k = d_v
constexpr int kRowBlocks = 4;    // workgroups per (sequence, head): 4 beat 8 and 2 on the hybrid step
constexpr int kRowsPerBlock = kD / kRowBlocks;
constexpr float kNormEps = 1e-6f;

struct GdnArgs {
  float* S;                  // recurrent pool [L][B][3][H][d][d]
  uint16_t* conv;            // convolution pool [L][B][3][W-1][C]
  const uint8_t* slot;
  const uint8_t* flag;
  const uint16_t* x;         // [B][C]
  const uint16_t* w;         // [C][W]
  const float* alpha;        // [B][H]
  const float* beta;
  uint16_t* out;             // [B][H][d]
  int32_t layer, B, H, W, C;
};

__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + expf(-x)); }

template <int BRANCH, int W>
__global__ void __launch_bounds__(256) k_gdn_step(GdnArgs a) {
  __shared__ float s_q[kD], s_k[kD], s_v[kD];
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  if (BRANCH == ODA_GDN_FULL && a.flag[b] == 0) return;
  const int c = a.slot[b] % 3, dst = (c + 1 + BRANCH) % 3;
  const int Hd = a.H * kD, C = a.C;
  const size_t lb = (size_t)a.layer * a.B + b;
  const uint16_t* cs = a.conv + (lb * 3 + c) * (size_t)(W - 1) * C;
  uint16_t* cd = a.conv + (lb * 3 + dst) * (size_t)(W - 1) * C;
  const uint16_t* xb = a.x + (size_t)b * C;
  const int wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, g = lane >> 4;
  const size_t head_off = (size_t)h * kD * kD;
  const float* Ss = a.S + (lb * 3 + c) * (size_t)a.H * kD * kD + head_off;
  float* Sd = a.S + (lb * 3 + dst) * (size_t)a.H * kD * kD + head_off;

  // 1. the convolution inputs of this thread's channels (ch = tid, tid + 256
  // of the head's 3 d: q, k, v), first, so that the convolution waits for
  // them alone
  uint16_t wv[2][W], sv[2][W - 1], xt[2];
  int ccs[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int ch = tid + 256 * u;
    const int chc = ch < 3 * kD ? ch : 0;
    const int cc = (chc / kD) * Hd + h * kD + chc % kD;
    ccs[u] = cc;
#pragma unroll
    for (int j = 0; j < W; ++j) wv[u][j] = a.w[(size_t)cc * W + j];
#pragma unroll
    for (int j = 0; j < W - 1; ++j) sv[u][j] = cs[(size_t)j * C + cc];
    xt[u] = xb[cc];
  }
  // 2. this workgroup's state rows: they do not depend on q, k, v, so their
  // latency overlaps the convolution
  constexpr int kPasses = kRowsPerBlock / 16;
  float4 rows[kPasses][2];
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int i = blk * kRowsPerBlock + pass * 16 + wave * 4 + g;
    const float4* src = reinterpret_cast<const float4*>(Ss + (size_t)i * kD + 8 * li);
    rows[pass][0] = src[0];
    rows[pass][1] = src[1];
  }
  // 3. convolution, SiLU; the row block 0 workgroup writes the new
  // convolution state (s_1, ..., s_{W-2}, x_t)
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int ch = tid + 256 * u;
    if (ch < 3 * kD) {
      const int grp = ch / kD, i = ch % kD, cc = ccs[u];
      float y = 0.0f;
#pragma unroll
      for (int j = 0; j < W - 1; ++j) y += bf16_to_f32(wv[u][j]) * bf16_to_f32(sv[u][j]);
      y += bf16_to_f32(wv[u][W - 1]) * bf16_to_f32(xt[u]);
      const float v = silu_f(y);
      if (grp == 0) s_q[i] = v;
      else if (grp == 1) s_k[i] = v;
      else s_v[i] = v;
      if (blk == 0) {
#pragma unroll
        for (int j = 0; j + 1 < W - 1; ++j) cd[(size_t)j * C + cc] = sv[u][j + 1];
        cd[(size_t)(W - 2) * C + cc] = xt[u];
      }
    }
  }
  __syncthreads();
  // |q|^2 and |k|^2 over the 128 LDS values, reduced by every wave itself
  float sq = s_q[lane] * s_q[lane] + s_q[lane + 64] * s_q[lane + 64];
  float sk = s_k[lane] * s_k[lane] + s_k[lane + 64] * s_k[lane + 64];
  sq = row16_sum(sq);
  sk = row16_sum(sk);
  sq = (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(sq), 0)) +
        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sq), 16))) +
       (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(sq), 32)) +
        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sq), 48)));
  sk = (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(sk), 0)) +
        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sk), 16))) +
       (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(sk), 32)) +
        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sk), 48)));
  const float rq = 1.0f / sqrtf(sq + kNormEps);
  const float rk = 1.0f / sqrtf(sk + kNormEps);

  // 4. rows of the state: lanes 16 g .. 16 g + 15 of a wave take one row,
  // lane li its columns 8 li .. 8 li + 7
  float qh[8], kh[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    qh[j] = s_q[8 * li + j] * rq;
    kh[j] = s_k[8 * li + j] * rk;
  }
  const float al = a.alpha[(size_t)b * a.H + h], be = a.beta[(size_t)b * a.H + h];
  const float inv_sqrt_d = 1.0f / sqrtf((float)kD);
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int i = blk * kRowsPerBlock + pass * 16 + wave * 4 + g;
    const float4 r0 = rows[pass][0], r1 = rows[pass][1];
    float s[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
    float u = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) u += s[j] * kh[j];
    u = row16_sum(u);
    const float coef = be * (s_v[i] - al * u);
    float o = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      s[j] = al * s[j] + coef * kh[j];
      o += s[j] * qh[j];
    }
    o = row16_sum(o);
    float4* d4 = reinterpret_cast<float4*>(Sd + (size_t)i * kD + 8 * li);
    d4[0] = make_float4(s[0], s[1], s[2], s[3]);
    d4[1] = make_float4(s[4], s[5], s[6], s[7]);
    if (li == 0) a.out[((size_t)b * a.H + h) * kD + i] = f32_to_bf16(o * inv_sqrt_d);
  }
}

template <int BRANCH>
int launch_gdn(const GdnArgs& a, dim3 grid, hipStream_t st) {
  switch (a.W) {
    case 2: hipLaunchKernelGGL((k_gdn_step<BRANCH, 2>), grid, dim3(256), 0, st, a); break;
    case 3: hipLaunchKernelGGL((k_gdn_step<BRANCH, 3>), grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_gdn_step<BRANCH, 4>), grid, dim3(256), 0, st, a); break;
    case 5: hipLaunchKernelGGL((k_gdn_step<BRANCH, 5>), grid, dim3(256), 0, st, a); break;
    case 6: hipLaunchKernelGGL((k_gdn_step<BRANCH, 6>), grid, dim3(256), 0, st, a); break;
    case 7: hipLaunchKernelGGL((k_gdn_step<BRANCH, 7>), grid, dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL((k_gdn_step<BRANCH, 8>), grid, dim3(256), 0, st, a); break;
    default: return ODA_E_UNSUPPORTED;
  }
  return ODA_OK;
}

__global__ void k_gdn_commit(uint8_t* slot, const uint8_t* flag, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) slot[b] = (uint8_t)((slot[b] % 3 + 1 + (flag[b] != 0 ? 1 : 0)) % 3);
}

bool gdn_dims_ok(const oda_gdn_dims* d) {
  return d != nullptr && d->num_layers >= 1 && d->batch >= 1 && d->batch <= 1024 && d->heads >= 1 &&
         d->heads <= 64 && d->head_dim == kD && d->conv_width >= 2 && d->conv_width <= 8;
}

size_t gdn_rec_bytes(const oda_gdn_dims* d) {
  return (size_t)d->num_layers * d->batch * ODA_GDN_SLOTS * d->heads * kD * kD * sizeof(float);
}

size_t gdn_conv_bytes(const oda_gdn_dims* d) {
  return (size_t)d->num_layers * d->batch * ODA_GDN_SLOTS * (d->conv_width - 1) * 3 * d->heads * kD * 2;
}

}  // namespace
}  // namespace oda

using namespace oda;

extern "C" {

size_t oda_gdn_state_bytes(const oda_gdn_dims* dims) {
  if (!gdn_dims_ok(dims)) return 0;
  return gdn_rec_bytes(dims) + gdn_conv_bytes(dims);
}

size_t oda_gdn_conv_offset(const oda_gdn_dims* dims) {
  if (!gdn_dims_ok(dims)) return 0;
  return gdn_rec_bytes(dims);
}

int oda_gdn_step(const oda_gdn_dims* dims, int32_t layer, int32_t branch, void* state, const uint8_t* slot,
                 const uint8_t* flag, const oda_bf16* x, const oda_bf16* conv_w, const float* alpha,
                 const float* beta, oda_bf16* out, hipStream_t stream) {
  if (dims == nullptr || state == nullptr || slot == nullptr || x == nullptr || conv_w == nullptr ||
      alpha == nullptr || beta == nullptr || out == nullptr)
    return ODA_E_NULL;
  if (!gdn_dims_ok(dims)) return ODA_E_DIMS;
  if (branch != ODA_GDN_LOCAL && branch != ODA_GDN_FULL) return ODA_E_DIMS;
  if (branch == ODA_GDN_FULL && flag == nullptr) return ODA_E_NULL;
  if (layer < 0 || layer >= dims->num_layers) return ODA_E_LAYER;
  if (((uintptr_t)state & 15) != 0) return ODA_E_DIMS;
  GdnArgs a;
  a.S = static_cast<float*>(state);
  a.conv = reinterpret_cast<uint16_t*>(static_cast<char*>(state) + gdn_rec_bytes(dims));
  a.slot = slot;
  a.flag = flag;
  a.x = x;
  a.w = conv_w;
  a.alpha = alpha;
  a.beta = beta;
  a.out = out;
  a.layer = layer;
  a.B = dims->batch;
  a.H = dims->heads;
  a.W = dims->conv_width;
  a.C = 3 * dims->heads * kD;
  dim3 grid(kRowBlocks, dims->heads, dims->batch);
  const int st = branch == ODA_GDN_LOCAL ? launch_gdn<ODA_GDN_LOCAL>(a, grid, stream)
                                         : launch_gdn<ODA_GDN_FULL>(a, grid, stream);
  if (st != ODA_OK) return st;
  return hipGetLastError() == hipSuccess ? ODA_OK : ODA_E_LAUNCH;
}

int oda_gdn_commit(const oda_gdn_dims* dims, uint8_t* slot, const uint8_t* flag, hipStream_t stream) {
  if (dims == nullptr || slot == nullptr || flag == nullptr) return ODA_E_NULL;
  if (!gdn_dims_ok(dims)) return ODA_E_DIMS;
  hipLaunchKernelGGL(k_gdn_commit, dim3((dims->batch + 255) / 256), dim3(256), 0, stream, slot, flag, dims->batch);
  return hipGetLastError() == hipSuccess ? ODA_OK : ODA_E_LAUNCH;
}

}  // extern "C"
