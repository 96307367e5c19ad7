// Commit of the chosen branch, the local-range query and workspace fill.
//
// Commit  [On-Demand Attention notes §2.3, equation h_t = h_t^{b_t},
// C_t = C_{t-1} || dC_t^{b_t}]: every layer's slot pos[b] receives the staged
// K/V of the branch chosen for b, h_prev[b] receives that branch's last-layer
// output, and pos[b] advances by one.  Output and cache come from the same
// branch by construction: both are selected by the same flag[b].
//
// Grid (L, B): one workgroup copies one (layer, sequence) slot (Hkv rows of
// K and of V, 16-byte vector copies).  The workgroups of a sequence take a
// ticket after their copy; the last one (every other one has read pos[b]
// by then) copies the hidden state, advances pos[b] and clears the ticket.
#include "oda_internal.h"

namespace oda {
namespace {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads) k_commit(CommitParams P) {
  const int l = blockIdx.x, b = blockIdx.y;
  const int p = P.pos[b];
  if (p < 0 || (int64_t)p >= P.t_max) {
    if (l == 0 && threadIdx.x == 0) atomicOr(P.err, ODA_ERR_CAPACITY);
    return;
  }
  size_t row_base;  // element offset of row (g = 0) of the slot inside layer l
  size_t g_stride;
  if (P.tables == nullptr) {
    row_base = ((size_t)b * P.Hkv * (size_t)P.t_cap + (size_t)p) * kHeadDim;
    g_stride = (size_t)P.t_cap * kHeadDim;
  } else {
    const int32_t blk = P.tables[(size_t)b * P.max_blocks + (p >> P.log2_block)];
    if (blk < 0 || (int64_t)blk >= P.num_blocks) {
      if (l == 0 && threadIdx.x == 0) atomicOr(P.err, ODA_ERR_BLOCK);
      return;
    }
    row_base = ((((size_t)blk * P.Hkv) << P.log2_block) | (size_t)(p & ((1 << P.log2_block) - 1))) * kHeadDim;
    g_stride = ((size_t)1 << P.log2_block) * kHeadDim;
  }
  const bool full = P.flag[b] != 0;
  const uint16_t* sk = full ? P.kF : P.kL;
  const uint16_t* sv = full ? P.vF : P.vL;
  const size_t src_base = ((size_t)l * P.B + b) * P.Hkv * kHeadDim;
  const size_t dst_layer = (size_t)l * P.layer_stride;
  const int per = P.Hkv * (kHeadDim / 8);  // 16-byte chunks per K (or V) slot
  for (int i = threadIdx.x; i < 2 * per; i += kThreads) {
    const int which = i / per;
    const int j = i % per;
    const int g = j / (kHeadDim / 8);
    const int c = j % (kHeadDim / 8);
    const uint16_t* src = (which ? sv : sk) + src_base + (size_t)g * kHeadDim + c * 8;
    uint16_t* dst = (which ? P.V : P.K) + dst_layer + row_base + (size_t)g * g_stride + c * 8;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }
  // The ticket only orders this workgroup's read of pos[b] (already
  // complete: every store above used it) before the last workgroup's
  // increment.  The copied slots and h_prev are read by later kernels only,
  // so no device-wide fence is needed.
  __syncthreads();
  __shared__ int s_last;
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(P.tickets + b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == P.L - 1;
  __syncthreads();
  if (!s_last) return;
  const uint16_t* so = (full ? P.oF : P.oL) + (size_t)b * P.D;
  uint16_t* dh = P.h_prev + (size_t)b * P.D;
  for (int i = threadIdx.x; i < P.D / 8; i += kThreads)
    reinterpret_cast<uint4*>(dh)[i] = reinterpret_cast<const uint4*>(so)[i];
  __syncthreads();
  if (threadIdx.x == 0) {
    P.pos[b] = p + 1;
    __hip_atomic_store(P.tickets + b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__global__ void k_ranges(const int32_t* pos, int32_t* ranges, int B, int sink, int window) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int32_t t = pos[b] + 1;
  const LocalSet S = local_set(t > 0 ? t : 0, sink, window);
  ranges[4 * b + 0] = 0;
  ranges[4 * b + 1] = S.n0;
  ranges[4 * b + 2] = S.s1;
  ranges[4 * b + 3] = S.t;
}

__global__ void k_fill_zero(int32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

}  // namespace

int launch_commit(const CommitParams& p, hipStream_t s) {
  hipLaunchKernelGGL(k_commit, dim3(p.L, p.B), dim3(kThreads), 0, s, p);
  return hipGetLastError() == hipSuccess ? ODA_OK : ODA_E_LAUNCH;
}

int launch_ranges(const int32_t* pos, int32_t* ranges, int B, int sink, int window, hipStream_t s) {
  hipLaunchKernelGGL(k_ranges, dim3(1), dim3(64), 0, s, pos, ranges, B, sink, window);
  return hipGetLastError() == hipSuccess ? ODA_OK : ODA_E_LAUNCH;
}

int launch_fill_zero(int32_t* p, size_t n, hipStream_t s) {
  size_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  if (blocks == 0) return ODA_OK;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return hipGetLastError() == hipSuccess ? ODA_OK : ODA_E_LAUNCH;
}

}  // namespace oda
