// Local-branch attention for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  The kernels are oda_local_attn's; their scratch (split
// partials, completion tickets, the header word) lives in a fixed device
// array of this library instead of a caller workspace.  Each GPU holds its
// own copy of the array until the process ends; calls on one GPU share it,
// so calls that overlap on one GPU race and must be ordered by the caller.
#include <mutex>

#include "oda_internal.h"
#include "abi_align.h"

namespace oda {
namespace {

constexpr size_t kScratchBytes = (size_t)ODA_NOALLOC_SCRATCH_BYTES;
constexpr size_t kHeaderBytes = 256;   // int32[64]: [0] error word when the caller passes none
constexpr int kMaxDevices = 64;

// Zero at code-object load; the tickets are cleared again at set-up and the
// kernels leave them cleared after every call.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
unsigned char* g_addr[kMaxDevices];  // device address of `scratch` per device, once set up

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Bytes of scratch a call with these dims uses: header, tickets [B * Hkv],
// partials [B * Hkv * kLocalMaxSplits * G * kPartStride] floats.
size_t scratch_need(const ::oda_dims* d, size_t* tick_off, size_t* part_off) {
  const size_t pairs = (size_t)d->batch * d->num_kv_heads;
  const size_t G = (size_t)(d->num_q_heads / d->num_kv_heads);
  *tick_off = kHeaderBytes;
  *part_off = align256(*tick_off + pairs * sizeof(int32_t));
  return *part_off + pairs * kLocalMaxSplits * G * kPartStride * sizeof(float);
}

// The device address of `scratch` on the current device; on the first call
// for a device it is looked up (hipGetSymbolAddress, with that device
// current) and the header and ticket region is cleared with a fill kernel on
// `s`.  Host code never uses the array's name as an address.
int scratch_address(unsigned char** out, hipStream_t s) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ODA_E_LAUNCH;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return ODA_E_LAUNCH;
    const size_t clear = align256(kHeaderBytes + (size_t)kMaxBatch * 1024 * sizeof(int32_t));
    const int st = launch_fill_zero(static_cast<int32_t*>(p), clear / sizeof(int32_t), s);
    if (st != ODA_OK) return st;
    g_addr[dev] = static_cast<unsigned char*>(p);
  }
  *out = g_addr[dev];
  return ODA_OK;
}

}  // namespace
}  // namespace oda

using namespace oda;

extern "C" int oda_local_attn_noalloc(const oda_dims* dims, int32_t layer, const oda_kv* kv, const int32_t* pos,
                                      const oda_bf16* q, const oda_bf16* k_cur, const oda_bf16* v_cur,
                                      oda_bf16* out, float* lse, int32_t* err, hipStream_t stream) {
  const int st = check_attn_operands(dims, layer, kv, pos, q, k_cur, v_cur, out);
  if (st != ODA_OK) return st;
  if (!aligned_to(lse, 4) || !aligned_to(err, 4)) return ODA_E_ALIGN;
  size_t tick_off, part_off;
  const size_t need = scratch_need(dims, &tick_off, &part_off);
  // the ticket region cleared at set-up covers up to kMaxBatch * 1024 pairs
  if (need > kScratchBytes || (size_t)dims->batch * dims->num_kv_heads > (size_t)kMaxBatch * 1024)
    return ODA_E_WORKSPACE;
  unsigned char* base = nullptr;
  const int sa = scratch_address(&base, stream);
  if (sa != ODA_OK) return sa;
  int32_t* header = reinterpret_cast<int32_t*>(base);
  AttnParams p = attn_params_at(dims, layer, kv, pos, q, k_cur, v_cur, out, lse,
                                reinterpret_cast<float*>(base + part_off), reinterpret_cast<int32_t*>(base + tick_off),
                                header, nullptr);
  if (err != nullptr) p.err = err;
  return launch_local_attn(p, dims->num_q_heads / dims->num_kv_heads, dims->kv_layout == ODA_KV_PAGED, stream);
}
