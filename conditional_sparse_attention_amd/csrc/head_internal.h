// Internal declarations of the recall head: workspace sub-regions, launch
// parameters and the wave reduction its kernels share.
#pragma once

#include "oda_internal.h"

namespace oda {

// head activation sub-regions (float offsets inside WsLayout::head)
constexpr int kHeadTickets = 256;
// Batches from here on take the dense (MFMA) head path.  The GEMV's cost
// grows with every batch row it sweeps, the MFMA path's does not up to 16
// columns; measured at D = 1024 to 4096 they cross between 6 and 8 sequences
// (GEMV 53.5 / 56.6 us against 61.3 / 61.5 us at 5 / 6 sequences, D = 2048;
// 63.1 against 61.9 us at 8).
constexpr int kHeadDenseMin = 7;
struct HeadWs {
  float* towers;  // [3][B][T]  (a, b, c)
  float* u0;      // [B][T]
  float* hdn;     // [B][F]
  float* u1;      // [B][T]
  float* u2;      // [B][T]
  float* part;    // split-K partial tiles of the dense path (B >= kHeadDenseMin)
};
// floats of split-K partial tiles the dense head GEMMs need (largest layer)
size_t dense_head_part_floats(int B, int D);
inline size_t head_ws_floats(int B, int D) {
  size_t n = (size_t)B * (3 * kTower + kTower + kFfn + 2 * kTower);
  if (B >= kHeadDenseMin) n += dense_head_part_floats(B, D);
  return n;
}
inline HeadWs head_ws(void* ws, const WsLayout& L, int B, int D) {
  float* base = reinterpret_cast<float*>(static_cast<char*>(ws) + L.head);
  HeadWs h;
  h.towers = base;
  h.u0 = h.towers + 3 * B * kTower;
  h.hdn = h.u0 + B * kTower;
  h.u1 = h.hdn + B * kFfn;
  h.u2 = h.u1 + B * kTower;
  h.part = h.u2 + B * kTower;
  return h;
}

// ---------------------------------------------------------------------------
// recall head launch parameters
// ---------------------------------------------------------------------------
struct HeadParams {
  const float* w;          // packed blob
  const int64_t* offs;     // unused on device; host-side offsets
  const uint16_t* h_prev;
  const uint16_t* emb;
  const uint16_t* h_local;
  float theta;
  const int8_t* force;
  const int32_t* pos;
  float* score;
  uint8_t* flag;
  int32_t* worklist;
  int32_t* tickets;   // kHeadTickets, zero between calls
  int32_t B, D;
  int32_t Hkv;        // KV heads of the attention layers (split policy)
  HeadWs act;
};
int launch_recall_head(const HeadParams& p, const int64_t* offs, hipStream_t s);
int launch_worklist(const uint8_t* flag, const int32_t* pos, int32_t* worklist, int B, int Hkv, hipStream_t s);

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------
// Sum over the 64 lanes of a wave, identical (wave-uniform) in every lane:
// row sums by DPP, then the four row results read out and added in fixed order.
__device__ __forceinline__ float wave_sum64(float x) {
  x = row16_sum(x);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return (r0 + r1) + (r2 + r3);
}

}  // namespace oda
