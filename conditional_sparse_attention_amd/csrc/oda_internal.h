// Internal declarations of liboda: workspace layout, launch parameter
// blocks and small device helpers shared by the kernels.  Written for gfx950
// (CDNA4): 64-wide wavefronts, DPP row operations, v_dot2_f32_bf16.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "oda.h"

namespace oda {

constexpr int kHeadDim = 128;
constexpr int kMaxBatch = 32;
constexpr int kLocalMaxSplits = 16;    // splits of one (sequence, KV head) in the local branch
constexpr int kLocalMinChunk = 64;     // fewer keys than this per split is not worth a split
constexpr int kPartStride = 132;       // floats per partial: acc[128], m, l, 2 pad (16-B aligned)
constexpr int kTower = ODA_HEAD_TOWER;
constexpr int kFfn = ODA_HEAD_FFN;
constexpr int kFullMinChunk = ODA_FULL_MIN_CHUNK;
constexpr int kFullFineChunk = ODA_FULL_FINE_CHUNK;
constexpr int kFullFillUnits = ODA_FULL_FILL_UNITS;
constexpr int kFullRoundUnits = ODA_FULL_ROUND_UNITS;
constexpr int kFullMaxSplits = ODA_FULL_MAX_SPLITS;
constexpr int kFullRaggedRounds = ODA_FULL_RAGGED_ROUNDS;
constexpr int kFullUnitCostKeys = ODA_FULL_UNIT_COST_KEYS;

// ---------------------------------------------------------------------------
// workspace layout (byte offsets, each region 256-B aligned)
// ---------------------------------------------------------------------------
struct WsLayout {
  size_t header;       // int32[64]: [0] error bits, [1] [2] the full kernel's unit queue and exit count
  size_t worklist;     // int32 count, then int32 items[B * kFullMaxSplits]
  size_t tick_local;   // int32[B * Hkv]
  size_t tick_full;    // int32[B * Hkv]
  size_t tick_commit;  // int32[B]
  size_t tick_head;    // int32[kHeadTickets] (dense-batch head GEMM, head_internal.h)
  size_t part_local;   // float[B * Hkv * kLocalMaxSplits * G * kPartStride]
  size_t part_full;    // float[B * Hkv * kFullMaxSplits * G * kPartStride]
  size_t head;         // float: head activations (HeadWs, head_internal.h)
  size_t total;
  int64_t t_max;            // capacity of one sequence in positions
};

// Candidate A of the full branch's split policy (one round) for a sequence
// of t keys when nflag sequences with hkv KV heads each are flagged, holding
// `total` keys together: chunks of kFullMinChunk keys or more, cut finer (not
// below kFullFineChunk keys) while the launch would hold fewer than
// kFullFillUnits units; and at most the sequence's share of one round of
// kFullRoundUnits units in proportion to its length, floor(kFullRoundUnits
// t / (total hkv)), but at least 1.  Every split is non-empty: (n - 1)^2 < t
// for n <= ceil(t / 256).
__device__ __host__ __forceinline__ int full_nsplit_round(int t, int nflag, int hkv, int64_t total) {
  int n = (t + kFullMinChunk - 1) / kFullMinChunk;
  n = n < kFullMaxSplits ? n : kFullMaxSplits;
  const int per = nflag * hkv;
  int fine = per > 0 ? kFullFillUnits / per : 0;
  const int by_chunk = (t + kFullFineChunk - 1) / kFullFineChunk;
  fine = fine < by_chunk ? fine : by_chunk;
  fine = fine < kFullMaxSplits ? fine : kFullMaxSplits;
  n = n > fine ? n : fine;
  if (per > 0 && total > 0) {
    const int64_t share = ((int64_t)kFullRoundUnits * t) / (total * hkv);
    const int cap = share < 1 ? 1 : (share > kFullMaxSplits ? kFullMaxSplits : (int)share);
    n = n < cap ? n : cap;
  }
  return n;
}

// Candidate B (several rounds of smaller units): chunks of
// max(kFullMinChunk, ceil(total hkv / (kFullRaggedRounds kFullRoundUnits)))
// keys, at most kFullMaxSplits splits.
__device__ __host__ __forceinline__ int full_nsplit_rounds(int t, int hkv, int64_t total) {
  const int64_t units = (int64_t)kFullRaggedRounds * kFullRoundUnits;
  int64_t c = (total * hkv + units - 1) / units;
  c = c > kFullMinChunk ? c : kFullMinChunk;
  const int64_t n = (t + c - 1) / c;
  return n < 1 ? 1 : (n > kFullMaxSplits ? kFullMaxSplits : (int)n);
}

// Estimated time of a candidate cut, in keys: with N units whose longest is
// U and shortest u over a grid of kFullRoundUnits workgroups (largest units
// first), the smaller of two estimates, ceil(N / grid) rounds of the longest
// unit, and the even share of all keys plus one shortest unit when units
// remain after the first round (never below U); each round adds a unit's
// fixed cost.
__device__ __host__ __forceinline__ int64_t full_split_cost(int64_t units, int64_t longest, int64_t shortest,
                                                            int64_t total, int hkv) {
  const int64_t rounds = (units + kFullRoundUnits - 1) / kFullRoundUnits;
  const int64_t by_rounds = rounds * (longest + kFullUnitCostKeys);
  int64_t even = (total * hkv + kFullRoundUnits - 1) / kFullRoundUnits + (units > kFullRoundUnits ? shortest : 0);
  even = (even > longest ? even : longest) + rounds * kFullUnitCostKeys;
  return by_rounds < even ? by_rounds : even;
}

// Work-list items: (b << 20) | (nsplit << 10) | split.
__device__ __host__ __forceinline__ int32_t full_item(int b, int ns, int s) { return (b << 20) | (ns << 10) | s; }

bool dims_valid(const oda_dims* d, int* status);
WsLayout ws_layout(const oda_dims* d);

// ---------------------------------------------------------------------------
// attention launch parameters
// ---------------------------------------------------------------------------
struct AttnParams {
  const uint16_t* K;  // layer base of the cache
  const uint16_t* V;
  const int32_t* tables;
  int64_t t_cap;      // contiguous: row stride per (b, g)
  int64_t num_blocks;
  int32_t max_blocks;
  int32_t log2_block;
  const int32_t* pos;
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  uint16_t* out;
  float* lse;
  float* part;
  int32_t* tickets;
  int32_t* err;
  const int32_t* worklist;  // count at [0], items from [1]
  int32_t* queue;           // full branch: [0] next unit past the first round, [1] workgroups done (zero between launches)
  int32_t B, Hq, Hkv, sink, window;
  int64_t t_max;
  float scale_log2;         // log2(e) / sqrt(d)
  int32_t local_splits;     // local branch: workgroups per (sequence, KV head), set at launch
  // Decoder mode only (the local kernel's ROPE instantiation): q and kc point
  // at the raw projection rows [B][(Hq + 2 Hkv) d] (q heads, then k, then v),
  // the kernel applies the QK-norm (gains gq / gk, epsilon qk_eps) and RoPE
  // from the step's table rope [B][d/2][2] (cos, sin), and the workgroup
  // holding the current token writes the staged key / value [B][Hkv][d] to
  // k_stage / v_stage.
  const uint16_t* gq;
  const uint16_t* gk;
  const float* rope;
  uint16_t* k_stage;
  uint16_t* v_stage;
  float qk_eps;
};

// Attention parameters of one layer with the split partials, tickets, the
// header (error word, then the full kernel's queue counters) and the work
// list at the given device addresses.
AttnParams attn_params_at(const ::oda_dims* d, int32_t layer, const ::oda_kv* kv, const int32_t* pos,
                          const uint16_t* q, const uint16_t* kc, const uint16_t* vc, uint16_t* out, float* lse,
                          float* part, int32_t* tickets, int32_t* header, const int32_t* worklist);
// The argument checks every attention call makes (dims, non-NULL operands,
// block tables of a paged cache, layer range); ODA_OK or an error code.
int check_attn_operands(const ::oda_dims* d, int32_t layer, const ::oda_kv* kv, const int32_t* pos,
                        const uint16_t* q, const uint16_t* kc, const uint16_t* vc, const uint16_t* out);

int launch_local_attn(const AttnParams& p, int G, bool paged, hipStream_t s, bool rope = false);
int launch_full_attn(const AttnParams& p, int G, bool paged, hipStream_t s);

// The decoder's local attention call: the ODA local branch of one layer in
// decoder mode (see AttnParams).  Checks its arguments as oda_local_attn does.
int decoder_local_attn(const ::oda_dims* d, int32_t layer, const ::oda_kv* kv, const int32_t* pos,
                       const uint16_t* qkv, const uint16_t* gq, const uint16_t* gk, const float* rope, float qk_eps,
                       uint16_t* k_stage, uint16_t* v_stage, uint16_t* out, void* ws, size_t ws_bytes,
                       hipStream_t s);

// ---------------------------------------------------------------------------
// commit / ranges / init
// ---------------------------------------------------------------------------
struct CommitParams {
  uint16_t* K;
  uint16_t* V;
  const int32_t* tables;
  int64_t t_cap, num_blocks, layer_stride;  // elements per layer of the cache
  int32_t max_blocks, log2_block;
  int32_t* pos;
  const uint8_t* flag;
  const uint16_t *kL, *vL, *kF, *vF;
  const uint16_t *oL, *oF;
  uint16_t* h_prev;
  int32_t* tickets;
  int32_t* err;
  int32_t L, B, Hkv, D;
  int64_t t_max;
};
int launch_commit(const CommitParams& p, hipStream_t s);
int launch_ranges(const int32_t* pos, int32_t* ranges, int B, int sink, int window, hipStream_t s);
int launch_fill_zero(int32_t* p, size_t n, hipStream_t s);

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// round-to-nearest-even fp32 -> bf16 (NaN kept quiet)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// DPP move within a 16-lane row (compile-time control word).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the same bits.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);  // row_half_mirror
  x += dpp_mov<0x140>(x);  // row_mirror
  return x;
}

// Local index set S^L of a sequence whose current 0-based position is t-1:
// [0, n0) followed by [s1, t) (s1 >= n0); n0 == t when the parts touch.
struct LocalSet {
  int32_t n0;   // length of the first range [0, n0)
  int32_t s1;   // start of the second range
  int32_t t;    // end of the second range (exclusive) = current position + 1
  __device__ __host__ int32_t size() const { return n0 + (t - s1); }
};
__device__ __host__ __forceinline__ LocalSet local_set(int32_t t, int32_t sink, int32_t window) {
  LocalSet r;
  int32_t a1 = sink < t ? sink : t;
  int32_t b0 = t - window > 0 ? t - window : 0;
  if (b0 <= a1) {
    r.n0 = t;
    r.s1 = t;
  } else {
    r.n0 = a1;
    r.s1 = b0;
  }
  r.t = t;
  return r;
}

}  // namespace oda
