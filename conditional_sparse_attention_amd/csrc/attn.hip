// Split-K GQA decode attention over an index set, for gfx950.
//
// Computes o = softmax(q K~[S]^T / sqrt(d)) V~[S] for every query head of a
// KV group  [On-Demand Attention notes §2.1, equation for o_t], where K~, V~
// are the committed cache rows followed by the branch's staged current row,
// and S is either the local set S^L (sink + window, §2.1) or the full set
// S^F = [0, t).
//
// Work unit: (sequence b, KV head g, split) -- a contiguous run of the index
// set.  One workgroup of NW waves processes a unit:
//   * lane layout: a 256-byte bf16 row (d = 128) is read by 16 lanes with one
//     16-byte load each, so one wave instruction reads 4 whole rows (1 KB,
//     fully coalesced); each lane handles 8 dims of its row;
//   * q.k uses v_dot2_f32_bf16 on the raw bf16 pairs, and the 16 partial dot
//     products of a row are summed with four DPP row operations
//     (quad_perm x2, row_half_mirror, row_mirror), which leave the bit-same
//     sum in all 16 lanes;
//   * online softmax in the log2 domain (scores pre-multiplied by
//     log2(e)/sqrt(d)), fp32 running max / sum / accumulator per row group,
//     one rescale per block of UNROLL rows;
//   * the 4 row groups of a wave merge through cross-lane shuffles, the NW
//     waves through LDS.
// A unit that covers its whole (b, g) writes the output directly; otherwise
// it stores a partial (acc[128], m, l) and takes a ticket; the last unit of a
// (b, g) merges all partials in split order (deterministic: no float
// atomics) and resets the ticket.
//
// The local kernel runs on a grid (split, g, b).  The full kernel runs on a
// fixed persistent grid whose workgroups walk the device-side work list
// written by the recall-score step, so the host never learns which
// sequences were flagged.
#include <atomic>

#include "oda_internal.h"

namespace oda {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned v4u_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const v4u_t gv4_t;

#ifndef ODA_LOCAL_DEPTH
#define ODA_LOCAL_DEPTH 2
#endif
#ifndef ODA_FULL_DEPTH
#define ODA_FULL_DEPTH 3
#endif
// Workgroups per (sequence, KV head) in the local branch, between these
// bounds (see local_splits()).
constexpr int kLocalSplitsMin = 1;
constexpr int kLocalSplitsMax = 8;
constexpr int kLocalSplitsMaxPaged = 16;  // a paged walk still gains at one sequence
// Waves per workgroup of the local kernel: kLocalWaves, or kLocalWavesWide
// when a (sequence, KV head) is cut into at most kLocalWideMax splits (each
// workgroup then streams a larger share alone).
constexpr int kLocalWaves = 4;
constexpr int kLocalWavesWide = 8;
constexpr int kLocalWideMax = 2;
#ifndef ODA_FULL_WAVES_SMALL_G
#define ODA_FULL_WAVES_SMALL_G 12
#endif

// Row blocks per lane per pipeline stage (a stage is 4*U rows of a wave).
// Two stages are in flight: the next block's loads are issued before the
// current block is consumed.
#ifndef ODA_LOCAL_U
#define ODA_LOCAL_U 2
#endif
#ifndef ODA_FULL_U
#define ODA_FULL_U 2
#endif
// Full kernel shape per group size: G = 2 (the 16/8-head models) runs 12
// waves (3 per SIMD) with a 3-stage ring; G = 4 keeps twice the query and
// accumulator state per lane and runs 12 waves with a 2-stage ring (165
// registers: 4.6-5.9% faster per launch than 8 waves with 4 stages at 8
// flagged 64K sequences, e.g. 355.9 / 372.9 us at 16 x 64K, the same at 2-4
// flagged; 3 stages spill at 12 waves); G = 1 runs 8 waves with a 4-stage
// ring.  The paged layout holds more per row in flight (a block and an
// address), so its rings are a stage shorter (G = 2: 2 stages; a 3-stage
// ring spills at 12 waves and measured slower at 8), and G = 2 runs 8 waves
// there: 1-4% faster per launch than 12 (e.g. 27.1 / 28.2 us at 8 flagged 4K
// sequences of 32, 88.4 / 89.7 us at one flagged 128K sequence).
template <int G, bool PAGED>
struct FullWaves {
  static constexpr int value = G == 2 ? (PAGED ? 8 : ODA_FULL_WAVES_SMALL_G) : (G == 4 && !PAGED ? 12 : 8);
};
template <int G, bool PAGED>
struct FullDepth {
  static constexpr int value = PAGED ? (G == 2 ? 2 : 3) : (G == 2 ? ODA_FULL_DEPTH : (G == 4 ? 2 : 4));
};

__device__ __forceinline__ float dot8_bf16(const uint4 a, const uint4 b) {
  float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x),
                                            __builtin_bit_cast(bf16x2_t, b.x), 0.0f, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y),
                                      __builtin_bit_cast(bf16x2_t, b.y), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z),
                                      __builtin_bit_cast(bf16x2_t, b.z), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w),
                                      __builtin_bit_cast(bf16x2_t, b.w), s, false);
  return s;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kNegBig = -1.0e30f;

template <int G>
struct State {
  float m[G];
  float l[G];
  float acc[G][8];
};

// Row index of cache row p of (b, g) (times kHeadDim: its element offset).
// In the paged layout the block comes from the workgroup's copy of the
// block-table entries in LDS (tab[i] = entry blk0 + i of the sequence's
// row); an entry outside the pool marks the row invalid (ok = false) and
// yields a safe address.
template <bool PAGED>
__device__ __forceinline__ size_t row_index(const AttnParams& P, int b, int g, int p, const int32_t* tab, int blk0,
                                            bool& ok) {
  if (!PAGED) {
    return ((size_t)(b * P.Hkv + g) * (size_t)P.t_cap + (size_t)p);
  } else {
    int32_t blk = tab[(p >> P.log2_block) - blk0];
    if (blk < 0 || (int64_t)blk >= P.num_blocks) {
      ok = false;
      blk = 0;
    }
    return ((((size_t)blk * P.Hkv + g) << P.log2_block) | (size_t)(p & ((1 << P.log2_block) - 1)));
  }
}

template <int G, int kUnroll>
__device__ __forceinline__ void block_update(const uint4 (&qv)[G], State<G>& st, const uint4 (&kk)[kUnroll],
                                             const uint4 (&vv)[kUnroll], const bool (&ok)[kUnroll],
                                             float scale) {
  // scores of the kUnroll rows of this lane's row group, log2 domain
  float s[kUnroll][G];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float x = row16_sum(dot8_bf16(qv[h], kk[u])) * scale;
      s[u][h] = ok[u] ? x : -INFINITY;
    }
  }
  // one rescale per block; s[][] becomes the unnormalised weights p
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = s[0][h];
#pragma unroll
    for (int u = 1; u < kUnroll; ++u) mx = fmaxf(mx, s[u][h]);
    const float mn = fmaxf(st.m[h], mx);
    const float alpha = fast_exp2(st.m[h] - mn);
    st.m[h] = mn;
    st.l[h] *= alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) st.acc[h][i] *= alpha;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      s[u][h] = fast_exp2(s[u][h] - mn);
      st.l[h] += s[u][h];
    }
  }
  // p * v, one row's 8 values converted at a time
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    float vf[8];
    vf[0] = bf16lo(vv[u].x);
    vf[1] = bf16hi(vv[u].x);
    vf[2] = bf16lo(vv[u].y);
    vf[3] = bf16hi(vv[u].y);
    vf[4] = bf16lo(vv[u].z);
    vf[5] = bf16hi(vv[u].z);
    vf[6] = bf16lo(vv[u].w);
    vf[7] = bf16hi(vv[u].w);
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int i = 0; i < 8; ++i) st.acc[h][i] = fmaf(s[u][h], vf[i], st.acc[h][i]);
    }
  }
}

__device__ __forceinline__ uint4 load_stream(const uint16_t* p) {
  // streamed once: non-temporal global load (keeps L2 / MALL for reused data)
  const v4u_t x = __builtin_nontemporal_load((gv4_t*)(p));
  return make_uint4(x.x, x.y, x.z, x.w);
}

// Loads one pipeline stage: rows base + u*4 + r (u < U) of this lane's row
// group, clamped to p_hi - 1 and marked invalid beyond it.
template <bool PAGED, int U>
__device__ __forceinline__ void load_stage(const AttnParams& P, const uint16_t* Kbg, const uint16_t* Vbg, int b,
                                           int g, int base, int p_hi, int r, int c, const int32_t* tab, int blk0,
                                           uint4 (&kk)[U], uint4 (&vv)[U], bool (&ok)[U]) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int p = base + u * 4 + r;
    bool valid = p < p_hi;
    const int pp = valid ? p : p_hi - 1;
    size_t off;
    if (!PAGED) {
      off = (size_t)pp * kHeadDim;
    } else {
      bool bok = true;
      off = row_index<true>(P, b, g, pp, tab, blk0, bok) * kHeadDim;
      if (!bok) {
        if (valid && c == 0) atomicOr(P.err, ODA_ERR_BLOCK);
        valid = false;
      }
    }
    ok[u] = valid;
    kk[u] = load_stream(Kbg + off + c * 8);
    vv[u] = load_stream(Vbg + off + c * 8);
  }
}

// Decoder mode: what a lane needs to form its q / k dims, loaded with the raw
// q rows before the cache stream starts: the two QK-norm gains (dims 8c ..
// 8c+7) and the step's (cos, sin) for the 8 angles of those dims.
struct RopeLane {
  uint4 gq, gk;
  uint4 cs[4];
};

__device__ __forceinline__ void rope_lane_load(const AttnParams& P, int b, int c, RopeLane& rl) {
  rl.gq = *reinterpret_cast<const uint4*>(P.gq + 8 * c);
  rl.gk = *reinterpret_cast<const uint4*>(P.gk + 8 * c);
  const uint4* t = reinterpret_cast<const uint4*>(P.rope + (size_t)b * kHeadDim + 16 * (c & 7));
#pragma unroll
  for (int j = 0; j < 4; ++j) rl.cs[j] = t[j];
}

// QK-norm and RoPE of one head vector held 8 dims per lane (lane c of a
// 16-lane row holds dims 8c .. 8c+7): y = gamma x / sqrt(mean(x^2) + eps),
// then each pair (i, i + d/2) rotated by the step's angle i: y_i cos -
// y_{i+d/2} sin and y_{i+d/2} cos + y_i sin; rounded to bf16.  The partner
// of a dim sits in lane c ^ 8.
__device__ __forceinline__ uint4 norm_rope8(const uint4 raw, const uint4 gr, const uint4 (&cs)[4], int c, float eps) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float x[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = bf16lo(w[j]);
    x[2 * j + 1] = bf16hi(w[j]);
  }
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) ss += x[j] * x[j];
  ss = row16_sum(ss);
  const float rs = rsqrtf(ss / (float)kHeadDim + eps);
  const uint32_t gw[4] = {gr.x, gr.y, gr.z, gr.w};
  float y[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    y[2 * j] = bf16lo(gw[j]) * x[2 * j] * rs;
    y[2 * j + 1] = bf16hi(gw[j]) * x[2 * j + 1] * rs;
  }
  float t[16];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    t[4 * j] = __uint_as_float(cs[j].x);
    t[4 * j + 1] = __uint_as_float(cs[j].y);
    t[4 * j + 2] = __uint_as_float(cs[j].z);
    t[4 * j + 3] = __uint_as_float(cs[j].w);
  }
  const bool first = c < 8;
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float v2[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int jj = 2 * j + e;
      const float partner = __shfl_xor(y[jj], 8, 64);
      const float co = t[2 * jj], si = t[2 * jj + 1];
      v2[e] = first ? y[jj] * co - partner * si : y[jj] * co + partner * si;
    }
    o[j] = (uint32_t)f32_to_bf16(v2[0]) | ((uint32_t)f32_to_bf16(v2[1]) << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Decoder mode: the G query heads of this lane, raw rows in, QK-normed and
// rotated rows out.
template <int G>
__device__ __forceinline__ void rope_q(const AttnParams& P, uint4 (&qv)[G], const RopeLane& rl, int c) {
#pragma unroll
  for (int h = 0; h < G; ++h) qv[h] = norm_rope8(qv[h], rl.gq, rl.cs, c, P.qk_eps);
}

// Shared memory of a workgroup, in floats: wg_merge needs NW*G*(128+2),
// merge_partials NW*64*6; while the cache rows stream, the same memory holds
// block-table entries of the paged layout.
template <int G, int NW>
constexpr int lds_floats() {
  constexpr int a = NW * G * (kHeadDim + 2);
  constexpr int b = 6 * NW * 64;
  return a > b ? a : b;
}

// Rows [p_lo, p_hi) of the cache.  Wave w takes stages starting at
// p_lo + (k*NW + w) * 4U.  A ring of DEPTH register stages keeps DEPTH-1
// stages in flight while one is consumed; its refill is issued right after.
template <int G, bool PAGED, int NW, int DEPTH, int U, bool ROPE>
__device__ __forceinline__ void stream_rows(const AttnParams& P, uint4 (&qv)[G], bool& q_ready, const RopeLane& rl,
                                            State<G>& st, int b, int g, int p_lo, int p_hi, int wave, int r, int c,
                                            const int32_t* tab, int blk0) {
  constexpr int kStage = 4 * U;
  constexpr int kStride = NW * kStage;
  const uint16_t* Kbg = P.K;
  const uint16_t* Vbg = P.V;
  if (!PAGED) {
    const size_t bg = ((size_t)b * P.Hkv + g) * (size_t)P.t_cap * kHeadDim;
    Kbg += bg;
    Vbg += bg;
  }
  const int first = p_lo + wave * kStage;
  if (first >= p_hi) return;
  uint4 kk[DEPTH][U], vv[DEPTH][U];
  bool ok[DEPTH][U];
  // This wave's stages are first + k * kStride for k < nst.  Every load is
  // unconditional (rows past p_hi are clamped to p_hi - 1 and masked), so the
  // same number of loads is outstanding at every wait and the wait before a
  // stage is consumed leaves the DEPTH - 1 stages after it in flight; the
  // scheduling barrier keeps each refill ahead of the next stage's arithmetic.
  const int nst = (p_hi - first + kStride - 1) / kStride;
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    load_stage<PAGED, U>(P, Kbg, Vbg, b, g, first + d * kStride, p_hi, r, c, tab, blk0, kk[d], vv[d], ok[d]);
  // decoder mode: the raw q rows were loaded first; form q while the ring fills
  if constexpr (ROPE) {
    if (!q_ready) {
      rope_q<G>(P, qv, rl, c);
      q_ready = true;
    }
  }
  int k = 0;
  for (; k + DEPTH <= nst; k += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      block_update<G, U>(qv, st, kk[d], vv[d], ok[d], P.scale_log2);
      load_stage<PAGED, U>(P, Kbg, Vbg, b, g, first + (k + d + DEPTH) * kStride, p_hi, r, c, tab, blk0, kk[d], vv[d],
                           ok[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const int rem = nst - k;
#pragma unroll
  for (int d = 0; d + 1 < DEPTH; ++d)
    if (d < rem) block_update<G, U>(qv, st, kk[d], vv[d], ok[d], P.scale_log2);
}

// Rows [p_lo, p_hi) of the cache, called by every thread of the workgroup.
// Paged layout: the block-table entries of the rows are first copied into
// the workgroup's shared memory (as many blocks at a time as it holds), so
// that a row's address needs no global load of its own: a table load would
// have to wait behind every cache load already in flight (the vector memory
// counter completes in order) and would drain the ring at each stage.
template <int G, bool PAGED, int NW, int DEPTH, int U, bool ROPE>
__device__ __forceinline__ void cache_rows(const AttnParams& P, uint4 (&qv)[G], bool& q_ready, const RopeLane& rl,
                                           State<G>& st, int b, int g, int p_lo, int p_hi, int wave, int r, int c,
                                           float* lds) {
  if constexpr (!PAGED) {
    stream_rows<G, PAGED, NW, DEPTH, U, ROPE>(P, qv, q_ready, rl, st, b, g, p_lo, p_hi, wave, r, c, nullptr, 0);
  } else {
    constexpr int kCap = lds_floats<G, NW>();  // table entries per window
    int32_t* tab = reinterpret_cast<int32_t*>(lds);
    const int lb = P.log2_block;
    const int32_t* row = P.tables + (size_t)b * P.max_blocks;
    for (int w_lo = p_lo; w_lo < p_hi;) {
      const int blk0 = w_lo >> lb;
      const int64_t w_end = ((int64_t)blk0 + kCap) << lb;
      const int w_hi = w_end < (int64_t)p_hi ? (int)w_end : p_hi;
      const int nblk = ((w_hi - 1) >> lb) - blk0 + 1;
      for (int i = threadIdx.x; i < nblk; i += NW * 64) tab[i] = row[blk0 + i];
      __syncthreads();
      stream_rows<G, PAGED, NW, DEPTH, U, ROPE>(P, qv, q_ready, rl, st, b, g, w_lo, w_hi, wave, r, c, tab, blk0);
      __syncthreads();  // every wave is done with this window's entries
      w_lo = w_hi;
    }
  }
}

// The current token: one staged row, handled by wave 0 / row group 0.  In
// decoder mode the row is formed here from the raw projection and written to
// the staging buffers, which the commit reads.
template <int G, bool ROPE>
__device__ __forceinline__ void current_row(const AttnParams& P, const uint4 (&qv)[G], const RopeLane& rl,
                                            State<G>& st, int b, int g, int wave, int r, int c) {
  if (wave != 0) return;
  uint4 kk[1], vv[1];
  bool ok[1];
  const size_t base = ((size_t)b * P.Hkv + g) * kHeadDim + c * 8;
  if constexpr (ROPE) {
    const size_t nh = (size_t)P.Hq + 2 * P.Hkv;
    const uint16_t* row = P.kc + (size_t)b * nh * kHeadDim + c * 8;
    kk[0] = norm_rope8(*reinterpret_cast<const uint4*>(row + ((size_t)P.Hq + g) * kHeadDim), rl.gk, rl.cs, c,
                       P.qk_eps);
    vv[0] = *reinterpret_cast<const uint4*>(row + ((size_t)P.Hq + P.Hkv + g) * kHeadDim);
    if (r == 0) {
      *reinterpret_cast<uint4*>(P.k_stage + base) = kk[0];
      *reinterpret_cast<uint4*>(P.v_stage + base) = vv[0];
    }
  } else {
    kk[0] = *reinterpret_cast<const uint4*>(P.kc + base);
    vv[0] = *reinterpret_cast<const uint4*>(P.vc + base);
  }
  ok[0] = (r == 0);
  block_update<G, 1>(qv, st, kk, vv, ok, P.scale_log2);
}

__device__ __forceinline__ float shfl_xor_f(float x, int m) { return __shfl_xor(x, m, 64); }

// Split hand-off.  The workgroups of one (b, g) may run on different XCDs,
// whose L2 caches are not coherent with each other, so partials never go
// through a cached path: they are stored and loaded with agent-scope atomic
// accesses.  On gfx950 those loads and stores carry the device-scope cache
// policy (sc1: coherent across the XCDs, not served from a stale L2 line),
// and atomic read-modify-writes at agent scope are device coherent.  The
// ordering argument, in hardware terms:
//  1. each thread's partial stores are issued, then s_waitcnt vmcnt(0) waits
//     until all of them are acknowledged (gfx9 counts stores in vmcnt, and a
//     device-scope store is acknowledged once it is visible device-wide);
//  2. a workgroup barrier, so every wave of the workgroup has passed 1;
//  3. one thread takes the ticket with a returning agent-scope atomic add
//     (performed at the coherence point; it is issued only after 2);
//  4. the workgroup that reads nsplit - 1 uses the returned value (so its
//     wave waited for the atomic to complete), publishes it through LDS and a
//     barrier, and only then issues its agent-scope loads of the partials.
// Every other workgroup's atomic preceded the last one's, and followed that
// workgroup's acknowledged stores, so the loads of 4 observe every partial.
// No float atomics: the merge adds the partials in split order.
__device__ __forceinline__ void part_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float part_load(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Takes the (b, g) ticket after this workgroup's partial is visible (steps 1
// to 4 above); returns true in the workgroup that completes the set.
__device__ __forceinline__ bool take_ticket(int32_t* ticket, int nsplit) {
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nsplit - 1;
  __syncthreads();
  return s_last;
}

__device__ __forceinline__ void reset_ticket(int32_t* ticket) {
  __hip_atomic_store(ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge the 4 row groups of each wave (shuffles), then the NW waves (LDS).
// On return, threads idx < G*128 hold (M, L, O) of (head idx/128, dim idx%128)
// for idx = tid (and tid + NW*64 when G*128 exceeds the block).
template <int G, int NW>
__device__ __forceinline__ void wg_merge(State<G>& st, float* lds, int wave, int lane, int c) {
  float* lacc = lds;                      // [NW][G][128]
  float* lml = lds + NW * G * kHeadDim;   // [NW][G][2]
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float M = fmaxf(st.m[h], shfl_xor_f(st.m[h], 16));
    M = fmaxf(M, shfl_xor_f(M, 32));
    const float sc = fast_exp2(st.m[h] - M);
    float l = st.l[h] * sc;
    l += shfl_xor_f(l, 16);
    l += shfl_xor_f(l, 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float a = st.acc[h][i] * sc;
      a += shfl_xor_f(a, 16);
      a += shfl_xor_f(a, 32);
      st.acc[h][i] = a;
    }
    if (lane < 16) {
      float4* dst = reinterpret_cast<float4*>(lacc + ((wave * G + h) * kHeadDim) + c * 8);
      dst[0] = make_float4(st.acc[h][0], st.acc[h][1], st.acc[h][2], st.acc[h][3]);
      dst[1] = make_float4(st.acc[h][4], st.acc[h][5], st.acc[h][6], st.acc[h][7]);
      if (lane == 0) {
        lml[(wave * G + h) * 2 + 0] = M;
        lml[(wave * G + h) * 2 + 1] = l;
      }
    }
  }
  __syncthreads();
}

// After wg_merge: value of (head h, dim dd) merged over the waves.
template <int G, int NW>
__device__ __forceinline__ void wg_value(const float* lds, int h, int dd, float& M, float& L, float& O) {
  const float* lacc = lds;
  const float* lml = lds + NW * G * kHeadDim;
  M = kNegBig;
#pragma unroll
  for (int w = 0; w < NW; ++w) M = fmaxf(M, lml[(w * G + h) * 2]);
  L = 0.0f;
  O = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float sc = fast_exp2(lml[(w * G + h) * 2] - M);
    L = fmaf(lml[(w * G + h) * 2 + 1], sc, L);
    O = fmaf(lacc[(w * G + h) * kHeadDim + dd], sc, O);
  }
}

__device__ __forceinline__ void write_out(const AttnParams& P, int b, int hq, int dd, float M, float L, float O) {
  const float v = L > 0.0f ? O / L : 0.0f;
  P.out[((size_t)b * P.Hq + hq) * kHeadDim + dd] = f32_to_bf16(v);
  if (P.lse != nullptr && dd == 0) {
    P.lse[(size_t)b * P.Hq + hq] = L > 0.0f ? (M + __log2f(L)) * 0.69314718055994531f : -INFINITY;
  }
}

// Final merge of nsplit (<= MAXS) partials of (b, g) by the last workgroup.
// Thread (group sg, head h, dims 4*d4..) issues all its coherent loads (m, l,
// acc of splits sg, sg + groups, ...) in one batch, merges them in split
// order, and the groups are then merged in group order through LDS, so the
// result does not depend on timing.
template <int G, int NW, int MAXS>
__device__ __forceinline__ void merge_partials(const AttnParams& P, const float* part, int nsplit, int b, int g,
                                               float* lds) {
  constexpr int NT = NW * 64;
  constexpr int kLanes = G * (kHeadDim / 4);  // (h, d4) pairs
  constexpr int kGroups = NT / kLanes;
  static_assert(kGroups >= 1 && kGroups * kLanes == NT, "block shape does not fit the merge");
  constexpr int kPer = (MAXS + kGroups - 1) / kGroups;
  const int tid = threadIdx.x;
  const int hd = tid % kLanes;
  const int sg = tid / kLanes;
  const int h = hd / (kHeadDim / 4);
  const int d4 = hd % (kHeadDim / 4);
  float m[kPer], l[kPer];
  float4 a[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int s = sg + k * kGroups;
    if (s < nsplit) {
      const float* pp = part + ((size_t)s * G + h) * kPartStride;
      m[k] = part_load(pp + kHeadDim);
      l[k] = part_load(pp + kHeadDim + 1);
      a[k] = make_float4(part_load(pp + d4 * 4), part_load(pp + d4 * 4 + 1), part_load(pp + d4 * 4 + 2),
                         part_load(pp + d4 * 4 + 3));
    } else {
      m[k] = kNegBig;
      l[k] = 0.0f;
      a[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  float M = kNegBig;
#pragma unroll
  for (int k = 0; k < kPer; ++k) M = fmaxf(M, m[k]);
  float L = 0.0f;
  float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const float w = fast_exp2(m[k] - M);
    L = fmaf(l[k], w, L);
    O.x = fmaf(a[k].x, w, O.x);
    O.y = fmaf(a[k].y, w, O.y);
    O.z = fmaf(a[k].z, w, O.z);
    O.w = fmaf(a[k].w, w, O.w);
  }
  float* red = lds;  // [kGroups][kLanes][6]
  __syncthreads();
  {
    float* r = red + ((size_t)sg * kLanes + hd) * 6;
    r[0] = M;
    r[1] = L;
    r[2] = O.x;
    r[3] = O.y;
    r[4] = O.z;
    r[5] = O.w;
  }
  __syncthreads();
  if (sg == 0) {
    float Mt = kNegBig;
    for (int k = 0; k < kGroups; ++k) Mt = fmaxf(Mt, red[((size_t)k * kLanes + hd) * 6]);
    float Lt = 0.0f;
    float4 Ot = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < kGroups; ++k) {
      const float* r = red + ((size_t)k * kLanes + hd) * 6;
      const float w = fast_exp2(r[0] - Mt);
      Lt = fmaf(r[1], w, Lt);
      Ot.x = fmaf(r[2], w, Ot.x);
      Ot.y = fmaf(r[3], w, Ot.y);
      Ot.z = fmaf(r[4], w, Ot.z);
      Ot.w = fmaf(r[5], w, Ot.w);
    }
    const int hq = g * G + h;
    write_out(P, b, hq, d4 * 4 + 0, Mt, Lt, Ot.x);
    write_out(P, b, hq, d4 * 4 + 1, Mt, Lt, Ot.y);
    write_out(P, b, hq, d4 * 4 + 2, Mt, Lt, Ot.z);
    write_out(P, b, hq, d4 * 4 + 3, Mt, Lt, Ot.w);
  }
}

// One unit: keys of S with virtual indices [v_lo, v_hi) where S = [0, n0)
// followed by [s1, t); the last virtual index (n0 + t - s1 - 1) is the
// current token and is read from staging.
template <int G, bool PAGED, int NW, int DEPTH, int U, int MAXS, bool ROPE>
__device__ void attn_unit(const AttnParams& P, int b, int g, int split, int nsplit, int v_lo, int v_hi,
                          const LocalSet& S, int32_t* ticket, float* part_bg, float* lds) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r = lane >> 4;
  const int c = lane & 15;

  // decoder mode loads the raw rows here and forms q once the first stages
  // of the ring are in flight (q_ready)
  uint4 qv[G];
  bool q_ready = !ROPE;
  const size_t q_row = ROPE ? (size_t)b * (P.Hq + 2 * P.Hkv) : (size_t)b * P.Hq;
#pragma unroll
  for (int h = 0; h < G; ++h)
    qv[h] = *reinterpret_cast<const uint4*>(P.q + (q_row + g * G + h) * kHeadDim + c * 8);
  RopeLane rl;
  if constexpr (ROPE) rope_lane_load(P, b, c, rl);

  State<G> st;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = kNegBig;
    st.l[h] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) st.acc[h][i] = 0.0f;
  }

  const int n_total = S.size();
  const bool has_current = (v_hi == n_total);
  const int v_cache_hi = has_current ? v_hi - 1 : v_hi;
  // first range [0, n0) -> positions equal virtual indices
  if (v_lo < S.n0) {
    const int hi = v_cache_hi < S.n0 ? v_cache_hi : S.n0;
    if (hi > v_lo) cache_rows<G, PAGED, NW, DEPTH, U, ROPE>(P, qv, q_ready, rl, st, b, g, v_lo, hi, wave, r, c, lds);
  }
  // second range: virtual n0 + k  ->  position s1 + k
  {
    const int lo = v_lo > S.n0 ? v_lo : S.n0;
    if (v_cache_hi > lo)
      cache_rows<G, PAGED, NW, DEPTH, U, ROPE>(P, qv, q_ready, rl, st, b, g, S.s1 + (lo - S.n0),
                                               S.s1 + (v_cache_hi - S.n0), wave, r, c, lds);
  }
  if constexpr (ROPE) {
    if (!q_ready) {  // this wave streamed no cache rows
      rope_q<G>(P, qv, rl, c);
      q_ready = true;
    }
  }
  if (has_current) current_row<G, ROPE>(P, qv, rl, st, b, g, wave, r, c);

  wg_merge<G, NW>(st, lds, wave, lane, c);

  constexpr int NT = NW * 64;
  if (nsplit == 1) {
    for (int idx = tid; idx < G * kHeadDim; idx += NT) {
      const int h = idx / kHeadDim, dd = idx % kHeadDim;
      float M, L, O;
      wg_value<G, NW>(lds, h, dd, M, L, O);
      write_out(P, b, g * G + h, dd, M, L, O);
    }
    __syncthreads();
    return;
  }
  // store this split's partial
  for (int idx = tid; idx < G * kHeadDim; idx += NT) {
    const int h = idx / kHeadDim, dd = idx % kHeadDim;
    float M, L, O;
    wg_value<G, NW>(lds, h, dd, M, L, O);
    float* pp = part_bg + ((size_t)split * G + h) * kPartStride;
    part_store(pp + dd, O);
    if (dd == 0) {
      part_store(pp + kHeadDim, M);
      part_store(pp + kHeadDim + 1, L);
    }
  }
  if (take_ticket(ticket, nsplit)) {
    merge_partials<G, NW, MAXS>(P, part_bg, nsplit, b, g, lds);
    if (tid == 0) reset_ticket(ticket);
  }
  __syncthreads();
}

template <int G, bool PAGED, bool ROPE, int NW>
__global__ void __launch_bounds__(NW * 64) k_attn_local(AttnParams P) {
  __shared__ float lds[lds_floats<G, NW>()];
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int pos = P.pos[b];
  const int t = pos + 1;
  if (pos < 0 || (int64_t)t > P.t_max) {
    if (split == 0 && g == 0 && threadIdx.x == 0) atomicOr(P.err, ODA_ERR_CAPACITY);
    return;
  }
  const LocalSet S = local_set(t, P.sink, P.window);
  const int n = S.size();
  int ns = (n + kLocalMinChunk - 1) / kLocalMinChunk;
  ns = ns < P.local_splits ? ns : P.local_splits;
  const int chunk = (n + ns - 1) / ns;
  if (split >= ns) return;
  const int v_lo = split * chunk;
  const int v_hi = (v_lo + chunk) < n ? v_lo + chunk : n;
  float* part_bg = P.part + ((size_t)(b * P.Hkv + g) * kLocalMaxSplits) * G * kPartStride;
  constexpr int kMaxS = PAGED ? kLocalSplitsMaxPaged : kLocalSplitsMax;
  attn_unit<G, PAGED, NW, ODA_LOCAL_DEPTH, ODA_LOCAL_U, kMaxS, ROPE>(P, b, g, split, ns, v_lo, v_hi, S, P.tickets + b * P.Hkv + g, part_bg, lds);
}

// The persistent grid walks units u = (work-list item) * Hkv + KV head.
// Workgroup i takes unit i; when the list holds more units than the grid,
// the rest are handed out in list order (largest units first) through an
// atomic counter, each workgroup asking for its next unit while it streams
// the current one.  Once every workgroup has found the list exhausted, the
// last one to finish clears the counters, so each launch starts from zero.
template <int G, bool PAGED>
__global__ void __launch_bounds__((FullWaves<G, PAGED>::value * 64)) k_attn_full(AttnParams P) {
  constexpr int NW = FullWaves<G, PAGED>::value;
  __shared__ float lds[lds_floats<G, NW>()];
  __shared__ int s_next;
  int count = P.worklist[0];
  count = count < 0 ? 0 : (count > P.B * kFullMaxSplits ? P.B * kFullMaxSplits : count);
  const int units = count * P.Hkv;
  const int grid = (int)gridDim.x;
  const bool queued = units > grid;
  int u = blockIdx.x;
  while (u < units) {
    int next = 0;
    if (queued && threadIdx.x == 0)
      next = grid + __hip_atomic_fetch_add(P.queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int item = P.worklist[1 + u / P.Hkv];
    const int g = u % P.Hkv;
    const int b = item >> 20;
    const int ns = (item >> 10) & 0x3FF;
    const int split = item & 0x3FF;
    const int pos = (b >= 0 && b < P.B) ? P.pos[b] : -1;
    const int t = pos + 1;
    if (b < 0 || b >= P.B || ns < 1 || ns > kFullMaxSplits || split >= ns) {
      // malformed item: skipped
    } else if (pos < 0 || (int64_t)t > P.t_max) {
      if (split == 0 && g == 0 && threadIdx.x == 0) atomicOr(P.err, ODA_ERR_CAPACITY);
    } else {
      const int chunk = (t + ns - 1) / ns;
      const int v_lo = split * chunk;
      const int v_hi = (v_lo + chunk) < t ? v_lo + chunk : t;
      LocalSet S;
      S.n0 = t;
      S.s1 = t;
      S.t = t;
      float* part_bg = P.part + ((size_t)(b * P.Hkv + g) * kFullMaxSplits) * G * kPartStride;
      attn_unit<G, PAGED, NW, FullDepth<G, PAGED>::value, ODA_FULL_U, kFullMaxSplits, false>(P, b, g, split, ns, v_lo, v_hi, S, P.tickets + b * P.Hkv + g, part_bg, lds);
    }
    if (!queued) break;
    if (threadIdx.x == 0) s_next = next;
    __syncthreads();
    u = s_next;
    __syncthreads();
  }
  if (queued && threadIdx.x == 0) {
    if (__hip_atomic_fetch_add(P.queue + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == grid - 1) {
      // every other workgroup has drawn past the end and will not touch the
      // counters again in this launch
      __hip_atomic_store(P.queue, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(P.queue + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Compute units of the current device, queried once per device (host
// threads may race on the first query; each stores the same value).
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Workgroups per (sequence, KV head) in the local branch: enough for one per
// compute unit over the whole batch, ceil(CUs / (B Hkv)), within
// [kLocalSplitsMin, kLocalSplitsMax] for a contiguous cache and
// [kLocalSplitsMin, kLocalSplitsMaxPaged] for a paged one.  The local set is
// small (at most sink + window keys): for a contiguous cache past 8 splits
// the cross-workgroup merge costs more than the extra streaming parallelism
// gains (16 splits: the same at 1 sequence, 10-13% slower at 2 and 3); the
// paged walk still gains from 16 at one sequence (9.9 against 11.1 us per
// launch at 128K, 16 / 8 heads).  Per launch, paged, one workgroup per
// compute unit against two: 12.6 / 15.2 us at 4 x 128K, 45.6 / 47.4 us at
// 32 x 4K, 27.3 / 27.5 us at 16 x 16K.  Contiguous, against four per compute
// unit: 16.2 / 17.2 us at 8 x 16K, 28.9 / 33.0 us at 16 x 64K with group
// size 4, 43.4 / 48.8 us at 32 x 4K, the same within 2% at 4 x 128K.  At 8
// KV heads: 8 splits (16 paged at one sequence) up to 4 sequences, 4 at 8,
// 2 at 16, 1 (no merge at all) at 32.
int local_splits(const AttnParams& p, bool paged) {
  const int pairs = p.B * p.Hkv;
  const int cap = paged ? kLocalSplitsMaxPaged : kLocalSplitsMax;
  const int ns = (device_cus() + pairs - 1) / pairs;
  return ns < kLocalSplitsMin ? kLocalSplitsMin : (ns > cap ? cap : ns);
}

template <int G, bool PAGED, bool ROPE>
int launch_local_t(const AttnParams& p_in, hipStream_t s) {
  static_assert(kLocalSplitsMax <= kLocalMaxSplits && kLocalSplitsMaxPaged <= kLocalMaxSplits,
                "local splits exceed the workspace slots");
  AttnParams p = p_in;
  p.local_splits = local_splits(p, PAGED);
  dim3 grid(p.local_splits, p.Hkv, p.B);
  if (p.local_splits <= kLocalWideMax)
    hipLaunchKernelGGL((k_attn_local<G, PAGED, ROPE, kLocalWavesWide>), grid, dim3(kLocalWavesWide * 64), 0, s, p);
  else
    hipLaunchKernelGGL((k_attn_local<G, PAGED, ROPE, kLocalWaves>), grid, dim3(kLocalWaves * 64), 0, s, p);
  return hipGetLastError() == hipSuccess ? ODA_OK : ODA_E_LAUNCH;
}

int full_grid(const AttnParams& p) {
  const long units_max = (long)p.B * p.Hkv * kFullMaxSplits;
  const long grid = device_cus();
  return (int)(units_max < grid ? units_max : grid);
}

template <int G, bool PAGED>
int launch_full_t(const AttnParams& p, hipStream_t s) {
  dim3 grid(full_grid(p));
  hipLaunchKernelGGL((k_attn_full<G, PAGED>), grid, dim3(FullWaves<G, PAGED>::value * 64), 0, s, p);
  return hipGetLastError() == hipSuccess ? ODA_OK : ODA_E_LAUNCH;
}

}  // namespace

namespace {
template <bool ROPE>
int launch_local_g(const AttnParams& p, int G, bool paged, hipStream_t s) {
  switch (G) {
    case 1: return paged ? launch_local_t<1, true, ROPE>(p, s) : launch_local_t<1, false, ROPE>(p, s);
    case 2: return paged ? launch_local_t<2, true, ROPE>(p, s) : launch_local_t<2, false, ROPE>(p, s);
    case 4: return paged ? launch_local_t<4, true, ROPE>(p, s) : launch_local_t<4, false, ROPE>(p, s);
    default: return ODA_E_UNSUPPORTED;
  }
}

}  // namespace

int launch_local_attn(const AttnParams& p, int G, bool paged, hipStream_t s, bool rope) {
  return rope ? launch_local_g<true>(p, G, paged, s) : launch_local_g<false>(p, G, paged, s);
}

int launch_full_attn(const AttnParams& p, int G, bool paged, hipStream_t s) {
  switch (G) {
    case 1: return paged ? launch_full_t<1, true>(p, s) : launch_full_t<1, false>(p, s);
    case 2: return paged ? launch_full_t<2, true>(p, s) : launch_full_t<2, false>(p, s);
    case 4: return paged ? launch_full_t<4, true>(p, s) : launch_full_t<4, false>(p, s);
    default: return ODA_E_UNSUPPORTED;
  }
}

}  // namespace oda
