// The extern "C" entry points of liboda: argument validation, workspace
// layout and kernel launches.  No allocation, no synchronisation, no device
// reads on the host; every entry point can be captured into a hipGraph.
#include <math.h>
#include <string.h>

#include "head_internal.h"
#include "abi_align.h"

namespace oda {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

static int log2i(int32_t x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

bool dims_valid(const oda_dims* d, int* status) {
  *status = ODA_OK;
  if (d == nullptr) {
    *status = ODA_E_NULL;
    return false;
  }
  if (d->num_layers < 1 || d->batch < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->head_dim < 1 ||
      d->sink < 0 || d->window < 1 || d->reserved0 != 0 || d->num_q_heads % d->num_kv_heads != 0 ||
      (int64_t)d->hidden != (int64_t)d->num_q_heads * d->head_dim) {
    *status = ODA_E_DIMS;
    return false;
  }
  const int G = d->num_q_heads / d->num_kv_heads;
  if (d->head_dim != kHeadDim || d->batch > kMaxBatch || (G != 1 && G != 2 && G != 4)) {
    *status = ODA_E_UNSUPPORTED;
    return false;
  }
  if (d->kv_layout == ODA_KV_CONTIG) {
    if (d->t_cap < 1 || d->t_cap > ((int64_t)1 << 30)) {
      *status = ODA_E_DIMS;
      return false;
    }
  } else if (d->kv_layout == ODA_KV_PAGED) {
    if (!is_pow2(d->block_size) || d->max_blocks_per_seq < 1 || d->num_blocks < 1 ||
        (int64_t)d->block_size * d->max_blocks_per_seq > ((int64_t)1 << 30)) {
      *status = ODA_E_DIMS;
      return false;
    }
  } else {
    *status = ODA_E_DIMS;
    return false;
  }
  return true;
}

WsLayout ws_layout(const oda_dims* d) {
  WsLayout L;
  const int B = d->batch, Hkv = d->num_kv_heads, G = d->num_q_heads / d->num_kv_heads;
  size_t at = 0;
  L.header = at;
  at = align256(at + 64 * sizeof(int32_t));
  L.worklist = at;
  at = align256(at + (1 + (size_t)B * kFullMaxSplits) * sizeof(int32_t));
  L.tick_local = at;
  at = align256(at + (size_t)B * Hkv * sizeof(int32_t));
  L.tick_full = at;
  at = align256(at + (size_t)B * Hkv * sizeof(int32_t));
  L.tick_commit = at;
  at = align256(at + (size_t)B * sizeof(int32_t));
  L.tick_head = at;
  at = align256(at + (size_t)kHeadTickets * sizeof(int32_t));
  L.part_local = at;
  at = align256(at + (size_t)B * Hkv * kLocalMaxSplits * G * kPartStride * sizeof(float));
  L.part_full = at;
  at = align256(at + (size_t)B * Hkv * kFullMaxSplits * G * kPartStride * sizeof(float));
  L.head = at;
  at = align256(at + head_ws_floats(B, d->hidden) * sizeof(float));
  L.total = at;
  L.t_max = d->kv_layout == ODA_KV_CONTIG ? d->t_cap : (int64_t)d->block_size * d->max_blocks_per_seq;
  return L;
}

static int head_offsets_impl(int32_t hidden, int64_t* offs) {
  if (offs == nullptr) return ODA_E_NULL;
  if (hidden < 1) return ODA_E_DIMS;
  const int64_t D = hidden, T = kTower, F = kFfn;
  const int64_t sizes[ODA_HEAD_NTENSORS] = {
      D, T * D, T,             // tower H
      D, T * D, T,             // tower E
      D, T * D, T,             // tower L
      T * 9 * T, T,            // interaction
      T, F * T, F * T, T * F,  // ffn 1
      T, F * T, F * T, T * F,  // ffn 2
      T, T, 1};                // out
  int64_t at = 0;
  for (int i = 0; i < ODA_HEAD_NTENSORS; ++i) {
    offs[i] = at;
    at += sizes[i];
  }
  offs[ODA_HEAD_NTENSORS] = at;
  return ODA_OK;
}

AttnParams attn_params_at(const oda_dims* d, int32_t layer, const oda_kv* kv, const int32_t* pos, const oda_bf16* q,
                          const oda_bf16* kc, const oda_bf16* vc, oda_bf16* out, float* lse, float* part,
                          int32_t* tickets, int32_t* header, const int32_t* worklist) {
  AttnParams p;
  memset(&p, 0, sizeof(p));
  size_t layer_stride;
  if (d->kv_layout == ODA_KV_CONTIG) {
    layer_stride = (size_t)d->batch * d->num_kv_heads * (size_t)d->t_cap * kHeadDim;
  } else {
    layer_stride = (size_t)d->num_blocks * d->num_kv_heads * (size_t)d->block_size * kHeadDim;
  }
  p.K = kv->k + (size_t)layer * layer_stride;
  p.V = kv->v + (size_t)layer * layer_stride;
  p.tables = d->kv_layout == ODA_KV_PAGED ? kv->block_tables : nullptr;
  p.t_cap = d->t_cap;
  p.num_blocks = d->num_blocks;
  p.max_blocks = d->max_blocks_per_seq;
  p.log2_block = d->kv_layout == ODA_KV_PAGED ? log2i(d->block_size) : 0;
  p.pos = pos;
  p.q = q;
  p.kc = kc;
  p.vc = vc;
  p.out = out;
  p.lse = lse;
  p.part = part;
  p.tickets = tickets;
  p.err = header;
  p.queue = header + 1;
  p.worklist = worklist;
  p.B = d->batch;
  p.Hq = d->num_q_heads;
  p.Hkv = d->num_kv_heads;
  p.sink = d->sink;
  p.window = d->window;
  p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d->head_dim));
  p.t_max = d->kv_layout == ODA_KV_CONTIG ? d->t_cap : (int64_t)d->block_size * d->max_blocks_per_seq;
  return p;
}

static AttnParams attn_params(const oda_dims* d, int32_t layer, const oda_kv* kv, const int32_t* pos,
                              const oda_bf16* q, const oda_bf16* kc, const oda_bf16* vc, oda_bf16* out, float* lse,
                              void* ws, const WsLayout& L, bool full) {
  char* w = static_cast<char*>(ws);
  return attn_params_at(d, layer, kv, pos, q, kc, vc, out, lse,
                        reinterpret_cast<float*>(w + (full ? L.part_full : L.part_local)),
                        reinterpret_cast<int32_t*>(w + (full ? L.tick_full : L.tick_local)),
                        reinterpret_cast<int32_t*>(w + L.header), reinterpret_cast<const int32_t*>(w + L.worklist));
}

int check_attn_operands(const oda_dims* d, int32_t layer, const oda_kv* kv, const int32_t* pos, const oda_bf16* q,
                        const oda_bf16* kc, const oda_bf16* vc, const oda_bf16* out) {
  int st;
  if (!dims_valid(d, &st)) return st;
  if (kv == nullptr || kv->k == nullptr || kv->v == nullptr || pos == nullptr || q == nullptr || kc == nullptr ||
      vc == nullptr || out == nullptr)
    return ODA_E_NULL;
  if (d->kv_layout == ODA_KV_PAGED && kv->block_tables == nullptr) return ODA_E_NULL;
  if (layer < 0 || layer >= d->num_layers) return ODA_E_LAYER;
  if (!aligned_to(kv->k, 16) || !aligned_to(kv->v, 16) || !aligned_to(kv->block_tables, 4) || !aligned_to(pos, 4) ||
      !aligned_to(q, 16) || !aligned_to(kc, 16) || !aligned_to(vc, 16) || !aligned_to(out, 16))
    return ODA_E_ALIGN;
  return ODA_OK;
}

static int check_attn_args(const oda_dims* d, int32_t layer, const oda_kv* kv, const int32_t* pos, const oda_bf16* q,
                           const oda_bf16* kc, const oda_bf16* vc, oda_bf16* out, void* ws, size_t ws_bytes,
                           WsLayout* L) {
  const int st = check_attn_operands(d, layer, kv, pos, q, kc, vc, out);
  if (st != ODA_OK) return st;
  if (ws == nullptr) return ODA_E_NULL;
  if (!aligned_to(ws, 16)) return ODA_E_ALIGN;
  *L = ws_layout(d);
  if (ws_bytes < L->total) return ODA_E_WORKSPACE;
  return ODA_OK;
}

int decoder_local_attn(const ::oda_dims* d, int32_t layer, const ::oda_kv* kv, const int32_t* pos,
                       const uint16_t* qkv, const uint16_t* gq, const uint16_t* gk, const float* rope, float qk_eps,
                       uint16_t* k_stage, uint16_t* v_stage, uint16_t* out, void* ws, size_t ws_bytes,
                       hipStream_t s) {
  WsLayout L;
  const int st = check_attn_args(d, layer, kv, pos, qkv, k_stage, v_stage, out, ws, ws_bytes, &L);
  if (st != ODA_OK) return st;
  if (gq == nullptr || gk == nullptr || rope == nullptr) return ODA_E_NULL;
  AttnParams p = attn_params(d, layer, kv, pos, qkv, qkv, qkv, out, nullptr, ws, L, false);
  p.gq = gq;
  p.gk = gk;
  p.rope = rope;
  p.k_stage = k_stage;
  p.v_stage = v_stage;
  p.qk_eps = qk_eps;
  return launch_local_attn(p, d->num_q_heads / d->num_kv_heads, d->kv_layout == ODA_KV_PAGED, s, true);
}

}  // namespace oda

using namespace oda;

extern "C" {

int oda_abi_version(void) { return ODA_ABI_VERSION; }

const char* oda_status_str(int status) {
  switch (status) {
    case ODA_OK: return "ok";
    case ODA_E_NULL: return "a required pointer is NULL";
    case ODA_E_DIMS: return "inconsistent or out-of-range dimensions";
    case ODA_E_UNSUPPORTED: return "dimensions not supported by liboda";
    case ODA_E_WORKSPACE: return "workspace smaller than oda_workspace_bytes()";
    case ODA_E_LAYER: return "layer index out of range";
    case ODA_E_LAUNCH: return "kernel launch failed";
    case ODA_E_ALIGN: return "a device pointer is not aligned as the ABI requires";
    default: return "unknown status";
  }
}

int64_t oda_head_param_count(int32_t hidden) {
  int64_t offs[ODA_HEAD_NTENSORS + 1];
  if (head_offsets_impl(hidden, offs) != ODA_OK) return -1;
  return offs[ODA_HEAD_NTENSORS];
}

int oda_head_offsets(int32_t hidden, int64_t* offsets) { return head_offsets_impl(hidden, offsets); }

size_t oda_workspace_bytes(const oda_dims* dims) {
  int st;
  if (!dims_valid(dims, &st)) return 0;
  return ws_layout(dims).total;
}

size_t oda_workspace_worklist_offset(const oda_dims* dims) {
  int st;
  if (!dims_valid(dims, &st)) return 0;
  return ws_layout(dims).worklist;
}

int oda_workspace_init(const oda_dims* dims, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st;
  if (!dims_valid(dims, &st)) return st;
  if (ws == nullptr) return ODA_E_NULL;
  if (!aligned_to(ws, 16)) return ODA_E_ALIGN;
  const WsLayout L = ws_layout(dims);
  if (ws_bytes < L.total) return ODA_E_WORKSPACE;
  // header, work list and every ticket array lie in [0, part_local)
  return launch_fill_zero(static_cast<int32_t*>(ws), L.part_local / sizeof(int32_t), stream);
}

int oda_local_ranges(const oda_dims* dims, const int32_t* pos, int32_t* ranges, hipStream_t stream) {
  int st;
  if (!dims_valid(dims, &st)) return st;
  if (pos == nullptr || ranges == nullptr) return ODA_E_NULL;
  if (!aligned_to(pos, 4) || !aligned_to(ranges, 4)) return ODA_E_ALIGN;
  return launch_ranges(pos, ranges, dims->batch, dims->sink, dims->window, stream);
}

int oda_local_attn(const oda_dims* dims, int32_t layer, const oda_kv* kv, const int32_t* pos, const oda_bf16* q,
                   const oda_bf16* k_cur, const oda_bf16* v_cur, oda_bf16* out, float* lse, void* ws,
                   size_t ws_bytes, hipStream_t stream) {
  WsLayout L;
  const int st = check_attn_args(dims, layer, kv, pos, q, k_cur, v_cur, out, ws, ws_bytes, &L);
  if (st != ODA_OK) return st;
  if (!aligned_to(lse, 4)) return ODA_E_ALIGN;
  const AttnParams p = attn_params(dims, layer, kv, pos, q, k_cur, v_cur, out, lse, ws, L, false);
  return launch_local_attn(p, dims->num_q_heads / dims->num_kv_heads, dims->kv_layout == ODA_KV_PAGED, stream);
}

int oda_full_attn_if(const oda_dims* dims, int32_t layer, const oda_kv* kv, const int32_t* pos, const oda_bf16* q,
                     const oda_bf16* k_cur, const oda_bf16* v_cur, oda_bf16* out, float* lse, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  WsLayout L;
  const int st = check_attn_args(dims, layer, kv, pos, q, k_cur, v_cur, out, ws, ws_bytes, &L);
  if (st != ODA_OK) return st;
  if (!aligned_to(lse, 4)) return ODA_E_ALIGN;
  const AttnParams p = attn_params(dims, layer, kv, pos, q, k_cur, v_cur, out, lse, ws, L, true);
  return launch_full_attn(p, dims->num_q_heads / dims->num_kv_heads, dims->kv_layout == ODA_KV_PAGED, stream);
}

int oda_recall_score(const oda_dims* dims, const float* head_w, const oda_bf16* h_prev, const oda_bf16* emb,
                     const oda_bf16* h_local, float theta, const int8_t* force, const int32_t* pos, float* score,
                     uint8_t* flag, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st;
  if (!dims_valid(dims, &st)) return st;
  if (head_w == nullptr || h_prev == nullptr || emb == nullptr || h_local == nullptr || pos == nullptr ||
      score == nullptr || flag == nullptr || ws == nullptr)
    return ODA_E_NULL;
  if (!aligned_to(head_w, 16) || !aligned_to(h_prev, 16) || !aligned_to(emb, 16) || !aligned_to(h_local, 16) ||
      !aligned_to(pos, 4) || !aligned_to(score, 4) || !aligned_to(ws, 16))
    return ODA_E_ALIGN;
  const WsLayout L = ws_layout(dims);
  if (ws_bytes < L.total) return ODA_E_WORKSPACE;
  int64_t offs[ODA_HEAD_NTENSORS + 1];
  head_offsets_impl(dims->hidden, offs);
  HeadParams p;
  memset(&p, 0, sizeof(p));
  p.w = head_w;
  p.h_prev = h_prev;
  p.emb = emb;
  p.h_local = h_local;
  p.theta = theta;
  p.force = force;
  p.pos = pos;
  p.score = score;
  p.flag = flag;
  p.worklist = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + L.worklist);
  p.B = dims->batch;
  p.D = dims->hidden;
  p.Hkv = dims->num_kv_heads;
  p.tickets = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + L.tick_head);
  p.act = head_ws(ws, L, dims->batch, dims->hidden);
  return launch_recall_head(p, offs, stream);
}

int oda_worklist(const oda_dims* dims, const uint8_t* flag, const int32_t* pos, void* ws, size_t ws_bytes,
                 hipStream_t stream) {
  int st;
  if (!dims_valid(dims, &st)) return st;
  if (flag == nullptr || pos == nullptr || ws == nullptr) return ODA_E_NULL;
  if (!aligned_to(pos, 4) || !aligned_to(ws, 16)) return ODA_E_ALIGN;
  const WsLayout L = ws_layout(dims);
  if (ws_bytes < L.total) return ODA_E_WORKSPACE;
  return launch_worklist(flag, pos, reinterpret_cast<int32_t*>(static_cast<char*>(ws) + L.worklist), dims->batch,
                         dims->num_kv_heads, stream);
}

int oda_commit(const oda_dims* dims, const oda_kv* kv, int32_t* pos, const uint8_t* flag, const oda_bf16* k_cur_L,
               const oda_bf16* v_cur_L, const oda_bf16* k_cur_F, const oda_bf16* v_cur_F,
               const oda_bf16* out_last_L, const oda_bf16* out_last_F, oda_bf16* h_prev, void* ws, size_t ws_bytes,
               hipStream_t stream) {
  int st;
  if (!dims_valid(dims, &st)) return st;
  if (kv == nullptr || kv->k == nullptr || kv->v == nullptr || pos == nullptr || flag == nullptr ||
      k_cur_L == nullptr || v_cur_L == nullptr || k_cur_F == nullptr || v_cur_F == nullptr ||
      out_last_L == nullptr || out_last_F == nullptr || h_prev == nullptr || ws == nullptr)
    return ODA_E_NULL;
  if (dims->kv_layout == ODA_KV_PAGED && kv->block_tables == nullptr) return ODA_E_NULL;
  if (!aligned_to(kv->k, 16) || !aligned_to(kv->v, 16) || !aligned_to(kv->block_tables, 4) || !aligned_to(pos, 4) ||
      !aligned_to(k_cur_L, 16) || !aligned_to(v_cur_L, 16) || !aligned_to(k_cur_F, 16) || !aligned_to(v_cur_F, 16) ||
      !aligned_to(out_last_L, 16) || !aligned_to(out_last_F, 16) || !aligned_to(h_prev, 16) || !aligned_to(ws, 16))
    return ODA_E_ALIGN;
  const WsLayout L = ws_layout(dims);
  if (ws_bytes < L.total) return ODA_E_WORKSPACE;
  CommitParams p;
  memset(&p, 0, sizeof(p));
  p.K = kv->k;
  p.V = kv->v;
  const bool paged = dims->kv_layout == ODA_KV_PAGED;
  p.tables = paged ? kv->block_tables : nullptr;
  p.t_cap = dims->t_cap;
  p.num_blocks = dims->num_blocks;
  p.layer_stride = paged ? (int64_t)dims->num_blocks * dims->num_kv_heads * dims->block_size * kHeadDim
                         : (int64_t)dims->batch * dims->num_kv_heads * dims->t_cap * kHeadDim;
  p.max_blocks = dims->max_blocks_per_seq;
  p.log2_block = paged ? log2i(dims->block_size) : 0;
  p.pos = pos;
  p.flag = flag;
  p.kL = k_cur_L;
  p.vL = v_cur_L;
  p.kF = k_cur_F;
  p.vF = v_cur_F;
  p.oL = out_last_L;
  p.oF = out_last_F;
  p.h_prev = h_prev;
  char* w = static_cast<char*>(ws);
  p.tickets = reinterpret_cast<int32_t*>(w + L.tick_commit);
  p.err = reinterpret_cast<int32_t*>(w + L.header);
  p.L = dims->num_layers;
  p.B = dims->batch;
  p.Hkv = dims->num_kv_heads;
  p.D = dims->hidden;
  p.t_max = L.t_max;
  return launch_commit(p, stream);
}

}  // extern "C"
