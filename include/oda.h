/*
 * oda.h -- C ABI of liboda, the On-Demand Attention (ODA) decode step on
 * AMD Instinct MI355X (gfx950).
 *
 * Method source: the page "On-Demand Attention：让语言模型按需读取完整历史"
 * (notes on arXiv 2609.20734), cited as [ODA notes] with section / equation.
 *
 * One decode step of a batch of B sequences is four calls, in this order on
 * one stream (or with equivalent event ordering):
 *
 *   1. oda_local_attn    for every layer l       [ODA notes §2.1, eq. o_t over S^L]
 *   2. oda_recall_score  once                    [ODA notes §2.2 eq. q_t; §2.3 rule]
 *   3. oda_full_attn_if  for every layer l       [ODA notes §2.1 eq. o_t over S^F; §2.3]
 *   4. oda_commit        once                    [ODA notes §2.3 eq. h_t, C_t]
 *
 * General rules for every entry point:
 *  - Every pointer argument is a DEVICE pointer owned by the caller, except
 *    `dims`, `kv` and `offsets`, which are HOST pointers read during the
 *    call only.  The library never allocates or frees memory, never
 *    synchronises a stream and never reads device memory from the host, so
 *    every call may be captured into a hipGraph.
 *  - The library keeps no mutable global state beyond a per-device cache of
 *    the compute-unit count (queried once, used to size grids).  Calls that
 *    share a workspace `ws` must be ordered (same stream); calls on
 *    different workspaces may run concurrently.
 *  - Alignment: bf16 and float arrays (q, k_cur, v_cur, out, the caches,
 *    head_w, h_prev, emb, h_local, the staged rows) and `ws` must be 16-byte
 *    aligned, int32 arrays (pos, block tables, ranges, lse, score) 4-byte
 *    aligned; the kernels read them with 16-byte vector and direct-to-LDS
 *    loads.  hipMalloc and torch allocations are 256-byte aligned, and every
 *    row of the layouts below starts on a 16-byte boundary.  A pointer that
 *    breaks this is refused with ODA_E_ALIGN.
 *  - Return value: ODA_OK (0) or a negative ODA_E_* code.  On an error
 *    nothing has been launched and no memory has been touched.
 *  - Conditions that can only be seen on the device (a position beyond the
 *    cache capacity, a block-table entry outside the pool) set sticky bits
 *    in the workspace error word (ODA_WS_ERROR_WORD, an int32 at byte 0 of
 *    `ws`); the affected sequence is skipped.  The caller may read the word
 *    after synchronising.  A non-finite recall score is not an error: the
 *    rule sends that sequence to the full branch.
 *
 * Data types and layouts (all row-major, innermost index last):
 *  - oda_bf16 is the raw bit pattern of a bfloat16 value.
 *  - d = head_dim = 128; G = Hq / Hkv query heads share one KV head, query
 *    head h reading KV head h / G (consecutive heads share).
 *  - pos[b] (int32) is the committed length of sequence b: the current
 *    token has 0-based position pos[b], the pages' t is pos[b] + 1.
 *  - Contiguous KV cache (kv_layout = ODA_KV_CONTIG): k, v are
 *    [L][B][Hkv][t_cap][d].
 *  - Paged KV cache (ODA_KV_PAGED): k, v are [L][num_blocks][Hkv][block_size][d];
 *    block_tables is [B][max_blocks_per_seq] int32, logical position p of
 *    sequence b lives in physical block block_tables[b][p / block_size] at
 *    row p % block_size.  block_size must be a power of two.
 *  - Per-layer attention operands: q [B][Hq][d]; staged current key/value
 *    k_cur, v_cur [B][Hkv][d]; out [B][Hq][d] (= [B][D] with D = Hq*d);
 *    optional lse [B][Hq] float (natural-log log-sum-exp of the scaled
 *    scores), NULL to skip.
 */
#ifndef ODA_H_
#define ODA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ODA_ABI_VERSION 1

/* status codes */
#define ODA_OK 0
#define ODA_E_NULL (-1)        /* a required pointer is NULL */
#define ODA_E_DIMS (-2)        /* inconsistent or out-of-range dimensions */
#define ODA_E_UNSUPPORTED (-3) /* valid but not supported by liboda (head_dim != 128, B > 32, ...) */
#define ODA_E_WORKSPACE (-4)   /* ws_bytes smaller than oda_workspace_bytes(dims) */
#define ODA_E_LAYER (-5)       /* layer index outside [0, num_layers) */
#define ODA_E_LAUNCH (-6)      /* the HIP runtime rejected a kernel launch */
#define ODA_E_ALIGN (-7)       /* a device pointer is not aligned as the rules above require */

/* kv_layout */
#define ODA_KV_CONTIG 0
#define ODA_KV_PAGED 1

/* sticky device-side error bits in the workspace error word */
#define ODA_WS_ERROR_WORD 0
#define ODA_ERR_CAPACITY 1   /* pos[b] + 1 exceeds the sequence's capacity */
#define ODA_ERR_BLOCK 2      /* a block-table entry is outside [0, num_blocks) */
#define ODA_ERR_TOKEN 4      /* a token id is outside [0, vocab) (oda_decoder.h, oda_train.h) */
#define ODA_ERR_ROW 8        /* a previous-row index is outside [-1, rows) (oda_train.h) */

/* recall head geometry [ODA notes §2.2]: three 1024-wide towers, a
 * 9*1024-wide interaction, two gated FFN blocks of hidden width 2048 */
#define ODA_HEAD_TOWER 1024
#define ODA_HEAD_FFN 2048
#define ODA_HEAD_NTENSORS 22

/* Split policy of the full branch.  With F flagged sequences holding T keys
 * together (t = pos + 1 keys each) and Hkv KV heads (P = F * Hkv units per
 * split index), each flagged sequence is cut into nsplit(t) contiguous
 * splits of ceil(t / nsplit) keys (the last one shorter, none empty).  Two
 * candidate cuts are formed:
 *  A, one round:
 *   n0 = max(min(ODA_FULL_MAX_SPLITS, ceil(t / ODA_FULL_MIN_CHUNK)),
 *            min(ODA_FULL_MAX_SPLITS, ceil(t / ODA_FULL_FINE_CHUNK),
 *                floor(ODA_FULL_FILL_UNITS / P)))
 *   share = max(1, floor(ODA_FULL_ROUND_UNITS * t / (T * Hkv)))
 *   nA = min(n0, share)
 *   -- chunks of ODA_FULL_MIN_CHUNK keys or more, cut finer (down to
 *   ODA_FULL_FINE_CHUNK) while the launch would hold fewer than
 *   ODA_FULL_FILL_UNITS units, and at most the sequence's share, in
 *   proportion to its length, of one round of ODA_FULL_ROUND_UNITS units of
 *   the full kernel's persistent grid (one workgroup per compute unit of an
 *   MI355X); for equal lengths the share is floor(ODA_FULL_ROUND_UNITS / P);
 *  B, several rounds of smaller units:
 *   C = max(ODA_FULL_MIN_CHUNK,
 *           ceil(T * Hkv / (ODA_FULL_RAGGED_ROUNDS * ODA_FULL_ROUND_UNITS)))
 *   nB = min(ODA_FULL_MAX_SPLITS, ceil(t / C)).
 * Each candidate X has N_X = Hkv * sum(nX) units, R_X =
 * ceil(N_X / ODA_FULL_ROUND_UNITS) rounds, the longest unit U_X and the
 * shortest u_X (units of ceil(t / nX) keys), and the estimated time in keys
 *   cost_X = min(R_X * (U_X + K0),
 *                max(U_X, ceil(T * Hkv / ODA_FULL_ROUND_UNITS)
 *                         + (N_X > ODA_FULL_ROUND_UNITS ? u_X : 0)) + R_X * K0)
 * with K0 = ODA_FULL_UNIT_COST_KEYS, a unit's fixed cost in keys (the first
 * term is exact for equal units; the second, for units of mixed size handed
 * out largest first, is the even share of all keys plus a short unit left
 * over).  B is used when cost_B < cost_A, else A: equal lengths that divide
 * into one round keep A; ragged lengths, whose one-round shares round to
 * units of unequal size, take B.  The work list has one item per (flagged
 * sequence, split); sequences are listed longest unit first
 * (ceil(t / nsplit) descending, ties by ascending b), their splits in
 * order.  Units past the first round are handed out by the kernel in list
 * order (largest first) as workgroups become free. */
#define ODA_FULL_MIN_CHUNK 1024
#define ODA_FULL_FINE_CHUNK 256
#define ODA_FULL_FILL_UNITS 128
#define ODA_FULL_ROUND_UNITS 256
#define ODA_FULL_MAX_SPLITS 32
#define ODA_FULL_RAGGED_ROUNDS 4
#define ODA_FULL_UNIT_COST_KEYS 128

typedef uint16_t oda_bf16;

typedef struct oda_dims {
  int32_t num_layers;          /* L >= 1 */
  int32_t batch;               /* B, 1..32 */
  int32_t num_q_heads;         /* Hq */
  int32_t num_kv_heads;        /* Hkv; Hq % Hkv == 0, Hq / Hkv in {1, 2, 4} */
  int32_t head_dim;            /* d; must be 128 */
  int32_t hidden;              /* D; must equal Hq * d (the recall-head input width; oda_recall_score takes 1024, 2048 or 4096) */
  int32_t sink;                /* s >= 0  (4 in [ODA notes §2.1]) */
  int32_t window;              /* w >= 1  (2048; includes the current token) */
  int32_t kv_layout;           /* ODA_KV_CONTIG or ODA_KV_PAGED */
  int32_t block_size;          /* paged only: tokens per block, power of two */
  int32_t max_blocks_per_seq;  /* paged only: block-table row length */
  int32_t reserved0;           /* must be 0 */
  int64_t t_cap;               /* contiguous only: positions per sequence */
  int64_t num_blocks;          /* paged only: physical blocks per layer */
} oda_dims;

typedef struct oda_kv {
  oda_bf16 *k;                 /* cache keys, layout per kv_layout */
  oda_bf16 *v;                 /* cache values, same layout */
  const int32_t *block_tables; /* paged: [B][max_blocks_per_seq]; contiguous: NULL */
} oda_kv;

/* ---- queries (host only, no device work) ---- */

/* ODA_ABI_VERSION of the loaded library. */
int oda_abi_version(void);

/* Static text for a status code. */
const char *oda_status_str(int status);

/* Number of fp32 parameters of the recall head for input width `hidden`
 * [ODA notes §2.2: 28,325,889 at hidden 2048]; -1 if hidden < 1. */
int64_t oda_head_param_count(int32_t hidden);

/* Float offsets of the ODA_HEAD_NTENSORS packed head tensors, plus the total
 * as entry ODA_HEAD_NTENSORS, written to the host array `offsets`
 * (ODA_HEAD_NTENSORS + 1 entries).  Order (matrices row-major [out][in]):
 *   gamma_H[D] W_H[1024][D] c_H[1024]  gamma_E W_E c_E  gamma_L W_L c_L
 *   W_I[1024][9216] c_I[1024]
 *   gamma_1[1024] Wg_1[2048][1024] Wu_1[2048][1024] Wd_1[1024][2048]
 *   gamma_2 Wg_2 Wu_2 Wd_2
 *   gamma_o[1024] w_o[1024] c_o[1]
 * Returns ODA_E_NULL / ODA_E_DIMS on bad arguments. */
int oda_head_offsets(int32_t hidden, int64_t *offsets);

/* Bytes of device workspace the step needs for `dims` (split partials, the
 * full-branch work list, completion tickets, recall-head activations and
 * the error word).  0 if dims are invalid. */
size_t oda_workspace_bytes(const oda_dims *dims);

/* Byte offset inside the workspace of the full-branch work list: an int32
 * count followed by `count` int32 items,
 * item = (b << 20) | (nsplit << 10) | split, in the order the split policy
 * above states.  Written by oda_recall_score and oda_worklist, read by
 * oda_full_attn_if. */
size_t oda_workspace_worklist_offset(const oda_dims *dims);

/* ---- device work ---- */

/* Clears the error word and the completion tickets of `ws` with a fill
 * kernel (no memset node, so it may be captured).  Call once after
 * allocating a workspace; the kernels leave the tickets cleared. */
int oda_workspace_init(const oda_dims *dims, void *ws, size_t ws_bytes, hipStream_t stream);

/* Local index set as at most two ranges [ODA notes §2.1, S^L_t =
 * {1..min(s,t)} U {max(1,t-w+1)..t}], 0-based: ranges[b] = {a0, a1, b0, b1}
 * with S^L = [a0, a1) U [b0, b1), b0 >= a1; when the two parts touch they
 * are merged into [0, t) and b0 = b1 = t.  ranges: [B][4] int32. */
int oda_local_ranges(const oda_dims *dims, const int32_t *pos, int32_t *ranges, hipStream_t stream);

/* Local-branch GQA decode attention of layer `layer` over S^L for every
 * sequence [ODA notes §2.1 eq. o_t]: the committed rows of the index set
 * come from the cache, the current position from this branch's staged
 * k_cur / v_cur.  Writes every row of `out` (and `lse` if non-NULL). */
int oda_local_attn(const oda_dims *dims, int32_t layer, const oda_kv *kv, const int32_t *pos,
                   const oda_bf16 *q, const oda_bf16 *k_cur, const oda_bf16 *v_cur,
                   oda_bf16 *out, float *lse, void *ws, size_t ws_bytes, hipStream_t stream);

/* Recall score, branch rule and full-branch work list.
 *  score[b] = R(h_prev[b], emb[b], h_local[b])  [ODA notes §2.2 eq. q_t], fp32
 *    head_w: packed fp32 parameters (layout of oda_head_offsets);
 *    h_prev, emb, h_local: [B][D] bf16 -- the previous step's chosen hidden
 *    state, the current token's embedding, and the local branch's last-layer
 *    output (the `out` of oda_local_attn for the last layer).
 *  flag[b] = force[b] >= 0 ? (force[b] != 0)
 *                          : (score[b] > theta || score[b] is not finite)
 *    [ODA notes §2.3]; force may be NULL (all decided by the head).
 *  The work list (see oda_workspace_worklist_offset) lists, for each flagged
 *  b, the splits 0 .. nsplit(pos[b]+1)-1 (split policy and order above). */
int oda_recall_score(const oda_dims *dims, const float *head_w, const oda_bf16 *h_prev,
                     const oda_bf16 *emb, const oda_bf16 *h_local, float theta, const int8_t *force,
                     const int32_t *pos, float *score, uint8_t *flag, void *ws, size_t ws_bytes,
                     hipStream_t stream);

/* Device-side compaction alone: writes the full-branch work list
 * of the workspace from caller-given flags (flag[b] != 0 -> sequence b runs
 * the full branch), exactly as oda_recall_score does after its rule.  For
 * schedules decided outside the head (forced calls, an always-full
 * baseline).  flag, pos: [B]. */
int oda_worklist(const oda_dims *dims, const uint8_t *flag, const int32_t *pos, void *ws, size_t ws_bytes,
                 hipStream_t stream);

/* Full-branch attention of layer `layer` over S^F = [0, pos[b]] for the
 * sequences on the work list [ODA notes §2.1 eq. o_t over S^F; §2.3: the
 * full branch restarts from the same pre-step state, so it reads the cache
 * as committed before this step plus its OWN staged k_cur / v_cur].  Rows
 * of unflagged sequences in `out` / `lse` are left untouched.  Launches a
 * fixed grid whose workgroups read the work list on the device: no host
 * synchronisation, capture-safe. */
int oda_full_attn_if(const oda_dims *dims, int32_t layer, const oda_kv *kv, const int32_t *pos,
                     const oda_bf16 *q, const oda_bf16 *k_cur, const oda_bf16 *v_cur,
                     oda_bf16 *out, float *lse, void *ws, size_t ws_bytes, hipStream_t stream);

/* Commit [ODA notes §2.3 eq. h_t = h_t^{b_t}, C_t = C_{t-1} || dC^{b_t}]:
 * for every sequence b with chosen branch beta = flag[b] ? full : local,
 *   every layer's cache slot pos[b] <- staged k/v of branch beta,
 *   h_prev[b] <- out_last of branch beta (bit copy),
 *   pos[b] += 1.
 * k_cur_L, v_cur_L, k_cur_F, v_cur_F: [L][B][Hkv][d]; out_last_L,
 * out_last_F: [B][D] (the last layer's outputs of the two branches);
 * h_prev: [B][D] output.  A sequence whose slot is out of capacity is left
 * unchanged and raises ODA_ERR_CAPACITY / ODA_ERR_BLOCK. */
int oda_commit(const oda_dims *dims, const oda_kv *kv, int32_t *pos, const uint8_t *flag,
               const oda_bf16 *k_cur_L, const oda_bf16 *v_cur_L, const oda_bf16 *k_cur_F,
               const oda_bf16 *v_cur_F, const oda_bf16 *out_last_L, const oda_bf16 *out_last_F,
               oda_bf16 *h_prev, void *ws, size_t ws_bytes, hipStream_t stream);

/* ---- for callers that cannot allocate ---- */

/* Bytes of the library's fixed per-GPU scratch array used by
 * oda_local_attn_noalloc: 16 MiB, held on each GPU the library runs on until
 * the process ends. */
#define ODA_NOALLOC_SCRATCH_BYTES (16u << 20)

/* oda_local_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, kernels and results as oda_local_attn, with the
 * split partials and completion tickets in the library's fixed scratch array
 * of ODA_NOALLOC_SCRATCH_BYTES instead of a caller workspace.  The caller
 * still passes every input and output.  err: device int32 that receives the
 * sticky device-side error bits (ODA_ERR_*), or NULL to drop them.
 * Returns ODA_E_WORKSPACE, launching nothing, when dims need more scratch
 * than the array holds (split partials of B * Hkv * 16 * (Hq / Hkv) * 528
 * bytes, plus tickets and a 256-byte header).  Calls no allocator.  The
 * first call on a GPU looks the array up and clears its tickets with a fill
 * kernel on `stream`; later calls find them cleared by the kernels.  Every
 * call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (different streams without ordering, or several host threads) race. */
int oda_local_attn_noalloc(const oda_dims *dims, int32_t layer, const oda_kv *kv, const int32_t *pos,
                           const oda_bf16 *q, const oda_bf16 *k_cur, const oda_bf16 *v_cur, oda_bf16 *out,
                           float *lse, int32_t *err, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ODA_H_ */
