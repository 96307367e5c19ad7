/*
 * oda_decoder.h -- C ABI of the dense decoder step around the ODA path
 * (part of liboda, MI355X / gfx950).
 *
 * The pages run ODA inside a dense Qwen3 backbone kept in BF16 ([ODA notes]
 * §3.3, efficiency paragraph), and both branches recompute the whole
 * backbone for the step from the same pre-step state ([ODA notes] §2.3).
 * These entry points supply that backbone around the attention calls of
 * oda.h, so one decode step of B sequences becomes:
 *
 *   oda_dec_embed                                  x_L = x_F = E[token], e = E[token]
 *   oda_dec_layer(l, LOCAL)  for l = 0 .. L-1      local branch (oda_local_attn inside)
 *   oda_dec_final_norm(LOCAL)                      h^L = RMSNorm(x_L)
 *   oda_recall_score(h_prev, e, h^L)               rule + work list   [oda.h]
 *   oda_dec_layer(l, FULL)   for l = 0 .. L-1      full branch (oda_full_attn_if inside)
 *   oda_dec_final_norm(FULL)                       h^F
 *   oda_dec_next_token                             argmax of E h^{b_t} per sequence
 *   oda_commit(k/v staged per branch, h^L, h^F)    [oda.h]
 *
 * Every FULL-branch kernel reads the work-list count that oda_recall_score
 * (or oda_worklist) wrote into the attention workspace and returns at once
 * when it is zero, so a captured graph of the whole step pays only launch
 * costs on steps that take no full branch.
 *
 * Layer (pre-norm; every stored activation bf16, rounded once, nearest-even):
 *   a   = bf16(gamma_in * x),  r = 1/sqrt(mean(x^2) + eps)
 *   qkv = bf16(r * W_qkv a)                 W_qkv [(Hq + 2 Hkv) d][D]: q rows, k rows, v rows
 *   q_h, k_g = bf16(RoPE(gamma_{q,k} * v / sqrt(mean(v^2) + eps), pos))   per head (QK-norm)
 *   o   = attention of the branch (oda_local_attn / oda_full_attn_if)
 *   x  += W_o o                              W_o [D][Hq d]; x stays fp32
 *   m   = bf16(SiLU(bf16(r2 W_gate a2)) * bf16(r2 W_up a2)),  a2 = bf16(gamma_post * x), r2 = rms scale of x
 *   x  += W_down m                           W_gate, W_up [I][D], W_down [D][I]
 * RoPE rotates the pair (v_i, v_{i+d/2}) by pos * theta^(-2i/d), i < d/2.
 * Final: h = bf16(gamma_f * x / sqrt(mean(x^2) + eps)); logits = E h with the
 * token embedding E [V][D] (tied); next token = smallest index of the maximum.
 *
 * One layer's weights are one bf16 blob, tensors in this order (each
 * row-major, offsets from oda_dec_layer_offsets):
 *   gamma_in[D] W_qkv[(Hq+2Hkv)d][D] gamma_q[d] gamma_k[d] W_o[D][Hq d] gamma_post[D]
 *   W_gate[I][D] W_up[I][D] W_down[D][I]
 *
 * Rules as in oda.h: device pointers owned by the caller (dims and offsets
 * are host pointers), no allocation, no synchronisation, graph-capturable;
 * calls sharing a decoder workspace must be ordered.  Return ODA_OK or a
 * negative ODA_E_* code, nothing launched on error.
 */
#ifndef ODA_DECODER_H_
#define ODA_DECODER_H_

#include "oda.h"

#ifdef __cplusplus
extern "C" {
#endif

#define ODA_DEC_LOCAL 0
#define ODA_DEC_FULL 1
#define ODA_DEC_NTENSORS 9

typedef struct oda_dec_dims {
  oda_dims attn;       /* the attention path's dims (layers, batch, heads, d = 128, D = Hq*d, cache) */
  int32_t inter;       /* I, MLP hidden width; multiple of 1024 */
  int32_t vocab;       /* V, rows of the tied embedding; multiple of 64 */
  float rope_theta;    /* RoPE base (1e6 for the Qwen3 family) */
  float eps;           /* RMSNorm epsilon (1e-6) */
} oda_dec_dims;
/* Also required: D = Hq * d a multiple of 1024 (1024, 2048 or 4096 for the
 * recall head of the step), B <= 32. */

/* bf16 elements of one layer blob; -1 if dims are invalid. */
int64_t oda_dec_layer_numel(const oda_dec_dims *dims);

/* Element offsets of the ODA_DEC_NTENSORS layer tensors, in blob order, plus
 * the total as entry ODA_DEC_NTENSORS, into the host array `offsets`. */
int oda_dec_layer_offsets(const oda_dec_dims *dims, int64_t *offsets);

/* Bytes of the decoder workspace (qkv and MLP activations, split-K partial
 * tiles, tickets, LM-head candidates); 0 if dims are invalid.  Separate
 * from the attention workspace of oda.h. */
size_t oda_dec_workspace_bytes(const oda_dec_dims *dims);

/* Zero the decoder workspace's tickets (once, before first use). */
int oda_dec_workspace_init(const oda_dec_dims *dims, void *dws, size_t dws_bytes, hipStream_t stream);

/* x_local[b], x_full[b] = E[tokens[b]] widened to fp32 ([B][D] each; either
 * may be NULL); emb[b] = E[tokens[b]] (bf16 [B][D], the head's E(x_t)).
 * A token outside [0, V) sets ODA_ERR_TOKEN in the attention workspace's
 * error word (when attn_ws is not NULL) and reads row 0. */
int oda_dec_embed(const oda_dec_dims *dims, const oda_bf16 *embed, const int32_t *tokens, float *x_local,
                  float *x_full, oda_bf16 *emb, void *attn_ws, size_t attn_ws_bytes, hipStream_t stream);

/* One decoder layer of one branch (ODA_DEC_LOCAL or ODA_DEC_FULL) for the
 * whole batch.  x [B][D] fp32 is the branch's residual stream (in/out).
 * Writes the branch's staged k_cur / v_cur [B][Hkv][d] of this layer (what
 * oda_commit writes if the branch is chosen) and the attention output o
 * [B][Hq][d].  The attention is the ODA local / full branch of oda.h with
 * `attn_ws`.  The local branch runs it in a mode that applies the QK-norm
 * and RoPE to the raw projection rows inside the attention kernel, from a
 * table of the step's RoPE angles that its layer 0 writes into `dws`, so a
 * local pass starts at layer 0 (the order below); the full branch applies
 * them in a kernel of its own.  q (device, [B][Hq][d]) is scratch: the full
 * branch writes it, the local branch does not, and it must be non-NULL. */
int oda_dec_layer(const oda_dec_dims *dims, int32_t layer, int32_t branch, const oda_bf16 *w_layer,
                  const oda_kv *kv, const int32_t *pos, float *x, oda_bf16 *q, oda_bf16 *k_cur,
                  oda_bf16 *v_cur, oda_bf16 *o, void *attn_ws, size_t attn_ws_bytes, void *dws,
                  size_t dws_bytes, hipStream_t stream);

/* h = bf16(gamma_f * x / rms(x)) per row ([B][D]); the FULL branch's call
 * does nothing when the work list is empty. */
int oda_dec_final_norm(const oda_dec_dims *dims, int32_t branch, const oda_bf16 *gamma_f, const float *x,
                       oda_bf16 *h, void *attn_ws, size_t attn_ws_bytes, hipStream_t stream);

/* tokens[b] = argmax_v (E h_b)_v with h_b = flag[b] ? h_full[b] : h_local[b]
 * (smallest index on ties); max_logit[b] (fp32, nullable) is that maximum. */
int oda_dec_next_token(const oda_dec_dims *dims, const oda_bf16 *embed, const oda_bf16 *h_local,
                       const oda_bf16 *h_full, const uint8_t *flag, int32_t *tokens, float *max_logit, void *dws,
                       size_t dws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* ODA_DECODER_H_ */
