/*
 * oda_hybrid.h -- C ABI of the recurrent-state transaction of a hybrid
 * backbone (part of liboda, MI355X / gfx950).
 *
 * Source: the page "On-Demand Attention：让语言模型按需读取完整历史", cited
 * as [ODA notes]: §2.3 (the state-commit paragraph and the equation for
 * C_t) and §3.3 (the cross-model paragraph).  In a hybrid backbone only the
 * full-attention layers are restricted to S^L (oda.h); the recurrent layers
 * keep their native computation in both branches.  Their convolution and
 * recurrent states must be saved before the local trial and restored before
 * the full retry, and only the chosen branch's update is committed.
 *
 * Layer (the pages leave it open; a gated delta rule decode layer, d_k =
 * d_v = d = 128, causal depthwise convolution of width W over the C = 3 H d
 * channels of the q | k | v projection):
 *   c        = sum_{j < W-1} w[:, j] s_j + w[:, W-1] x_t          (s_0 oldest)
 *   q, k, v  = SiLU(c), channel groups [0, Hd), [Hd, 2Hd), [2Hd, 3Hd), head h
 *              taking channels [h d, (h + 1) d) of each group
 *   q^, k^   = q / sqrt(|q|^2 + 1e-6), k / sqrt(|k|^2 + 1e-6)
 *   S'       = alpha S + beta (v - alpha S k^) k^T       S in R^{d x d}, [v index][k index]
 *   o        = S' q^ / sqrt(d)
 *   new convolution state (s_1, ..., s_{W-2}, x_t)
 * fp32 state, gates and arithmetic; bf16 inputs, weights, convolution state
 * (it holds past inputs) and outputs.
 *
 * Transaction.  The state pool keeps three slots per (layer, sequence).
 * slot[b] (uint8, one per sequence, shared by all layers) names the
 * committed slot c, which holds the pre-step state.  oda_gdn_step with
 * ODA_GDN_LOCAL reads slot c and writes slot (c + 1) mod 3; with
 * ODA_GDN_FULL it runs only for sequences with flag[b] != 0, reads slot c
 * and writes slot (c + 2) mod 3.  The full retry therefore starts from the
 * pre-step state whatever the local trial did ("restore"), and
 * oda_gdn_commit makes the chosen branch's slot the committed one: c <-
 * (c + 1 + flag[b]) mod 3.  Nothing is copied.
 *
 * Layouts (row-major, innermost last): state pool = recurrent part
 * [L][B][3][H][d][d] fp32, then (at oda_gdn_conv_offset) the convolution
 * part [L][B][3][W-1][C] bf16; x [B][C] bf16; conv_w [C][W] bf16; alpha,
 * beta [B][H] fp32; out [B][H][d] bf16.
 *
 * Order within a step: oda_gdn_step(LOCAL) for every recurrent layer,
 * oda_recall_score (oda.h), oda_gdn_step(FULL) for every recurrent layer,
 * then oda_gdn_commit (once per step, after every FULL call) next to
 * oda_commit.
 *
 * Rules as in oda.h: device pointers owned by the caller (dims is a host
 * pointer read during the call), no allocation, no synchronisation,
 * graph-capturable.  Return ODA_OK or a negative ODA_E_* code, nothing
 * launched on error.  slot values are taken modulo 3.
 */
#ifndef ODA_HYBRID_H_
#define ODA_HYBRID_H_

#include "oda.h"

#ifdef __cplusplus
extern "C" {
#endif

#define ODA_GDN_LOCAL 0
#define ODA_GDN_FULL 1
#define ODA_GDN_SLOTS 3

typedef struct oda_gdn_dims {
  int32_t num_layers;   /* recurrent layers in the pool, >= 1 */
  int32_t batch;        /* B, 1 .. 1024 */
  int32_t heads;        /* H, 1 .. 64 */
  int32_t head_dim;     /* d = d_k = d_v; 128 */
  int32_t conv_width;   /* W, 2 .. 8 (4 in the Qwen hybrid family) */
} oda_gdn_dims;

/* Bytes of the state pool (recurrent part, then convolution part); 0 if
 * dims are invalid. */
size_t oda_gdn_state_bytes(const oda_gdn_dims *dims);

/* Byte offset of the convolution part inside the pool; 0 if dims are
 * invalid. */
size_t oda_gdn_conv_offset(const oda_gdn_dims *dims);

/* One recurrent layer of one branch for every sequence (ODA_GDN_FULL: the
 * flagged ones; flag may be NULL for ODA_GDN_LOCAL). */
int oda_gdn_step(const oda_gdn_dims *dims, int32_t layer, int32_t branch, void *state, const uint8_t *slot,
                 const uint8_t *flag, const oda_bf16 *x, const oda_bf16 *conv_w, const float *alpha,
                 const float *beta, oda_bf16 *out, hipStream_t stream);

/* slot[b] <- (slot[b] + 1 + (flag[b] != 0)) mod 3 for every sequence. */
int oda_gdn_commit(const oda_gdn_dims *dims, uint8_t *slot, const uint8_t *flag, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ODA_HYBRID_H_ */
