/*
 * oda_train.h -- C ABI of one recall-head training step (part of liboda,
 * MI355X / gfx950).
 *
 * Source: the page "On-Demand Attention：让语言模型按需读取完整历史", cited
 * as [ODA notes]: §2.1 (equation for the gain g), §2.2 (equations for d, y
 * and the loss L; the paragraph on paired supervision).
 *
 * Only the recall head R_psi is trained; the backbone, the embedding and
 * the LM head are frozen and only produce features and supervision
 * ([ODA notes] §2.2, loss paragraph).  A micro-batch is N rows, one per
 * position of one or more sequences.  For row n the caller supplies the two
 * candidates' final hidden states at that position, both computed from the
 * same committed history, h^L (local index set) and h^F (full index set),
 * the current token x_t, the reference next token x_{t+1}, the 0-based
 * position and the row of the previous position.  A step is two calls:
 *
 *   oda_train_labels     log p^B(x) = (E h^B)[x] - logsumexp(E h^B), B in {L, F}
 *                        g = log p^F(x_{t+1}) - log p^L(x_{t+1})     [ODA notes §2.1]
 *                        d = g - lambda;  y = sign(d) log(1 + |d|)   [ODA notes §2.2]
 *                        valid = reference token present, g finite and
 *                                pos >= s + w (the index sets differ, t > s + w)
 *   oda_train_head_step  h_prev(n) = 0 when prev[n] < 0 (a sequence start), else
 *                                    h^F[prev] if d[prev] > 0 or d[prev] is not
 *                                    finite, h^L[prev] otherwise
 *                        q = R_psi(h_prev, E[x_t], h^L)              [ODA notes §2.2]
 *                        L = (1/|valid|) sum over valid rows of Huber_1(q - y)
 *                        grad = dL/dpsi for every packed head parameter
 *
 * The previous-state rule is a reading: the pages pick the previous state by
 * the previous position's reference benefit, taken here as the branch the
 * deployed rule would pick for a score with that benefit's sign.  A
 * micro-batch without valid rows has L = 0 and a zero gradient.  |x| is
 * differentiated as sign(x), 0 at 0.  The pages name no optimiser; the step
 * ends at the gradient.
 *
 * Precision: E and the hidden states are bf16 (the backbone's precision),
 * logits accumulate in fp32, the log-sum-exp and the labels are fp32; the
 * head, its activations and its gradient are fp32 ([ODA notes] §3.3: the
 * head runs in FP32).
 *
 * Layouts (row-major, innermost index last): lm_head [V][D] bf16 (the tied
 * token embedding, also read for E[x_t]); h_local, h_full [N][D] bf16;
 * next_tok, tokens, pos, prev [N] int32; gain, label, score [N] fp32; valid
 * [N] uint8; head_w and grad: the packed fp32 head of oda.h
 * (oda_head_offsets); loss: one fp32.
 *
 * Rules as in oda.h: device pointers owned by the caller (dims is a host
 * pointer read during the call), no allocation, no synchronisation,
 * graph-capturable; calls sharing a workspace must be ordered.  Return
 * ODA_OK or a negative ODA_E_* code, nothing launched on error.  A token id
 * outside [0, V) (other than next_tok = -1) sets ODA_ERR_TOKEN in the error
 * word at byte 0 of the workspace (clear it with oda_train_workspace_init);
 * such a row is treated as having no reference token (oda_train_labels) or
 * a zero embedding (oda_train_head_step).
 */
#ifndef ODA_TRAIN_H_
#define ODA_TRAIN_H_

#include "oda.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct oda_train_dims {
  int32_t rows;     /* N, rows of the micro-batch, 1 .. 65536 */
  int32_t hidden;   /* D, a multiple of 256 (2048 for Qwen3-1.7B) */
  int32_t vocab;    /* V, rows of the tied LM head, >= 1 */
  int32_t sink;     /* s = 4 */
  int32_t window;   /* w = 2048 */
  float lambda;     /* call penalty, >= 0 ([ODA notes] §2.2: 0 or 0.001) */
} oda_train_dims;

/* Bytes of the training workspace (activations of the head for the
 * backward pass, split-K partials, log-sum-exp partials, the error word);
 * 0 if dims are invalid. */
size_t oda_train_workspace_bytes(const oda_train_dims *dims);

/* Clears the error word of the training workspace. */
int oda_train_workspace_init(const oda_train_dims *dims, void *ws, size_t ws_bytes, hipStream_t stream);

/* Labels of the N rows: gain g, label y and membership of the valid set.
 * Rows with next_tok = -1 get g = y = 0 and valid = 0. */
int oda_train_labels(const oda_train_dims *dims, const oda_bf16 *lm_head, const oda_bf16 *h_local,
                     const oda_bf16 *h_full, const int32_t *next_tok, const int32_t *pos, float *gain,
                     float *label, uint8_t *valid, void *ws, size_t ws_bytes, hipStream_t stream);

/* Forward, loss and backward of the recall head on the N rows, given their
 * labels.  prev[n] is the row of position t-1 of the same sequence, or -1 at
 * a sequence start; it must index a row of this micro-batch.  Writes score
 * (q of every row), loss, and every element of grad. */
int oda_train_head_step(const oda_train_dims *dims, const float *head_w, const oda_bf16 *lm_head,
                        const oda_bf16 *h_local, const oda_bf16 *h_full, const int32_t *tokens,
                        const int32_t *prev, const float *gain, const float *label, const uint8_t *valid,
                        float *score, float *loss, float *grad, void *ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ODA_TRAIN_H_ */
