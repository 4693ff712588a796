/*
 * moe.h — C ABI of the fused mixture-of-experts (MoE) layer for small token
 * batches on MI355X (gfx950), part of libdcasparse.so.
 *
 * Source: xllm-io paper-review page, section 4 "Inference & deployment",
 * "MoE kernel optimisation" (Figure 8): the serving engine's MoE kernel is
 * memory-bound at generation batch sizes; it keeps the matrix cores busy in
 * that regime and is judged by the memory bandwidth it reaches (3.4 TB/s on
 * H20).  The model table of the same page (section 3) gives SwiGLU as the
 * feed-forward activation.
 *
 * What is computed, for token t with routed experts e_s = topk_ids[t][s] and
 * weights w_s = topk_weights[t][s] (s < top_k):
 *   g = W1_e x_t,  u = W3_e x_t          (d_ff each)
 *   a = silu(g) * u,  silu(z) = z / (1 + exp(-z))
 *   y = W2_e a                          (d_model)
 *   out_t = sum_s w_s * y_s
 * Slots whose expert id lies outside [0, n_experts) contribute nothing (a
 * dropped slot).  The routing itself (router logits, softmax, top-k) is the
 * caller's: ids and weights come in.
 *
 * Layouts (row-major, contiguous, device memory, raw bfloat16 bits):
 *   x            [n_tokens][d_model]
 *   topk_ids     [n_tokens][top_k]   int32
 *   topk_weights [n_tokens][top_k]   float32
 *   w13          [n_experts][2 * d_ff][d_model]: rows 0 .. d_ff-1 are W1
 *                (gate), rows d_ff .. 2 d_ff - 1 are W3 (up)
 *   w2           [n_experts][d_model][d_ff]
 *   out          [n_tokens][d_model]
 * moe_forward reads the weights in a packed layout that moe_pack_weights
 * writes once (same size): each expert matrix W [R][C] is cut into tiles of
 * 32 rows x 64 columns, stored tile row by tile row, and inside a tile the
 * 16-byte piece for MFMA step j (0..3) and lane l (0..63) holds
 * W[32 t + l % 32][64 s + 32 (l / 32) + 8 j .. + 7] at element offset
 * ((t * (C / 64) + s) * 4 + j) * 512 + 8 l.  A wave that owns 32 rows then
 * streams one contiguous region, 1 KB per load instruction.
 * Precision: bf16 operands, fp32 accumulation; the activation a is rounded to
 * bf16 between the two products; out is rounded to bf16 (nearest even).
 *
 * Conventions as in dcasparse.h: the caller owns every buffer, scratch comes
 * from cfg->workspace (moe_workspace_size), work is enqueued on cfg->stream,
 * validation happens before any launch, outputs are bitwise deterministic.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include "dcasparse.h"

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_STAGE_COUNT 4      /* 0: sort of the slots by expert, 1: gate/up product + SwiGLU, 2: down product, 3: weighted sum over slots */

typedef struct moe_cfg {
  int32_t n_tokens;       /* >= 1 */
  int32_t n_experts;      /* 1 .. 1023 */
  int32_t top_k;          /* 1 .. n_experts */
  int32_t d_model;        /* multiple of 128 */
  int32_t d_ff;           /* per-expert intermediate size, multiple of 128 */
  void   *workspace;      /* device scratch, >= moe_workspace_size bytes, 256-byte aligned */
  size_t  workspace_bytes;
  void   *stream;         /* hipStream_t; NULL = the null stream */
  void  **stage_events;   /* optional 2 * MOE_STAGE_COUNT hipEvent_t (start, stop per stage); NULL: none */
} moe_cfg;

/* Workspace bytes of moe_forward: slot order, the bf16 activations of every
 * (token, slot) and their fp32 expert outputs; for batches of a few tokens,
 * whose products run in k parts, the fp32 sums of each part.  Pure host
 * computation. */
DCA_API int moe_workspace_size(const moe_cfg *cfg, size_t *bytes);

/* Writes the packed layout of w13 and w2 (above) into w13_packed and
 * w2_packed (caller-owned, same sizes, not overlapping the sources).  Reads
 * cfg->n_experts, d_model, d_ff and stream; needs no workspace. */
DCA_API int moe_pack_weights(const dca_bf16 *w13, const dca_bf16 *w2, const moe_cfg *cfg, dca_bf16 *w13_packed,
                             dca_bf16 *w2_packed);

/* The fused MoE layer above, with packed weights.  Only the weights of
 * experts that receive a slot are read, each once per 64 of its slots. */
DCA_API int moe_forward(const dca_bf16 *x, const int32_t *topk_ids, const float *topk_weights,
                        const dca_bf16 *w13_packed, const dca_bf16 *w2_packed, const moe_cfg *cfg, dca_bf16 *out);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
