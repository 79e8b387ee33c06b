/*
 * moe_lora.h - C ABI of the MoE-LoRA expert layer for AMD MI355X (gfx950).
 *
 * The layer is the training forward and backward of one mixture-of-experts
 * MLP block whose stacked expert weights carry LoRA adapters:
 *
 *   route     top-k experts per token from router logits, and combine weights
 *   permute   (token, slot) pairs grouped by expert; rows gathered in that order
 *   experts   per expert e, over its rows X:
 *               h   = X W_gu[e]^T + s (X A_gu[e]^T) B_gu[e]^T     gate_up [E, 2I, H]
 *               act = silu(h[:, :I]) * h[:, I:]                    SwiGLU
 *               y   = act W_d[e]^T + s (act A_d[e]^T) B_d[e]^T     down    [E, H, I]
 *   combine   Y[t] = sum_j w[t, j] y[pos(t, j)]
 *
 * and the backward producing dX, d logits and the LoRA gradients dA, dB with
 * the base weights frozen. The adapter is applied in the "split" order, input
 * times A first and then B, so W + s B A is never formed.
 *
 * Sources: Unsloth, "Fine-tune MoE models 12x faster" (unsloth.ai docs,
 * faster-moe page): section "What is torch._grouped_mm?" for the per-expert
 * loop, the gate/up chunk and the stacked gate_up_proj [E, 2I, H] parameter;
 * section "Faster LoRA MoE training" for the split order (same outputs and
 * gradients, products reordered by associativity); section "Implementation
 * details" for the LoRA shapes (m, r), (r, n), the frozen router and the
 * per-expert cost model. The SwiGLU form (gate e, e * sigmoid(e), times up)
 * is the fused LoRA MLP definition in the aiflowlearn.net Unsloth tutorial,
 * section on the LoRA fine-tuning principle.
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers to row-major, contiguous memory that
 *    the caller allocates and owns. The library allocates and frees nothing,
 *    and never synchronises the stream: every call only enqueues kernels on
 *    `stream` (a hipStream_t; NULL means the default stream) and returns.
 *  - Shapes: T tokens, H hidden, I intermediate, E experts, k experts per
 *    token, r LoRA rank, N = T * k routed rows.
 *  - dtype (moe_shape.dtype) is the element type of x, the weights, the LoRA
 *    parameters, the saved activations, Y, dY, dX and the LoRA gradients:
 *    MOE_F32 (float), MOE_BF16 (bfloat16) or MOE_F16 (IEEE half, for parts
 *    whose grouped GEMM runs in float16: the faster-moe page's
 *    acknowledgements section credits float16 grouped_mm support for T4
 *    and A100). The 16-bit types share every kernel: only the MFMA
 *    instruction and the rounding of stored values differ. Products
 *    accumulate in float32. Router logits, combine weights and their
 *    gradients are always float32; indices are int32.
 *  - Outputs are fully overwritten (gradients are not accumulated into).
 *  - Token-row buffers that the gather and combine kernels move in 16-byte
 *    pieces start on a 16-byte boundary (any torch allocation does): x and
 *    x_perm of moe_permute, y_perm and y (or dx_perm and dx) of
 *    moe_unpermute_combine, dy, y_exp and dy_perm of the combine backwards.
 *    Weights and the other activations may sit anywhere (unaligned operands
 *    take element-wise loads).
 *  - Arguments are checked before anything is enqueued. Errors:
 *      MOE_ERR_INVALID_ARG   a NULL pointer that is not optional, T < 1,
 *                            k < 1, k > E, E < 1, E > 1024, H < 1, I < 1,
 *                            r < 1, N >= 2^31, N * max(2I, H) bytes of
 *                            `dtype` above 32 GiB (one activation tensor),
 *                            2I * H bytes of `dtype` at or above 2 GiB (one
 *                            expert's weight matrix), unknown router or dtype
 *                            or a token-row buffer (below) off a 16-byte
 *                            boundary
 *      MOE_ERR_UNSUPPORTED   H or I not a multiple of 8, r > 64, k > 32
 *      MOE_ERR_WORKSPACE     workspace smaller than moe_workspace_bytes says
 *      MOE_ERR_HIP           a launch failed (moe_last_error() has the text)
 *    Faults inside kernels surface at the caller's next synchronisation.
 *  - Entry points keep no state between calls (the optional kernel timer
 *    below aside), so calls on different streams may run concurrently if
 *    their buffers do not overlap.
 */
#ifndef MOE_LORA_H
#define MOE_LORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE = 3,
  MOE_ERR_HIP = 4
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_F16 = 2 } moe_dtype;

/* Router modes (how combine weights follow from the logits of the k chosen
 * experts; the choice itself is always the k largest logits, ties to the
 * lower expert index, ordered by logit descending):
 *   MOE_SOFTMAX_TOPK         w_j = softmax(logits)[S_j]
 *   MOE_SOFTMAX_TOPK_RENORM  w_j = softmax(logits)[S_j] / sum_j softmax(logits)[S_j]
 *   MOE_TOPK_SOFTMAX         w   = softmax(logits[S])
 *   MOE_SIGMOID_TOPK_RENORM  w_j = sigmoid(logits[S_j]) / sum_j sigmoid(logits[S_j])  */
typedef enum {
  MOE_SOFTMAX_TOPK = 0,
  MOE_SOFTMAX_TOPK_RENORM = 1,
  MOE_TOPK_SOFTMAX = 2,
  MOE_SIGMOID_TOPK_RENORM = 3
} moe_router;

/* lora_scale is s above (alpha / r in the usual LoRA parameterisation). */
typedef struct {
  int32_t T, H, I, E, k, r;
  int32_t dtype;      /* moe_dtype */
  float lora_scale;
} moe_shape;

/* Frozen base weights and LoRA parameters, all of `dtype`:
 *   w_gu [E, 2I, H]  (rows 0..I-1 gate, I..2I-1 up)   a_gu [E, r, H]   b_gu [E, 2I, r]
 *   w_d  [E, H, I]                                     a_d  [E, r, I]   b_d  [E, H, r]  */
typedef struct {
  const void *w_gu, *a_gu, *b_gu, *w_d, *a_d, *b_d;
} moe_weights;

/* Activations the forward writes and the backward reads, all of `dtype`,
 * rows in permuted (expert-grouped) order:
 *   h     [N, 2I]  gate_up output before SwiGLU
 *   act   [N, I]   SwiGLU output (input of down)
 *   u_gu  [N, r]   s * X A_gu^T   (the scaled LoRA side product of gate_up)
 *   u_d   [N, r]   s * act A_d^T  (the scaled LoRA side product of down)
 *   y_exp [N, H]   per-row expert output before the combine weights  */
typedef struct {
  void *h, *act, *u_gu, *u_d, *y_exp;
} moe_saved;

/* LoRA gradients, shapes of the parameters, all of `dtype`. Experts that
 * received no rows get zeros. */
typedef struct {
  void *da_gu, *db_gu, *da_d, *db_d;
} moe_lora_grads;

/* Base-weight gradients for full fine-tuning, shapes of the weights, all of
 * `dtype`:  dw_gu [E, 2I, H]   dw_d [E, H, I]. Experts that received no rows
 * get zeros. */
typedef struct {
  void *dw_gu, *dw_d;
} moe_base_grads;

/* Bytes of device scratch each call needs (0 is possible). Host-only, no HIP
 * call. Any pointer may be NULL to skip that figure. */
moe_status moe_workspace_bytes(const moe_shape *shape, size_t *fwd_ws, size_t *bwd_ws,
                               size_t *permute_ws);

/* Top-k routing (faster-moe page, "What is torch._grouped_mm?": the expert
 * mask the per-expert loop walks).
 *   logits   [T, E] float32 in
 *   topk_ids [T, k] int32 out: chosen experts, logit descending, ties to lower index
 *   topk_w   [T, k] float32 out: combine weights per `router`  */
moe_status moe_route(const float *logits, int32_t T, int32_t E, int32_t k, int32_t router,
                     int32_t *topk_ids, float *topk_w, void *stream);

/* Gradient of the routing weights with respect to the logits, the selection
 * held fixed (the router is frozen, faster-moe page, "Implementation
 * details", so this is the only router gradient).
 *   d_topk_w [T, k] float32 in;  d_logits [T, E] float32 out (zeros where the
 *   mode gives none)  */
moe_status moe_route_bwd(const float *logits, const int32_t *topk_ids, const float *d_topk_w,
                         int32_t T, int32_t E, int32_t k, int32_t router, float *d_logits,
                         void *stream);

/* Group the N (token, slot) pairs by expert, stably in pair order p = t*k + j
 * (the per-expert token_idx of the faster-moe page's loop), and gather rows.
 *   topk_ids    [T, k] int32 in, each in [0, E)
 *   x           [T, H] dtype in (may be NULL when x_perm is NULL)
 *   counts      [E] int32 out     rows per expert
 *   offsets     [E+1] int32 out   exclusive prefix sum; expert e owns rows
 *                                 offsets[e] .. offsets[e+1]-1
 *   sorted_pair [N] int32 out     pair at each permuted row
 *   inv_pos     [N] int32 out     permuted row of each pair
 *   x_perm      [N, H] dtype out  x[sorted_pair[i] / k]; NULL skips the gather
 *   ws          permute workspace (moe_workspace_bytes)  */
moe_status moe_permute(const moe_shape *shape, const int32_t *topk_ids, const void *x,
                       int32_t *counts, int32_t *offsets, int32_t *sorted_pair,
                       int32_t *inv_pos, void *x_perm, void *ws, size_t ws_bytes,
                       void *stream);

/* moe_permute without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops or harnesses
 * that forbid hipMalloc). Same arguments, outputs and results as moe_permute;
 * its per-chunk expert counts live in a library-owned device array of
 * MOE_PERMUTE_NOALLOC_BYTES per GPU (its first call on a GPU looks up that
 * GPU's copy; the array is held until the process ends). The GPU is the one
 * current on the calling thread, and `stream` must belong to it.
 *   Limit: E * ceil(T * k / 64) * 4 bytes <= MOE_PERMUTE_NOALLOC_BYTES, else
 *   MOE_ERR_UNSUPPORTED (checked before anything is enqueued).
 *   Calls on one GPU share the array: calls on one stream are ordered and
 *   safe, calls that overlap in time on one GPU (different streams, or host
 *   threads) race and give wrong results. Every call rewrites the part of the
 *   array it uses before reading it. Allocates nothing.  */
#define MOE_PERMUTE_NOALLOC_BYTES (4u << 20)
moe_status moe_permute_noalloc(const moe_shape *shape, const int32_t *topk_ids, const void *x,
                               int32_t *counts, int32_t *offsets, int32_t *sorted_pair,
                               int32_t *inv_pos, void *x_perm, void *stream);

/* Grouped expert forward with split LoRA and SwiGLU (faster-moe page, "Faster
 * LoRA MoE training" and "Implementation details"): fills every field of
 * `saved` for rows in permuted order. offsets is moe_permute's output.  */
moe_status moe_grouped_lora_fwd(const moe_shape *shape, const void *x_perm,
                                const int32_t *offsets, const moe_weights *weights,
                                const moe_saved *saved, void *ws, size_t ws_bytes,
                                void *stream);

/* Y[t] = sum_{j<k} w[t, j] * y_perm[inv_pos[t*k + j]], accumulated in float32
 * in slot order. topk_w NULL means all weights 1 (the plain sum that brings
 * dX_perm back to tokens).
 *   y_perm [N, H] dtype in, inv_pos [N] in, topk_w [T, k] float32 in, y [T, H] out  */
moe_status moe_unpermute_combine(const moe_shape *shape, const void *y_perm,
                                 const int32_t *inv_pos, const float *topk_w, void *y,
                                 void *stream);

/* Backward of the combine:
 *   dy_perm[inv_pos[t*k+j]] = w[t, j] * dy[t]          [N, H] dtype out
 *   d_topk_w[t, j] = <dy[t], y_exp[inv_pos[t*k+j]]>    [T, k] float32 out  */
moe_status moe_unpermute_combine_bwd(const moe_shape *shape, const void *dy,
                                     const void *y_exp, const int32_t *inv_pos,
                                     const float *topk_w, void *dy_perm, float *d_topk_w,
                                     void *stream);

/* Grouped expert backward, base weights frozen: from dy_perm (the combine
 * backward's output) and the saved activations, writes dx_perm [N, H] and the
 * four LoRA gradients.  */
moe_status moe_grouped_lora_bwd(const moe_shape *shape, const void *dy_perm,
                                const void *x_perm, const int32_t *offsets,
                                const moe_weights *weights, const moe_saved *saved,
                                void *dx_perm, const moe_lora_grads *grads, void *ws,
                                size_t ws_bytes, void *stream);

/* Grouped expert backward for full fine-tuning (the faster-moe page lists
 * full fine-tuning beside LoRA and QLoRA among the modes its kernels serve,
 * in its introduction, and recommends bf16 LoRA or full fine-tuning for MoE
 * models in its note on 4-bit QLoRA): everything moe_grouped_lora_bwd
 * writes, plus the base-weight gradients
 *   dW_gu[e] = dH_e^T X_e      [2I, H]   (dH = gradient at the gate_up output)
 *   dW_d[e]  = G_e^T act_e     [H, I]    (G = dy_perm rows of expert e)
 * each a reduction over the expert's rows, written in full (no accumulation).
 * Same arguments, workspace and errors as moe_grouped_lora_bwd; `base` and
 * both its pointers must be non-NULL and may not alias any other buffer.  */
moe_status moe_grouped_full_bwd(const moe_shape *shape, const void *dy_perm,
                                const void *x_perm, const int32_t *offsets,
                                const moe_weights *weights, const moe_saved *saved,
                                void *dx_perm, const moe_lora_grads *grads,
                                const moe_base_grads *base, void *ws, size_t ws_bytes,
                                void *stream);

/* Activation-lean mode for long contexts (the faster-moe page claims longer
 * contexts from lower memory in its introduction and gpt-oss benchmark
 * section, and its usage example at the end of "Faster LoRA MoE training"
 * turns on gradient checkpointing to cut memory): the forward keeps
 * h and act in its own workspace instead of `saved`, and the backward
 * recomputes them from x_perm and the saved u_gu with the same gate_up
 * kernel, so only u_gu, u_d and y_exp are held between forward and backward
 * (h [N, 2I] and act [N, I] are not). Outputs and gradients are bit-identical
 * to the saving mode; the backward does one more gate_up GEMM.
 *   moe_workspace_bytes_lean  workspace sizes of the two calls below
 *   moe_grouped_lora_fwd_lean    as moe_grouped_lora_fwd; saved->h and
 *                                saved->act are not used (may be NULL)
 *   moe_grouped_lora_bwd_recompute  as moe_grouped_lora_bwd (base NULL) or
 *                                moe_grouped_full_bwd (base non-NULL), from the
 *                                lean forward's saved fields
 * Same argument rules and errors as the saving-mode calls.  */
moe_status moe_workspace_bytes_lean(const moe_shape *shape, size_t *fwd_ws, size_t *bwd_ws);
moe_status moe_grouped_lora_fwd_lean(const moe_shape *shape, const void *x_perm,
                                     const int32_t *offsets, const moe_weights *weights,
                                     const moe_saved *saved, void *ws, size_t ws_bytes,
                                     void *stream);
moe_status moe_grouped_lora_bwd_recompute(const moe_shape *shape, const void *dy_perm,
                                          const void *x_perm, const int32_t *offsets,
                                          const moe_weights *weights, const moe_saved *saved,
                                          void *dx_perm, const moe_lora_grads *grads,
                                          const moe_base_grads *base, void *ws, size_t ws_bytes,
                                          void *stream);

/* The combine backward folded into the experts' backward, in one call: it
 * replaces moe_unpermute_combine_bwd followed by moe_grouped_lora_bwd (or
 * moe_grouped_full_bwd, or moe_grouped_lora_bwd_recompute with recompute != 0)
 * and gives the same results, but never forms G = w dY and does not read
 * y_exp, so y_exp [N, H] need not be kept from the forward (the combine's
 * output Y is all the forward must leave). It uses, by the chain rule through
 * the combine (the layer's output) and the split down projection (faster-moe
 * page, "Faster LoRA MoE training": the same gradients with the products
 * reordered),
 *   dw[t, j] = <dY[t], y_exp[p]> = <dY[t] W_d + s (dY[t] B_d) A_d, act[p]>
 * for p = inv_pos[t*k+j] and the pair's expert: the unweighted product of the
 * down backward, already formed there, dotted with the SwiGLU output it
 * recomputes from h; the weight w[t, j] is applied to that product before the
 * SwiGLU derivative and to the LoRA operands (dB_d = dY^T (w u_d), dA_d from
 * w s dY B_d).
 *   dy          [T, H] dtype in
 *   topk_w      [T, k] float32 in;  sorted_pair, inv_pos [N] int32 in (moe_route,
 *               moe_permute outputs); offsets [E+1] as for moe_grouped_lora_bwd
 *   saved       h, act (unless recompute), u_gu, u_d; y_exp is not read
 *   recompute   0: saving-mode forward; else the lean forward's saved fields
 *               (h and act recomputed in `ws`, as moe_grouped_lora_bwd_recompute)
 *   dy_perm     [N, H] dtype scratch, written: dy's rows in permuted order
 *               (unweighted; with base, scaled by w before dW_d is formed)
 *   dx_perm, grads, base (NULL: LoRA only)  as moe_grouped_lora_bwd /
 *               moe_grouped_full_bwd
 *   d_topk_w    [T, k] float32 out (the routing-weight gradient moe_route_bwd takes)
 *   ws          backward workspace: moe_workspace_bytes' bwd_ws, or
 *               moe_workspace_bytes_lean's when recompute != 0
 * Errors as moe_grouped_lora_bwd, plus a NULL dy, topk_w, sorted_pair,
 * inv_pos or d_topk_w, and dy_perm aliasing dy, x_perm or dx_perm.  */
moe_status moe_grouped_lora_combine_bwd(const moe_shape *shape, const void *dy,
                                        const float *topk_w, const int32_t *sorted_pair,
                                        const int32_t *inv_pos, const void *x_perm,
                                        const int32_t *offsets, const moe_weights *weights,
                                        const moe_saved *saved, int32_t recompute,
                                        void *dy_perm, void *dx_perm,
                                        const moe_lora_grads *grads, const moe_base_grads *base,
                                        float *d_topk_w, void *ws, size_t ws_bytes,
                                        void *stream);

/* The layer input read in token order (faster-moe page, "Implementation
 * details": the LoRA products run on the routed pairs only; here the expert
 * GEMMs also fetch each pair's row of x themselves, so x_perm is never
 * formed). x is [T, H] of `dtype` in token order, and row i of the permuted
 * order is row sorted_pair[i] / k of x (sorted_pair from moe_permute, which
 * can then be called with x_perm = NULL). The GEMMs that read x_perm in the
 * calls above (gate_up, its LoRA side product X A_gu^T, dA_gu and, with base,
 * dW_gu) read those rows of x instead. In the backward, dy_perm = NULL has
 * the GEMMs that read dY's rows in permuted order (the down backward, dB_d
 * and its side product dY B_d) read row sorted_pair[i] / k of dy likewise,
 * so no permuted copy is formed (MOE_ERR_INVALID_ARG with base, whose dW_d
 * needs w dY in permuted order, and for H <= 32); otherwise dy_perm is
 * written as in moe_grouped_lora_combine_bwd. Which is faster depends on the
 * shape: the copy streams well, the gathered reads skip it. Everything else,
 * and every result, is as in
 * moe_grouped_lora_fwd / moe_grouped_lora_fwd_lean (lean != 0) and
 * moe_grouped_lora_combine_bwd. Errors as those calls, plus a NULL
 * sorted_pair, and MOE_ERR_UNSUPPORTED when x is 2 GiB or larger (use x_perm
 * and the calls above).  */
moe_status moe_grouped_lora_fwd_gather(const moe_shape *shape, const void *x,
                                       const int32_t *sorted_pair, const int32_t *offsets,
                                       const moe_weights *weights, const moe_saved *saved,
                                       int32_t lean, void *ws, size_t ws_bytes, void *stream);
moe_status moe_grouped_lora_combine_bwd_gather(const moe_shape *shape, const void *dy,
                                               const float *topk_w, const int32_t *sorted_pair,
                                               const int32_t *inv_pos, const void *x,
                                               const int32_t *offsets, const moe_weights *weights,
                                               const moe_saved *saved, int32_t recompute,
                                               void *dy_perm, void *dx_perm,
                                               const moe_lora_grads *grads,
                                               const moe_base_grads *base, float *d_topk_w,
                                               void *ws, size_t ws_bytes, void *stream);

/* Router projection and its input gradient, for callers that start from
 * hidden states rather than logits. The pages keep the router frozen (faster-
 * moe page, "Implementation details"), so there is no router weight
 * gradient; the logits' gradient flows back into x:
 *   logits = x W_r^T        x [T, H] dtype, w_r [E, H] dtype, logits [T, E] float32
 *   dx    += d_logits W_r   d_logits [T, E] float32 in, dx [T, H] dtype accumulated
 * Float32 accumulation (bf16 layers: d_logits is rounded to bf16 to feed the
 * MFMA; dx is read, added to in float32 and rounded once). ws is the router
 * workspace (moe_router_workspace_bytes). Errors as for the layer calls; H
 * must be a multiple of 8 and 1 <= E <= 1024.  */
moe_status moe_router_workspace_bytes(int32_t T, int32_t H, int32_t E, int32_t dtype,
                                      size_t *ws_bytes);
moe_status moe_router_fwd(const void *x, const void *w_r, int32_t T, int32_t H, int32_t E,
                          int32_t dtype, float *logits, void *ws, size_t ws_bytes, void *stream);
moe_status moe_router_bwd(const float *d_logits, const void *w_r, int32_t T, int32_t H,
                          int32_t E, int32_t dtype, void *dx, void *ws, size_t ws_bytes,
                          void *stream);

/* Merged export of the adapters into the base weights, for inference or
 * saving a merged 16-bit model (the winningdata.io hands-on page, section
 * "4. Salvando o modelo", saves with the merged 16-bit method), per expert e:
 *   w_gu_merged[e] = w_gu[e] + s b_gu[e] a_gu[e]     [2I, H]
 *   w_d_merged[e]  = w_d[e]  + s b_d[e]  a_d[e]      [H, I]
 * where s = shape->lora_scale. The product is formed in float32 and the sum is
 * rounded once to `dtype`. Only E, H, I, r, dtype and lora_scale of `shape`
 * are read (T and k are ignored). Either output may be NULL (that projection
 * is skipped), and an output may be the base weight itself (in-place merge);
 * an output may not alias a LoRA parameter or the other projection. ws is the
 * merge workspace (moe_merge_workspace_bytes). Errors as for the layer calls;
 * E * max(2I, H) must be below 2^31.  */
moe_status moe_merge_workspace_bytes(const moe_shape *shape, size_t *ws_bytes);
moe_status moe_merge_lora(const moe_shape *shape, const moe_weights *weights, void *w_gu_merged,
                          void *w_d_merged, void *ws, size_t ws_bytes, void *stream);

/* dst[i] += src[i] for i < n, elements of `dtype`, sum in float32, one
 * rounding (adds a shared expert's output to the routed output, and its input
 * gradient to dx). src and dst may not overlap (MOE_ERR_INVALID_ARG).  */
moe_status moe_accumulate(int32_t dtype, int64_t n, const void *src, void *dst, void *stream);

const char *moe_status_str(moe_status status);

/* Text of the last error raised on the calling thread ("" if none). */
const char *moe_last_error(void);

/* Optional per-kernel timer (for measurement; off by default). While enabled,
 * the library records a HIP event pair on the launch stream around each
 * launch of the kernels listed in moe_kernel_id. moe_kernel_timer_read must be
 * called after the caller has synchronised those streams; it returns the
 * summed milliseconds and the number of launches since the last reset. Not
 * thread-safe against concurrent launches; meant for a benchmark loop. */
typedef enum {
  MOE_K_ROUTE = 0, MOE_K_PERMUTE = 1, MOE_K_GATHER = 2, MOE_K_GATE_UP_FWD = 3,
  MOE_K_DOWN_FWD = 4, MOE_K_COMBINE = 5, MOE_K_COMBINE_BWD = 6, MOE_K_ROUTE_BWD = 7,
  MOE_K_DOWN_BWD = 8, MOE_K_GATE_UP_BWD = 9, MOE_K_LORA_SIDE = 10, MOE_K_LORA_WGRAD = 11,
  MOE_K_UNPERMUTE = 12, MOE_K_BASE_WGRAD = 13, MOE_K_ROUTER_FWD = 14, MOE_K_ROUTER_BWD = 15,
  MOE_K_ACCUMULATE = 16, MOE_K_MERGE = 17, MOE_K_DY_GATHER = 18, MOE_K_DW_SUM = 19,
  MOE_K_ROW_SCALE = 20, MOE_K_COUNT = 21
} moe_kernel_id;
moe_status moe_kernel_timer_enable(int32_t on);
/* Time only the kernels whose bit (1u << id) is set in mask (all, by default):
 * a timed region can bracket just the kernel it reports with events, while the
 * other kernels are timed in a pass of their own. */
moe_status moe_kernel_timer_select(uint32_t mask);
moe_status moe_kernel_timer_reset(void);
moe_status moe_kernel_timer_read(int32_t kernel_id, double *total_ms, int32_t *launches);

#ifdef __cplusplus
}
#endif

#endif /* MOE_LORA_H */
