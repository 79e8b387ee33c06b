// Internal host-side interface between the C ABI (api.hip) and the kernel
// files. Not installed; the public interface is include/moe_lora.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_lora.h"  // include/ is on the compiler include path

namespace moe {

// Optional event timer around kernel launches (see moe_kernel_timer_* in the
// public header). A null KernelTimer* disables it.
class KernelTimer {
 public:
  void record_start(int id, hipStream_t s);
  void record_stop(int id, hipStream_t s);
};
KernelTimer* active_timer();

struct TimedScope {
  KernelTimer* tm;
  int id;
  hipStream_t s;
  TimedScope(KernelTimer* t, int i, hipStream_t st) : tm(t), id(i), s(st) {
    if (tm) tm->record_start(id, s);
  }
  ~TimedScope() {
    if (tm) tm->record_stop(id, s);
  }
};

// ---- routing
hipError_t launch_route(const float* logits, int T, int E, int k, int router, int32_t* ids,
                        float* w, hipStream_t s);
hipError_t launch_route_bwd(const float* logits, const int32_t* ids, const float* dw, int T,
                            int E, int k, int router, float* dlogits, hipStream_t s);

// ---- permutation
size_t permute_ws_bytes(int64_t N, int E);
// The current GPU's copy of the moe_permute_noalloc table
// (MOE_PERMUTE_NOALLOC_BYTES), looked up on the first call on each GPU.
hipError_t noalloc_permute_table(int32_t** table);
hipError_t launch_permute(const int32_t* ids, int64_t N, int E, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_pair, int32_t* inv_pos,
                          int32_t* table, hipStream_t s, KernelTimer* tm);
hipError_t launch_gather(const void* x, const int32_t* sorted_pair, const int32_t* offsets,
                         int E, int k, int64_t N, int64_t row_bytes, void* x_perm,
                         hipStream_t s, KernelTimer* tm);

// ---- combine
hipError_t launch_combine(int dtype, const void* y_perm, const int32_t* inv_pos, const float* w,
                          int T, int k, int H, void* y, hipStream_t s, KernelTimer* tm);
hipError_t launch_combine_bwd(int dtype, const void* dy, const void* y_exp,
                              const int32_t* inv_pos, const float* w, int T, int k, int H,
                              void* g, float* dw, hipStream_t s, KernelTimer* tm);

// Folded combine backward: w_perm[i] = w[sorted_pair[i]] (the routing weight
// of each permuted row) and wu[i][c] = w_perm[i] u[i][c] ([N, r] of `dtype`);
// d_topk_w[p] = sum over slots s (in order) of dwp[inv_pos[p] * slots + s]
// (0 where inv_pos[p] < 0).
hipError_t launch_perm_weights(int dtype, const float* w, const int32_t* sorted_pair, int64_t N,
                               const void* u, int r, float* w_perm, void* wu, hipStream_t s);
hipError_t launch_dw_sum(const float* dwp, int slots, const int32_t* inv_pos, int64_t npairs,
                         float* d_topk_w, hipStream_t s);

// ---- grouped expert GEMMs
// A token-row activation as the expert GEMMs read it (x, and dY in the
// backward): [N, H] in permuted order (rows null, e.g. x_perm), or [T, H] in
// token order, row i of the permuted order being token rows[i] / k
// (rows = sorted_pair; the GEMMs gather it).
struct XRows {
  const void* ptr;
  const int32_t* rows;
  int k, T;
};

struct ExpertDims {
  int64_t N;  // routed rows
  int H, I, E, r, dtype;
  float scale;
};

size_t experts_fwd_ws_bytes(const ExpertDims& d);
size_t experts_bwd_ws_bytes(const ExpertDims& d);

hipError_t launch_experts_fwd(const ExpertDims& d, const XRows& x, const int32_t* offsets,
                              const moe_weights& w, const moe_saved& sv, void* ws,
                              hipStream_t s, KernelTimer* tm);
// The combine backward folded into the experts' backward: G = w dY is never
// formed. dY's rows are gathered unweighted (in permuted order) into the
// caller's g buffer, the routing weights are applied inside the kernels, and
// dw = <dY, y_exp> is taken in the down backward's epilogue as <dAct', act>
// with dAct' the unweighted product (so y_exp need not be kept).
struct CombineBwd {
  const void* dy;        // [T, H]
  const float* topk_w;   // [T, k]
  const int32_t* sorted_pair;
  const int32_t* inv_pos;
  int T, k;
  float* d_topk_w;       // [T, k] out
  // The GEMMs read dY's rows through sorted_pair and g is not written (not
  // with base: the base-weight gradient needs w dY in expert order).
  bool gather_dy = false;
};

// `base` may be null (LoRA only); otherwise the base-weight gradients are written too.
// `cb` null: g holds G = w dY rows (read only). Otherwise g is an [N, H]
// buffer the call fills with dY's rows (unused with cb->gather_dy), and cb's
// d_topk_w is written.
hipError_t launch_experts_bwd(const ExpertDims& d, const void* g, const XRows& x,
                              const int32_t* offsets, const moe_weights& w,
                              const moe_saved& sv, void* dx_perm, const moe_lora_grads& gr,
                              const moe_base_grads* base, void* ws, hipStream_t s,
                              KernelTimer* tm, const CombineBwd* cb = nullptr);

// Recompute (activation-lean) mode: the forward keeps h and act in its
// workspace instead of `saved`; the backward recomputes them into its own.
size_t experts_fwd_lean_ws_bytes(const ExpertDims& d);
size_t experts_bwd_lean_ws_bytes(const ExpertDims& d);
hipError_t launch_experts_fwd_lean(const ExpertDims& d, const XRows& x,
                                   const int32_t* offsets, const moe_weights& w,
                                   const moe_saved& sv, void* ws, hipStream_t s,
                                   KernelTimer* tm);
hipError_t launch_experts_bwd_recompute(const ExpertDims& d, const void* g, const XRows& x,
                                        const int32_t* offsets, const moe_weights& w,
                                        const moe_saved& sv, void* dx_perm,
                                        const moe_lora_grads& gr, const moe_base_grads* base,
                                        void* ws, hipStream_t s, KernelTimer* tm,
                                        const CombineBwd* cb = nullptr);

// ---- merged export W + s B A (per expert, both projections; either output may be NULL)
size_t merge_ws_bytes(const ExpertDims& d);
hipError_t launch_merge(const ExpertDims& d, const moe_weights& w, void* w_gu_out, void* w_d_out,
                        void* ws, hipStream_t s, KernelTimer* tm);

// ---- router projection and element-wise accumulate
size_t router_ws_bytes(int T, int E, int dtype);
hipError_t launch_router_fwd(const void* x, const void* w_r, int T, int H, int E, int dtype,
                             float* logits, void* ws, hipStream_t s, KernelTimer* tm);
hipError_t launch_router_bwd(const float* d_logits, const void* w_r, int T, int H, int E,
                             int dtype, void* dx, void* ws, hipStream_t s, KernelTimer* tm);
hipError_t launch_accumulate(int dtype, int64_t n, const void* src, void* dst, hipStream_t s,
                             KernelTimer* tm);

}  // namespace moe
