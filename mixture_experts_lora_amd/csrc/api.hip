// C ABI of the MoE-LoRA expert layer: argument checks, workspace carving and
// launches on the caller's stream. Declarations and the contract of every
// entry point are in include/moe_lora.h.
#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "launch.h"

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status st, const std::string& what) {
  g_last_error = what;
  return st;
}

moe_status hip_fail(hipError_t e, const char* where) {
  return fail(MOE_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

#define CHECK_PTR(p)                                                                  \
  do {                                                                                \
    if ((p) == nullptr) return fail(MOE_ERR_INVALID_ARG, "null pointer: " #p);        \
  } while (0)

// Token-row buffers that the row kernels (gather, combine and their
// backwards) move in 16-byte pieces must start on a 16-byte boundary.
#define CHECK_ROWS(p)                                                                 \
  do {                                                                                \
    if ((reinterpret_cast<uintptr_t>(p) & 15) != 0)                                   \
      return fail(MOE_ERR_INVALID_ARG, #p " does not start on a 16-byte boundary");   \
  } while (0)

moe_status check_router(int32_t router) {
  if (router < MOE_SOFTMAX_TOPK || router > MOE_SIGMOID_TOPK_RENORM)
    return fail(MOE_ERR_INVALID_ARG, "unknown router mode " + std::to_string(router));
  return MOE_OK;
}

moe_status check_routing_dims(int64_t T, int64_t E, int64_t k) {
  if (T < 1) return fail(MOE_ERR_INVALID_ARG, "T must be >= 1");
  if (E < 1 || E > 1024) return fail(MOE_ERR_INVALID_ARG, "E must be in [1, 1024]");
  if (k < 1 || k > E) return fail(MOE_ERR_INVALID_ARG, "k must be in [1, E]");
  if (k > 32) return fail(MOE_ERR_UNSUPPORTED, "k > 32 is not supported");
  if (T * k >= (int64_t(1) << 31)) return fail(MOE_ERR_INVALID_ARG, "T*k must be < 2^31");
  return MOE_OK;
}

moe_status check_shape(const moe_shape* s) {
  if (!s) return fail(MOE_ERR_INVALID_ARG, "null shape");
  moe_status st = check_routing_dims(s->T, s->E, s->k);
  if (st != MOE_OK) return st;
  if (s->H < 1 || s->I < 1) return fail(MOE_ERR_INVALID_ARG, "H and I must be >= 1");
  if (s->r < 1) return fail(MOE_ERR_INVALID_ARG, "r must be >= 1");
  if (s->dtype != MOE_F32 && s->dtype != MOE_BF16 && s->dtype != MOE_F16)
    return fail(MOE_ERR_INVALID_ARG, "unknown dtype " + std::to_string(s->dtype));
  if (s->H % 8 != 0 || s->I % 8 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "H and I must be multiples of 8");
  if (s->r > 64) return fail(MOE_ERR_UNSUPPORTED, "r > 64 is not supported");
  // Activation tensors up to 32 GiB each, so that their 16-byte chunk
  // indices fit 32 bits in the element-wise kernels; one expert's weight
  // matrix below 2 GiB, the reach of a 32-bit buffer offset in the GEMMs.
  const int64_t N = int64_t(s->T) * s->k;
  const int64_t esz = s->dtype == MOE_F32 ? 4 : 2;
  const int64_t wide = std::max(2 * int64_t(s->I), int64_t(s->H));
  if (N * wide * esz > (int64_t(1) << 35))
    return fail(MOE_ERR_INVALID_ARG, "activation tensors larger than 32 GiB");
  if (2 * int64_t(s->I) * s->H * esz >= (int64_t(1) << 31))
    return fail(MOE_ERR_INVALID_ARG, "one expert's weight matrix must be smaller than 2 GiB");
  return MOE_OK;
}

moe::ExpertDims dims_of(const moe_shape* s) {
  moe::ExpertDims d;
  d.N = int64_t(s->T) * s->k;
  d.H = s->H;
  d.I = s->I;
  d.E = s->E;
  d.r = s->r;
  d.dtype = s->dtype;
  d.scale = s->lora_scale;
  return d;
}

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// ---------------------------------------------------------------- kernel timer
struct TimerRec {
  int id;
  hipEvent_t a, b;
};

struct TimerState {
  std::mutex mu;
  bool on = false;
  uint32_t mask = 0xffffffffu;  // kernel ids timed while on
  std::vector<TimerRec> recs;
  std::vector<hipEvent_t> pool;
  std::vector<int> open;  // index into recs of the pending start, per id
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};

TimerState& timer() {
  static TimerState t;
  return t;
}

moe::KernelTimer g_timer_handle;

}  // namespace

namespace moe {

KernelTimer* active_timer() { return timer().on ? &g_timer_handle : nullptr; }

void KernelTimer::record_start(int id, hipStream_t s) {
  TimerState& t = timer();
  std::lock_guard<std::mutex> lk(t.mu);
  if (!((t.mask >> id) & 1u)) return;
  if (t.open.size() < MOE_K_COUNT) t.open.assign(MOE_K_COUNT, -1);
  hipEvent_t a = t.get(), b = t.get();
  if (!a || !b) return;
  hipEventRecord(a, s);
  t.recs.push_back(TimerRec{id, a, b});
  t.open[id] = static_cast<int>(t.recs.size()) - 1;
}

void KernelTimer::record_stop(int id, hipStream_t s) {
  TimerState& t = timer();
  std::lock_guard<std::mutex> lk(t.mu);
  if (t.open.size() < MOE_K_COUNT || t.open[id] < 0) return;
  hipEventRecord(t.recs[t.open[id]].b, s);
  t.open[id] = -1;
}

}  // namespace moe

extern "C" {

const char* moe_status_str(moe_status st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

moe_status moe_workspace_bytes(const moe_shape* shape, size_t* fwd_ws, size_t* bwd_ws,
                               size_t* permute_ws) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe::ExpertDims d = dims_of(shape);
  if (fwd_ws) *fwd_ws = moe::experts_fwd_ws_bytes(d);
  if (bwd_ws) *bwd_ws = moe::experts_bwd_ws_bytes(d);
  if (permute_ws) *permute_ws = moe::permute_ws_bytes(d.N, d.E);
  return MOE_OK;
}

moe_status moe_workspace_bytes_lean(const moe_shape* shape, size_t* fwd_ws, size_t* bwd_ws) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe::ExpertDims d = dims_of(shape);
  if (fwd_ws) *fwd_ws = moe::experts_fwd_lean_ws_bytes(d);
  if (bwd_ws) *bwd_ws = moe::experts_bwd_lean_ws_bytes(d);
  return MOE_OK;
}

moe_status moe_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t router,
                     int32_t* topk_ids, float* topk_w, void* stream) {
  moe_status st = check_routing_dims(T, E, k);
  if (st != MOE_OK) return st;
  if ((st = check_router(router)) != MOE_OK) return st;
  CHECK_PTR(logits);
  CHECK_PTR(topk_ids);
  CHECK_PTR(topk_w);
  moe::TimedScope ts(moe::active_timer(), MOE_K_ROUTE, as_stream(stream));
  hipError_t e = moe::launch_route(logits, T, E, k, router, topk_ids, topk_w, as_stream(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_route");
}

moe_status moe_route_bwd(const float* logits, const int32_t* topk_ids, const float* d_topk_w,
                         int32_t T, int32_t E, int32_t k, int32_t router, float* d_logits,
                         void* stream) {
  moe_status st = check_routing_dims(T, E, k);
  if (st != MOE_OK) return st;
  if ((st = check_router(router)) != MOE_OK) return st;
  CHECK_PTR(logits);
  CHECK_PTR(topk_ids);
  CHECK_PTR(d_topk_w);
  CHECK_PTR(d_logits);
  if (static_cast<const void*>(d_logits) == static_cast<const void*>(logits))
    return fail(MOE_ERR_INVALID_ARG, "d_logits aliases logits");
  moe::TimedScope ts(moe::active_timer(), MOE_K_ROUTE_BWD, as_stream(stream));
  hipError_t e = moe::launch_route_bwd(logits, topk_ids, d_topk_w, T, E, k, router, d_logits,
                                       as_stream(stream));
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_route_bwd");
}

moe_status moe_permute(const moe_shape* shape, const int32_t* topk_ids, const void* x,
                       int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                       int32_t* inv_pos, void* x_perm, void* ws, size_t ws_bytes,
                       void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  CHECK_PTR(topk_ids);
  CHECK_PTR(counts);
  CHECK_PTR(offsets);
  CHECK_PTR(sorted_pair);
  CHECK_PTR(inv_pos);
  if (x_perm) {
    CHECK_PTR(x);
    CHECK_ROWS(x);
    CHECK_ROWS(x_perm);
  }
  if (x_perm && x_perm == x) return fail(MOE_ERR_INVALID_ARG, "x_perm aliases x");
  const moe::ExpertDims d = dims_of(shape);
  const size_t need = moe::permute_ws_bytes(d.N, d.E);
  if (need > 0) CHECK_PTR(ws);
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "permute workspace needs " + std::to_string(need) + " bytes");
  hipStream_t s = as_stream(stream);
  moe::KernelTimer* tm = moe::active_timer();
  hipError_t e = moe::launch_permute(topk_ids, d.N, d.E, counts, offsets, sorted_pair, inv_pos,
                                     static_cast<int32_t*>(ws), s, tm);
  if (e != hipSuccess) return hip_fail(e, "moe_permute");
  if (x_perm) {
    const int64_t row_bytes = int64_t(d.H) * (d.dtype == MOE_F32 ? 4 : 2);
    e = moe::launch_gather(x, sorted_pair, offsets, d.E, shape->k, d.N, row_bytes, x_perm, s, tm);
    if (e != hipSuccess) return hip_fail(e, "moe_permute(gather)");
  }
  return MOE_OK;
}

moe_status moe_permute_noalloc(const moe_shape* shape, const int32_t* topk_ids, const void* x,
                               int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                               int32_t* inv_pos, void* x_perm, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  CHECK_PTR(topk_ids);
  CHECK_PTR(counts);
  CHECK_PTR(offsets);
  CHECK_PTR(sorted_pair);
  CHECK_PTR(inv_pos);
  if (x_perm) {
    CHECK_PTR(x);
    CHECK_ROWS(x);
    CHECK_ROWS(x_perm);
  }
  if (x_perm && x_perm == x) return fail(MOE_ERR_INVALID_ARG, "x_perm aliases x");
  const moe::ExpertDims d = dims_of(shape);
  const size_t need = moe::permute_ws_bytes(d.N, d.E);
  if (need > MOE_PERMUTE_NOALLOC_BYTES)
    return fail(MOE_ERR_UNSUPPORTED, "moe_permute_noalloc: E * ceil(T*k/64) * 4 = " +
                                         std::to_string(need) + " bytes exceeds its " +
                                         std::to_string(MOE_PERMUTE_NOALLOC_BYTES) +
                                         "-byte table; use moe_permute with a workspace");
  int32_t* table = nullptr;
  hipError_t e = moe::noalloc_permute_table(&table);
  if (e != hipSuccess) return hip_fail(e, "moe_permute_noalloc(table lookup)");
  hipStream_t s = as_stream(stream);
  moe::KernelTimer* tm = moe::active_timer();
  e = moe::launch_permute(topk_ids, d.N, d.E, counts, offsets, sorted_pair, inv_pos, table, s, tm);
  if (e != hipSuccess) return hip_fail(e, "moe_permute_noalloc");
  if (x_perm) {
    const int64_t row_bytes = int64_t(d.H) * (d.dtype == MOE_F32 ? 4 : 2);
    e = moe::launch_gather(x, sorted_pair, offsets, d.E, shape->k, d.N, row_bytes, x_perm, s, tm);
    if (e != hipSuccess) return hip_fail(e, "moe_permute_noalloc(gather)");
  }
  return MOE_OK;
}

namespace {

// x rows read by the GEMMs through sorted_pair: one buffer resource spans x
moe_status check_gather(const moe_shape* shape, const int32_t* sorted_pair) {
  CHECK_PTR(sorted_pair);
  const int64_t bytes = int64_t(shape->T) * shape->H * (shape->dtype == MOE_F32 ? 4 : 2);
  if (bytes >= (int64_t{1} << 31))
    return fail(MOE_ERR_UNSUPPORTED, "x of " + std::to_string(bytes) +
                                         " bytes: gathered rows need x below 2 GiB (use x_perm)");
  return MOE_OK;
}

// x_perm: x_perm, or x in token order when sorted_pair is given (gathered)
moe_status grouped_fwd(const char* name, bool lean, const moe_shape* shape, const void* x_perm,
                       const int32_t* sorted_pair, const int32_t* offsets,
                       const moe_weights* weights, const moe_saved* saved, void* ws,
                       size_t ws_bytes, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  CHECK_PTR(x_perm);
  if (sorted_pair) {
    st = check_gather(shape, sorted_pair);
    if (st != MOE_OK) return st;
  }
  CHECK_PTR(offsets);
  CHECK_PTR(weights);
  CHECK_PTR(saved);
  CHECK_PTR(weights->w_gu);
  CHECK_PTR(weights->a_gu);
  CHECK_PTR(weights->b_gu);
  CHECK_PTR(weights->w_d);
  CHECK_PTR(weights->a_d);
  CHECK_PTR(weights->b_d);
  if (!lean) {
    CHECK_PTR(saved->h);
    CHECK_PTR(saved->act);
  }
  CHECK_PTR(saved->u_gu);
  CHECK_PTR(saved->u_d);
  CHECK_PTR(saved->y_exp);
  CHECK_PTR(ws);
  const moe::ExpertDims d = dims_of(shape);
  const size_t need = lean ? moe::experts_fwd_lean_ws_bytes(d) : moe::experts_fwd_ws_bytes(d);
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "forward workspace needs " + std::to_string(need) + " bytes");
  if ((!lean && (saved->h == x_perm || saved->act == x_perm)) || saved->y_exp == x_perm)
    return fail(MOE_ERR_INVALID_ARG, "a saved activation aliases x_perm");
  const moe::XRows x{x_perm, sorted_pair, shape->k, shape->T};
  hipError_t e = lean ? moe::launch_experts_fwd_lean(d, x, offsets, *weights, *saved, ws,
                                                     as_stream(stream), moe::active_timer())
                      : moe::launch_experts_fwd(d, x, offsets, *weights, *saved, ws,
                                                as_stream(stream), moe::active_timer());
  return e == hipSuccess ? MOE_OK : hip_fail(e, name);
}

}  // namespace

moe_status moe_grouped_lora_fwd(const moe_shape* shape, const void* x_perm,
                                const int32_t* offsets, const moe_weights* weights,
                                const moe_saved* saved, void* ws, size_t ws_bytes,
                                void* stream) {
  return grouped_fwd("moe_grouped_lora_fwd", false, shape, x_perm, nullptr, offsets, weights,
                     saved, ws, ws_bytes, stream);
}

moe_status moe_grouped_lora_fwd_lean(const moe_shape* shape, const void* x_perm,
                                     const int32_t* offsets, const moe_weights* weights,
                                     const moe_saved* saved, void* ws, size_t ws_bytes,
                                     void* stream) {
  return grouped_fwd("moe_grouped_lora_fwd_lean", true, shape, x_perm, nullptr, offsets, weights,
                     saved, ws, ws_bytes, stream);
}

moe_status moe_grouped_lora_fwd_gather(const moe_shape* shape, const void* x,
                                       const int32_t* sorted_pair, const int32_t* offsets,
                                       const moe_weights* weights, const moe_saved* saved,
                                       int32_t lean, void* ws, size_t ws_bytes, void* stream) {
  CHECK_PTR(sorted_pair);
  return grouped_fwd("moe_grouped_lora_fwd_gather", lean != 0, shape, x, sorted_pair, offsets,
                     weights, saved, ws, ws_bytes, stream);
}

moe_status moe_unpermute_combine(const moe_shape* shape, const void* y_perm,
                                 const int32_t* inv_pos, const float* topk_w, void* y,
                                 void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  CHECK_PTR(y_perm);
  CHECK_PTR(inv_pos);
  CHECK_PTR(y);
  CHECK_ROWS(y_perm);
  CHECK_ROWS(y);
  if (y == y_perm) return fail(MOE_ERR_INVALID_ARG, "y aliases y_perm");
  hipError_t e = moe::launch_combine(shape->dtype, y_perm, inv_pos, topk_w, shape->T, shape->k,
                                     shape->H, y, as_stream(stream), moe::active_timer());
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_unpermute_combine");
}

moe_status moe_unpermute_combine_bwd(const moe_shape* shape, const void* dy,
                                     const void* y_exp, const int32_t* inv_pos,
                                     const float* topk_w, void* dy_perm, float* d_topk_w,
                                     void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  CHECK_PTR(dy);
  CHECK_PTR(y_exp);
  CHECK_PTR(inv_pos);
  CHECK_PTR(topk_w);
  CHECK_PTR(dy_perm);
  CHECK_PTR(d_topk_w);
  CHECK_ROWS(dy);
  CHECK_ROWS(y_exp);
  CHECK_ROWS(dy_perm);
  if (dy_perm == dy || dy_perm == y_exp)
    return fail(MOE_ERR_INVALID_ARG, "dy_perm aliases an input");
  hipError_t e = moe::launch_combine_bwd(shape->dtype, dy, y_exp, inv_pos, topk_w, shape->T,
                                         shape->k, shape->H, dy_perm, d_topk_w,
                                         as_stream(stream), moe::active_timer());
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_unpermute_combine_bwd");
}

namespace {

moe_status grouped_bwd_check(bool lean, const moe_shape* shape, const void* dy_perm,
                             const void* x_perm, const int32_t* offsets,
                             const moe_weights* weights, const moe_saved* saved, void* dx_perm,
                             const moe_lora_grads* grads, const moe_base_grads* base, void* ws,
                             size_t ws_bytes) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  CHECK_PTR(dy_perm);
  CHECK_PTR(x_perm);
  CHECK_PTR(offsets);
  CHECK_PTR(weights);
  CHECK_PTR(saved);
  CHECK_PTR(grads);
  CHECK_PTR(dx_perm);
  CHECK_PTR(weights->w_gu);
  CHECK_PTR(weights->a_gu);
  CHECK_PTR(weights->b_gu);
  CHECK_PTR(weights->w_d);
  CHECK_PTR(weights->a_d);
  CHECK_PTR(weights->b_d);
  if (!lean) {
    CHECK_PTR(saved->h);
    CHECK_PTR(saved->act);
  }
  CHECK_PTR(saved->u_gu);
  CHECK_PTR(saved->u_d);
  CHECK_PTR(grads->da_gu);
  CHECK_PTR(grads->db_gu);
  CHECK_PTR(grads->da_d);
  CHECK_PTR(grads->db_d);
  CHECK_PTR(ws);
  if (dx_perm == dy_perm || dx_perm == x_perm)
    return fail(MOE_ERR_INVALID_ARG, "dx_perm aliases an input");
  if (base) {
    CHECK_PTR(base->dw_gu);
    CHECK_PTR(base->dw_d);
    const void* outs[] = {dx_perm, grads->da_gu, grads->db_gu, grads->da_d, grads->db_d};
    const void* ins[] = {dy_perm, x_perm, weights->w_gu, weights->w_d, lean ? nullptr : saved->act,
                         lean ? nullptr : saved->h};
    for (const void* b : {static_cast<const void*>(base->dw_gu), static_cast<const void*>(base->dw_d)}) {
      for (const void* o : outs)
        if (b == o) return fail(MOE_ERR_INVALID_ARG, "a base gradient aliases another output");
      for (const void* i : ins)
        if (b == i) return fail(MOE_ERR_INVALID_ARG, "a base gradient aliases an input");
    }
    if (base->dw_gu == base->dw_d)
      return fail(MOE_ERR_INVALID_ARG, "dw_gu and dw_d alias");
  }
  const moe::ExpertDims d = dims_of(shape);
  const size_t need = lean ? moe::experts_bwd_lean_ws_bytes(d) : moe::experts_bwd_ws_bytes(d);
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "backward workspace needs " + std::to_string(need) + " bytes");
  return MOE_OK;
}

moe_status grouped_bwd(const char* name, bool lean, const moe_shape* shape,
                       const void* dy_perm, const void* x_perm, const int32_t* offsets,
                       const moe_weights* weights, const moe_saved* saved, void* dx_perm,
                       const moe_lora_grads* grads, const moe_base_grads* base, void* ws,
                       size_t ws_bytes, void* stream) {
  moe_status st = grouped_bwd_check(lean, shape, dy_perm, x_perm, offsets, weights, saved,
                                    dx_perm, grads, base, ws, ws_bytes);
  if (st != MOE_OK) return st;
  const moe::ExpertDims d = dims_of(shape);
  const moe::XRows x{x_perm, nullptr, shape->k, shape->T};
  hipError_t e =
      lean ? moe::launch_experts_bwd_recompute(d, dy_perm, x, offsets, *weights, *saved,
                                               dx_perm, *grads, base, ws, as_stream(stream),
                                               moe::active_timer())
           : moe::launch_experts_bwd(d, dy_perm, x, offsets, *weights, *saved, dx_perm,
                                     *grads, base, ws, as_stream(stream), moe::active_timer());
  return e == hipSuccess ? MOE_OK : hip_fail(e, name);
}

}  // namespace

moe_status moe_grouped_lora_bwd(const moe_shape* shape, const void* dy_perm,
                                const void* x_perm, const int32_t* offsets,
                                const moe_weights* weights, const moe_saved* saved,
                                void* dx_perm, const moe_lora_grads* grads, void* ws,
                                size_t ws_bytes, void* stream) {
  return grouped_bwd("moe_grouped_lora_bwd", false, shape, dy_perm, x_perm, offsets, weights,
                     saved, dx_perm, grads, nullptr, ws, ws_bytes, stream);
}

moe_status moe_grouped_full_bwd(const moe_shape* shape, const void* dy_perm,
                                const void* x_perm, const int32_t* offsets,
                                const moe_weights* weights, const moe_saved* saved,
                                void* dx_perm, const moe_lora_grads* grads,
                                const moe_base_grads* base, void* ws, size_t ws_bytes,
                                void* stream) {
  CHECK_PTR(base);
  return grouped_bwd("moe_grouped_full_bwd", false, shape, dy_perm, x_perm, offsets, weights,
                     saved, dx_perm, grads, base, ws, ws_bytes, stream);
}

moe_status moe_grouped_lora_bwd_recompute(const moe_shape* shape, const void* dy_perm,
                                          const void* x_perm, const int32_t* offsets,
                                          const moe_weights* weights, const moe_saved* saved,
                                          void* dx_perm, const moe_lora_grads* grads,
                                          const moe_base_grads* base, void* ws,
                                          size_t ws_bytes, void* stream) {
  return grouped_bwd("moe_grouped_lora_bwd_recompute", true, shape, dy_perm, x_perm, offsets,
                     weights, saved, dx_perm, grads, base, ws, ws_bytes, stream);
}

namespace {

// gather: x_perm is x in token order, its rows read through sorted_pair
moe_status combine_bwd_impl(const char* name, bool gather, const moe_shape* shape,
                            const void* dy, const float* topk_w, const int32_t* sorted_pair,
                            const int32_t* inv_pos, const void* x_perm, const int32_t* offsets,
                            const moe_weights* weights, const moe_saved* saved, int32_t recompute,
                            void* dy_perm, void* dx_perm, const moe_lora_grads* grads,
                            const moe_base_grads* base, float* d_topk_w, void* ws,
                            size_t ws_bytes, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (gather) {
    st = check_gather(shape, sorted_pair);
    if (st != MOE_OK) return st;
  }
  CHECK_PTR(dy);
  CHECK_PTR(topk_w);
  CHECK_PTR(sorted_pair);
  CHECK_PTR(inv_pos);
  CHECK_PTR(d_topk_w);
  CHECK_ROWS(dy);
  const bool lean = recompute != 0;
  // Reading x in token order, a NULL dy_perm asks the GEMMs to read dY's rows
  // in place too; not with the base-weight gradients (dW_d needs w dY in
  // expert order), nor for H <= 32 (no tile shape of the dB_d gradient gathers).
  const bool gather_dy = gather && dy_perm == nullptr;
  if (gather_dy && base)
    return fail(MOE_ERR_INVALID_ARG, "dy_perm is required with base-weight gradients");
  if (gather_dy && shape->H <= 32) return fail(MOE_ERR_INVALID_ARG, "dy_perm is required for H <= 32");
  if (!gather_dy) {
    CHECK_ROWS(dy_perm);
    if (dy_perm == dy || dy_perm == x_perm || dy_perm == dx_perm)
      return fail(MOE_ERR_INVALID_ARG, "dy_perm aliases another tensor");
  }
  // the expert part: the same checks as the separate backward calls (the dY
  // rows take the place of the G input)
  st = grouped_bwd_check(lean, shape, gather_dy ? dy : dy_perm, x_perm, offsets, weights, saved,
                         dx_perm, grads, base, ws, ws_bytes);
  if (st != MOE_OK) return st;
  const moe::ExpertDims d = dims_of(shape);
  moe::CombineBwd cb;
  cb.dy = dy;
  cb.topk_w = topk_w;
  cb.sorted_pair = sorted_pair;
  cb.inv_pos = inv_pos;
  cb.T = shape->T;
  cb.k = shape->k;
  cb.d_topk_w = d_topk_w;
  cb.gather_dy = gather_dy;
  const moe::XRows x{x_perm, gather ? sorted_pair : nullptr, shape->k, shape->T};
  hipError_t e =
      lean ? moe::launch_experts_bwd_recompute(d, dy_perm, x, offsets, *weights, *saved,
                                               dx_perm, *grads, base, ws, as_stream(stream),
                                               moe::active_timer(), &cb)
           : moe::launch_experts_bwd(d, dy_perm, x, offsets, *weights, *saved, dx_perm,
                                     *grads, base, ws, as_stream(stream), moe::active_timer(),
                                     &cb);
  return e == hipSuccess ? MOE_OK : hip_fail(e, name);
}

}  // namespace

moe_status moe_grouped_lora_combine_bwd(const moe_shape* shape, const void* dy,
                                        const float* topk_w, const int32_t* sorted_pair,
                                        const int32_t* inv_pos, const void* x_perm,
                                        const int32_t* offsets, const moe_weights* weights,
                                        const moe_saved* saved, int32_t recompute,
                                        void* dy_perm, void* dx_perm,
                                        const moe_lora_grads* grads, const moe_base_grads* base,
                                        float* d_topk_w, void* ws, size_t ws_bytes,
                                        void* stream) {
  return combine_bwd_impl("moe_grouped_lora_combine_bwd", false, shape, dy, topk_w, sorted_pair,
                          inv_pos, x_perm, offsets, weights, saved, recompute, dy_perm, dx_perm,
                          grads, base, d_topk_w, ws, ws_bytes, stream);
}

moe_status moe_grouped_lora_combine_bwd_gather(const moe_shape* shape, const void* dy,
                                               const float* topk_w, const int32_t* sorted_pair,
                                               const int32_t* inv_pos, const void* x,
                                               const int32_t* offsets, const moe_weights* weights,
                                               const moe_saved* saved, int32_t recompute,
                                               void* dy_perm, void* dx_perm,
                                               const moe_lora_grads* grads,
                                               const moe_base_grads* base, float* d_topk_w,
                                               void* ws, size_t ws_bytes, void* stream) {
  return combine_bwd_impl("moe_grouped_lora_combine_bwd_gather", true, shape, dy, topk_w,
                          sorted_pair, inv_pos, x, offsets, weights, saved, recompute, dy_perm,
                          dx_perm, grads, base, d_topk_w, ws, ws_bytes, stream);
}

namespace {

moe_status check_router_dims(int32_t T, int32_t H, int32_t E, int32_t dtype) {
  if (T < 1 || H < 1 || E < 1 || E > 1024)
    return fail(MOE_ERR_INVALID_ARG, "need T >= 1, H >= 1, 1 <= E <= 1024");
  if (dtype != MOE_F32 && dtype != MOE_BF16 && dtype != MOE_F16)
    return fail(MOE_ERR_INVALID_ARG, "unknown dtype");
  if (H % 8 != 0) return fail(MOE_ERR_UNSUPPORTED, "H must be a multiple of 8");
  return MOE_OK;
}

}  // namespace

moe_status moe_router_workspace_bytes(int32_t T, int32_t H, int32_t E, int32_t dtype,
                                      size_t* ws_bytes) {
  moe_status st = check_router_dims(T, H, E, dtype);
  if (st != MOE_OK) return st;
  CHECK_PTR(ws_bytes);
  *ws_bytes = moe::router_ws_bytes(T, E, dtype);
  return MOE_OK;
}

moe_status moe_router_fwd(const void* x, const void* w_r, int32_t T, int32_t H, int32_t E,
                          int32_t dtype, float* logits, void* ws, size_t ws_bytes,
                          void* stream) {
  moe_status st = check_router_dims(T, H, E, dtype);
  if (st != MOE_OK) return st;
  CHECK_PTR(x);
  CHECK_PTR(w_r);
  CHECK_PTR(logits);
  CHECK_PTR(ws);
  if (logits == x || logits == w_r) return fail(MOE_ERR_INVALID_ARG, "logits aliases an input");
  const size_t need = moe::router_ws_bytes(T, E, dtype);
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "router workspace needs " + std::to_string(need) + " bytes");
  hipError_t e = moe::launch_router_fwd(x, w_r, T, H, E, dtype, logits, ws, as_stream(stream),
                                        moe::active_timer());
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_router_fwd");
}

moe_status moe_router_bwd(const float* d_logits, const void* w_r, int32_t T, int32_t H,
                          int32_t E, int32_t dtype, void* dx, void* ws, size_t ws_bytes,
                          void* stream) {
  moe_status st = check_router_dims(T, H, E, dtype);
  if (st != MOE_OK) return st;
  CHECK_PTR(d_logits);
  CHECK_PTR(w_r);
  CHECK_PTR(dx);
  CHECK_PTR(ws);
  if (dx == d_logits || dx == w_r) return fail(MOE_ERR_INVALID_ARG, "dx aliases an input");
  const size_t need = moe::router_ws_bytes(T, E, dtype);
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "router workspace needs " + std::to_string(need) + " bytes");
  hipError_t e = moe::launch_router_bwd(d_logits, w_r, T, H, E, dtype, dx, ws,
                                        as_stream(stream), moe::active_timer());
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_router_bwd");
}

namespace {

// The merged export needs only the weight shapes: T and k are not read.
moe_status check_merge_shape(const moe_shape* s) {
  if (!s) return fail(MOE_ERR_INVALID_ARG, "null shape");
  if (s->E < 1 || s->E > 1024) return fail(MOE_ERR_INVALID_ARG, "E must be in [1, 1024]");
  if (s->H < 1 || s->I < 1) return fail(MOE_ERR_INVALID_ARG, "H and I must be >= 1");
  if (s->r < 1) return fail(MOE_ERR_INVALID_ARG, "r must be >= 1");
  if (s->dtype != MOE_F32 && s->dtype != MOE_BF16 && s->dtype != MOE_F16)
    return fail(MOE_ERR_INVALID_ARG, "unknown dtype " + std::to_string(s->dtype));
  if (s->H % 8 != 0 || s->I % 8 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "H and I must be multiples of 8");
  if (s->r > 64) return fail(MOE_ERR_UNSUPPORTED, "r > 64 is not supported");
  if (int64_t(s->E) * std::max(2 * int64_t(s->I), int64_t(s->H)) >= (int64_t(1) << 31))
    return fail(MOE_ERR_INVALID_ARG, "E * max(2I, H) must be < 2^31");
  return MOE_OK;
}

moe::ExpertDims merge_dims_of(const moe_shape* s) {
  moe::ExpertDims d{};
  d.N = 0;
  d.H = s->H;
  d.I = s->I;
  d.E = s->E;
  d.r = s->r;
  d.dtype = s->dtype;
  d.scale = s->lora_scale;
  return d;
}

}  // namespace

moe_status moe_merge_workspace_bytes(const moe_shape* shape, size_t* ws_bytes) {
  moe_status st = check_merge_shape(shape);
  if (st != MOE_OK) return st;
  CHECK_PTR(ws_bytes);
  *ws_bytes = moe::merge_ws_bytes(merge_dims_of(shape));
  return MOE_OK;
}

moe_status moe_merge_lora(const moe_shape* shape, const moe_weights* weights, void* w_gu_merged,
                          void* w_d_merged, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_merge_shape(shape);
  if (st != MOE_OK) return st;
  CHECK_PTR(weights);
  CHECK_PTR(weights->w_gu);
  CHECK_PTR(weights->a_gu);
  CHECK_PTR(weights->b_gu);
  CHECK_PTR(weights->w_d);
  CHECK_PTR(weights->a_d);
  CHECK_PTR(weights->b_d);
  CHECK_PTR(ws);
  if (!w_gu_merged && !w_d_merged)
    return fail(MOE_ERR_INVALID_ARG, "no output: w_gu_merged and w_d_merged are both NULL");
  const void* lora[4] = {weights->a_gu, weights->b_gu, weights->a_d, weights->b_d};
  for (const void* q : lora)
    if (q == w_gu_merged || q == w_d_merged)
      return fail(MOE_ERR_INVALID_ARG, "a merged output aliases a LoRA parameter");
  if (w_gu_merged && (w_gu_merged == w_d_merged || w_gu_merged == weights->w_d))
    return fail(MOE_ERR_INVALID_ARG, "w_gu_merged aliases the down projection");
  if (w_d_merged && w_d_merged == weights->w_gu)
    return fail(MOE_ERR_INVALID_ARG, "w_d_merged aliases the gate_up projection");
  const moe::ExpertDims d = merge_dims_of(shape);
  const size_t need = moe::merge_ws_bytes(d);
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "merge workspace needs " + std::to_string(need) + " bytes");
  hipError_t e = moe::launch_merge(d, *weights, w_gu_merged, w_d_merged, ws, as_stream(stream),
                                   moe::active_timer());
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_merge_lora");
}

moe_status moe_accumulate(int32_t dtype, int64_t n, const void* src, void* dst, void* stream) {
  if (dtype != MOE_F32 && dtype != MOE_BF16 && dtype != MOE_F16)
    return fail(MOE_ERR_INVALID_ARG, "unknown dtype");
  if (n < 0) return fail(MOE_ERR_INVALID_ARG, "n < 0");
  if (n == 0) return MOE_OK;
  CHECK_PTR(src);
  CHECK_PTR(dst);
  {
    const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
    const uintptr_t bytes = static_cast<uintptr_t>(n) * (dtype == MOE_F32 ? 4 : 2);
    if (a < b + bytes && b < a + bytes) return fail(MOE_ERR_INVALID_ARG, "src and dst overlap");
  }
  hipError_t e = moe::launch_accumulate(dtype, n, src, dst, as_stream(stream), moe::active_timer());
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_accumulate");
}

moe_status moe_kernel_timer_enable(int32_t on) {
  TimerState& t = timer();
  std::lock_guard<std::mutex> lk(t.mu);
  t.on = on != 0;
  return MOE_OK;
}

moe_status moe_kernel_timer_select(uint32_t mask) {
  TimerState& t = timer();
  std::lock_guard<std::mutex> lk(t.mu);
  t.mask = mask;
  return MOE_OK;
}

moe_status moe_kernel_timer_reset(void) {
  TimerState& t = timer();
  std::lock_guard<std::mutex> lk(t.mu);
  for (auto& r : t.recs) {
    t.pool.push_back(r.a);
    t.pool.push_back(r.b);
  }
  t.recs.clear();
  t.open.assign(MOE_K_COUNT, -1);
  return MOE_OK;
}

moe_status moe_kernel_timer_read(int32_t kernel_id, double* total_ms, int32_t* launches) {
  if (kernel_id < 0 || kernel_id >= MOE_K_COUNT)
    return fail(MOE_ERR_INVALID_ARG, "unknown kernel id");
  TimerState& t = timer();
  std::lock_guard<std::mutex> lk(t.mu);
  double sum = 0.0;
  int n = 0;
  for (auto& r : t.recs) {
    if (r.id != kernel_id) continue;
    float ms = 0.f;
    hipError_t e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) return hip_fail(e, "moe_kernel_timer_read");
    sum += ms;
    ++n;
  }
  if (total_ms) *total_ms = sum;
  if (launches) *launches = n;
  return MOE_OK;
}

}  // extern "C"
