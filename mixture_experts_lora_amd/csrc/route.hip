// Top-k routing and its backward, one wave64 per token.
//
// Selection: the k largest logits, ordered by logit descending with ties to
// the lower expert index, found by k rounds of a wave-wide argmax over the
// float32 logits themselves (comparisons only, so the choice is exact). The
// combine weights follow the router mode. The faster-moe page (Unsloth,
// "Fine-tune MoE models 12x faster", section "What is torch._grouped_mm?")
// walks an expert mask built from such a choice; its section "Implementation
// details" keeps the router frozen, so the backward only produces d logits.
#include "device_common.h"
#include "launch.h"

#include <float.h>

namespace moe {

namespace {

constexpr int kMaxVals = 16;  // E <= 1024 = 16 values per lane

// The kernels hold NV logits per lane (NV >= ceil(E / 64); instantiated for
// 1, 2, 4 and kMaxVals, so the common expert counts loop over no empty slots).
inline int route_nv(int E) { return E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : kMaxVals; }

struct TopK {
  int id;      // valid in lane j < k: expert of slot j
  float val;   // its logit
};

// (bv, bi) := the better of itself and (ov, oi): larger logit, ties to the
// lower expert index. A total order, so both lanes of a pair agree.
__device__ __forceinline__ void take_better(float& bv, int& bi, float ov, int oi) {
  if (ov > bv || (ov == bv && oi < bi)) {
    bv = ov;
    bi = oi;
  }
}

template <int CTRL>
__device__ __forceinline__ void argmax_step(float& bv, int& bi) {
  take_better(bv, bi, dpp_f32<CTRL>(bv), dpp_i32<CTRL>(bi));
}

// Wave-wide argmax: within each row of 16 lanes by DPP moves, then over the
// four rows' winners (read into scalars) in a fixed order; every lane gets
// the result.
__device__ __forceinline__ void wave_argmax(float& bv, int& bi) {
  argmax_step<kDppSwap1>(bv, bi);
  argmax_step<kDppSwap2>(bv, bi);
  argmax_step<kDppHalfMirror>(bv, bi);
  argmax_step<kDppMirror>(bv, bi);
  float v = readlane_f32(bv, 0);
  int i = __builtin_amdgcn_readlane(bi, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r)
    take_better(v, i, readlane_f32(bv, 16 * r), __builtin_amdgcn_readlane(bi, 16 * r));
  bv = v;
  bi = i;
}

// k rounds of wave argmax. v[i] holds logit of expert lane + 64 i (-inf past E).
template <int NV>
__device__ __forceinline__ TopK wave_topk(const float (&v)[NV], int nv, int E, int k, int lane) {
  uint32_t taken = 0;
  TopK mine{-1, 0.f};
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = INT32_MAX;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if (i < nv) {
        int idx = lane + kWave * i;
        bool ok = idx < E && !((taken >> i) & 1u);
        if (ok && (v[i] > bv || (v[i] == bv && idx < bi))) {
          bv = v[i];
          bi = idx;
        }
      }
    }
    wave_argmax(bv, bi);
    if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
    if (lane == j) {
      mine.id = bi;
      mine.val = bv;
    }
  }
  return mine;
}

// Combine weight of this lane's slot (lanes >= k return 0). mx = top-1 logit.
template <int NV>
__device__ __forceinline__ float slot_weight(const float (&v)[NV], int nv, int E,
                                             int k, int router, const TopK& mine, float mx,
                                             int lane, float* p_all_sum) {
  bool act = lane < k;
  float w = 0.f;
  if (router == MOE_SOFTMAX_TOPK || router == MOE_SOFTMAX_TOPK_RENORM) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (i < nv && lane + kWave * i < E) s += expf(v[i] - mx);
    s = wave_sum(s);
    if (p_all_sum) *p_all_sum = s;
    float p = act ? expf(mine.val - mx) / s : 0.f;
    if (router == MOE_SOFTMAX_TOPK_RENORM) {
      float ps = wave_sum(p);
      w = act ? p / ps : 0.f;
    } else {
      w = p;
    }
  } else if (router == MOE_TOPK_SOFTMAX) {
    float e = act ? expf(mine.val - mx) : 0.f;
    float s = wave_sum(e);
    w = act ? e / s : 0.f;
  } else {
    float sg = act ? 1.0f / (1.0f + expf(-mine.val)) : 0.f;
    float s = wave_sum(sg);
    w = act ? sg / s : 0.f;
  }
  return w;
}

template <int NV>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T,
                                                    int E, int k, int router,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = (blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  if (t >= T) return;
  const float* l = logits + static_cast<size_t>(t) * E;
  const int nv = (E + kWave - 1) / kWave;
  float v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int idx = lane + kWave * i;
    v[i] = (i < nv && idx < E) ? l[idx] : -INFINITY;
  }
  TopK mine = wave_topk(v, nv, E, k, lane);
  float mx = readlane_f32(mine.val, 0);
  float wj = slot_weight(v, nv, E, k, router, mine, mx, lane, nullptr);
  if (lane < k) {
    ids[static_cast<size_t>(t) * k + lane] = mine.id;
    w[static_cast<size_t>(t) * k + lane] = wj;
  }
}

template <int NV>
__global__ __launch_bounds__(256) void route_bwd_kernel(const float* __restrict__ logits,
                                                        const int32_t* __restrict__ ids,
                                                        const float* __restrict__ dw, int T,
                                                        int E, int k, int router,
                                                        float* __restrict__ dlogits) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = (blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  if (t >= T) return;
  const float* l = logits + static_cast<size_t>(t) * E;
  const int nv = (E + kWave - 1) / kWave;
  float v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int idx = lane + kWave * i;
    v[i] = (i < nv && idx < E) ? l[idx] : -INFINITY;
  }
  TopK mine{-1, 0.f};
  float mydw = 0.f;
  if (lane < k) {
    mine.id = ids[static_cast<size_t>(t) * k + lane];
    // ids come from moe_route; an out-of-range id (caller error) is clamped so
    // the read stays in bounds (its gradient is then meaningless)
    if (mine.id < 0 || mine.id >= E) mine.id = 0;
    mine.val = l[mine.id];
    mydw = dw[static_cast<size_t>(t) * k + lane];
  }
  // top-1 logit = max over all logits (the selection is the top-k)
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < NV; ++i) mx = fmaxf(mx, v[i]);
  mx = wave_max(mx);
  float psum = 0.f;
  float wj = slot_weight(v, nv, E, k, router, mine, mx, lane, &psum);
  const float c = wave_sum(lane < k ? mydw * wj : 0.f);
  const float sg = lane < k ? 1.0f / (1.0f + expf(-mine.val)) : 0.f;
  const float ssum = wave_sum(sg);
  // per selected slot: dl[S_j] = coef_j in the selected-only modes; for
  // softmax_topk coef_j is dw_j, scattered below into dw^.
  float coef = 0.f;
  if (lane < k) {
    if (router == MOE_SOFTMAX_TOPK_RENORM || router == MOE_TOPK_SOFTMAX) {
      coef = wj * (mydw - c);
    } else if (router == MOE_SIGMOID_TOPK_RENORM) {
      coef = sg * (1.f - sg) * (mydw - c) / ssum;
    } else {
      coef = mydw;
    }
  }
  float out[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) out[i] = 0.f;
  if (router == MOE_SOFTMAX_TOPK) {
    // dl_i = p_i (dw^_i - c) for all i
    float dhat[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) dhat[i] = 0.f;
    for (int j = 0; j < k; ++j) {
      int idj = __builtin_amdgcn_readlane(mine.id, j);
      float dj = readlane_f32(coef, j);
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (lane + kWave * i == idj) dhat[i] = dj;
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float p = expf(v[i] - mx) / psum;
      out[i] = p * (dhat[i] - c);
    }
  } else {
    for (int j = 0; j < k; ++j) {
      int idj = __builtin_amdgcn_readlane(mine.id, j);
      float dj = readlane_f32(coef, j);
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (lane + kWave * i == idj) out[i] = dj;
    }
  }
  float* d = dlogits + static_cast<size_t>(t) * E;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int idx = lane + kWave * i;
    if (i < nv && idx < E) d[idx] = out[i];
  }
}

}  // namespace

hipError_t launch_route(const float* logits, int T, int E, int k, int router, int32_t* ids,
                        float* w, hipStream_t s) {
  const int per_block = 256 / kWave;
  dim3 grid((T + per_block - 1) / per_block);
  auto kern = route_kernel<kMaxVals>;
  switch (route_nv(E)) {
    case 1: kern = route_kernel<1>; break;
    case 2: kern = route_kernel<2>; break;
    case 4: kern = route_kernel<4>; break;
    default: break;
  }
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, logits, T, E, k, router, ids, w);
  return hipGetLastError();
}

hipError_t launch_route_bwd(const float* logits, const int32_t* ids, const float* dw, int T,
                            int E, int k, int router, float* dlogits, hipStream_t s) {
  const int per_block = 256 / kWave;
  dim3 grid((T + per_block - 1) / per_block);
  auto kern = route_bwd_kernel<kMaxVals>;
  switch (route_nv(E)) {
    case 1: kern = route_bwd_kernel<1>; break;
    case 2: kern = route_bwd_kernel<2>; break;
    case 4: kern = route_bwd_kernel<4>; break;
    default: break;
  }
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, logits, ids, dw, T, E, k, router, dlogits);
  return hipGetLastError();
}

}  // namespace moe
