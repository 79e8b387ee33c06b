// Weighted combine of the k expert outputs of each token, and its backward.
//
//   combine      Y[t] = sum_{j<k} w[t, j] y_perm[inv_pos[t*k + j]]
//                (w == NULL: plain sum, which brings dX_perm back to tokens)
//   combine_bwd  G[inv_pos[t*k + j]] = w[t, j] dY[t]
//                dw[t, j] = <dY[t], y_perm[inv_pos[t*k + j]]>
//
// Both are HBM-bound streams over rows; slots are summed in the fixed order
// j = 0..k-1 in float32, and the dot products reduce in a fixed tree, so
// results are identical run to run. The weighted sum over the selected
// experts closes the MoE block whose per-expert loop the faster-moe page
// (Unsloth, "Fine-tune MoE models 12x faster", section "What is
// torch._grouped_mm?") shows.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

template <typename T> struct Pack;  // 16 bytes of T
template <> struct Pack<bf16_t> {
  static constexpr int n = 8;
  __device__ static void unpack(const uint4& r, float (&v)[8]) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static uint4 pack(const float (&v)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f32_to_bf16(v[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16(v[2 * i + 1])) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};
template <> struct Pack<f16_t> {
  static constexpr int n = 8;
  __device__ static void unpack(const uint4& r, float (&v)[8]) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = static_cast<float>(__builtin_bit_cast(f16_t, static_cast<uint16_t>(w[i])));
      v[2 * i + 1] = static_cast<float>(__builtin_bit_cast(f16_t, static_cast<uint16_t>(w[i] >> 16)));
    }
  }
  __device__ static uint4 pack(const float (&v)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<f16_t>(v[2 * i]))) |
             (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<f16_t>(v[2 * i + 1])))
              << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};
template <> struct Pack<float> {
  static constexpr int n = 4;
  __device__ static void unpack(const uint4& r, float (&v)[4]) {
    v[0] = __uint_as_float(r.x); v[1] = __uint_as_float(r.y);
    v[2] = __uint_as_float(r.z); v[3] = __uint_as_float(r.w);
  }
  __device__ static uint4 pack(const float (&v)[4]) {
    return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                      __float_as_uint(v[3]));
  }
};

// One thread per (token, 16-byte column chunk); the chunk index is split
// with 32-bit unsigned arithmetic (a 64-bit division costs about ten times
// the instructions; the layer's shape limit keeps an activation tensor under
// 32 GiB, so its chunk count fits).
template <typename Elem>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ yp,
                                                      const int32_t* __restrict__ inv_pos,
                                                      const float* __restrict__ w, int T, int k,
                                                      uint32_t cpr, uint4* __restrict__ y) {
  typedef uint32_t Idx;
  constexpr int n = Pack<Elem>::n;
  const Idx g = static_cast<Idx>(blockIdx.x) * blockDim.x + threadIdx.x;
  const Idx tt = g / cpr, c = g - tt * cpr;
  if (tt >= static_cast<Idx>(T)) return;
  const int64_t t = static_cast<int64_t>(tt);
  float acc[n];
#pragma unroll
  for (int i = 0; i < n; ++i) acc[i] = 0.f;
  // slots in groups of four: the group's row loads are all issued before
  // any is summed (several loads in flight per thread), and the sum still
  // runs in slot order
  constexpr int G = 4;
  for (int j0 = 0; j0 < k; j0 += G) {
    int pos[G];
    float wj[G];
    uint4 raw[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int j = j0 + u;
      pos[u] = j < k ? inv_pos[t * k + j] : -1;
      wj[u] = j < k && w ? w[t * k + j] : 1.0f;
    }
#pragma unroll
    for (int u = 0; u < G; ++u)
      if (pos[u] >= 0) raw[u] = yp[static_cast<int64_t>(pos[u]) * cpr + c];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      if (pos[u] < 0) continue;
      float v[n];
      Pack<Elem>::unpack(raw[u], v);
#pragma unroll
      for (int i = 0; i < n; ++i) acc[i] += wj[u] * v[i];
    }
  }
  y[t * static_cast<int64_t>(cpr) + c] = Pack<Elem>::pack(acc);
}

// One block per token; threads stride over the row's 16-byte chunks. Each
// thread loads its chunks of dY once and serves every slot from them, keeping
// one partial dot product per slot (KMAX >= k slots, unrolled), so the slots'
// row loads are in flight together; the block reduces all slots at the end in
// the same order as slot by slot (per-thread chunk order, wave tree, waves in
// order), which leaves dw bit-identical.
template <typename Elem, int KMAX>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const uint4* __restrict__ dy,
                                                          const uint4* __restrict__ yexp,
                                                          const int32_t* __restrict__ inv_pos,
                                                          const float* __restrict__ w, int k,
                                                          int64_t cpr, uint4* __restrict__ g,
                                                          float* __restrict__ dw) {
  constexpr int n = Pack<Elem>::n;
  constexpr int NWV = 256 / kWave;
  __shared__ float red[KMAX][NWV];
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int pos[KMAX];
  float wj[KMAX], part[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    pos[j] = j < k ? inv_pos[t * k + j] : -1;
    wj[j] = j < k ? w[t * k + j] : 0.f;
    part[j] = 0.f;
  }
  for (int64_t c = threadIdx.x; c < cpr; c += blockDim.x) {
    float d[n];
    Pack<Elem>::unpack(dy[t * cpr + c], d);
    uint4 raw[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (pos[j] >= 0) raw[j] = yexp[static_cast<int64_t>(pos[j]) * cpr + c];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (pos[j] < 0) continue;
      float y[n], o[n];
      Pack<Elem>::unpack(raw[j], y);
#pragma unroll
      for (int i = 0; i < n; ++i) {
        part[j] += d[i] * y[i];
        o[i] = wj[j] * d[i];
      }
      g[static_cast<int64_t>(pos[j]) * cpr + c] = Pack<Elem>::pack(o);
    }
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j >= k) break;
    const float v = wave_sum(part[j]);
    if (lane == 0) red[j][wave] = v;
  }
  __syncthreads();
  if (threadIdx.x < k) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NWV; ++i) s += red[threadIdx.x][i];
    dw[t * k + threadIdx.x] = s;
  }
}

// Routing weight of each permuted row, and the row-weighted copy of u
// ([N, r]): one thread per element of u.
template <typename Elem>
__global__ __launch_bounds__(256) void perm_weights_kernel(const float* __restrict__ w,
                                                           const int32_t* __restrict__ sorted_pair,
                                                           int64_t N, const Elem* __restrict__ u,
                                                           int r, float* __restrict__ w_perm,
                                                           Elem* __restrict__ wu) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= N * r) return;
  const int64_t row = i / r;
  const float wr = w[sorted_pair[row]];
  wu[i] = from_f32<Elem>(wr * to_f32<Elem>(u[i]));
  if (i - row * r == 0) w_perm[row] = wr;
}

// d_topk_w[p]: the down backward's per-slot partial sums of <dAct', act> for
// pair p's row (contiguous per row), added in slot order (deterministic).
__global__ __launch_bounds__(256) void dw_sum_kernel(const float* __restrict__ dwp, int slots,
                                                     const int32_t* __restrict__ inv_pos,
                                                     int64_t npairs, float* __restrict__ dw) {
  const int64_t p = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (p >= npairs) return;
  const int32_t pos = inv_pos[p];
  float acc = 0.f;
  if (pos >= 0) {
    const float* q = dwp + static_cast<int64_t>(pos) * slots;
    for (int s = 0; s < slots; ++s) acc += q[s];
  }
  dw[p] = acc;
}

}  // namespace

hipError_t launch_perm_weights(int dtype, const float* w, const int32_t* sorted_pair, int64_t N,
                               const void* u, int r, float* w_perm, void* wu, hipStream_t s) {
  const int64_t total = N * r;
  if (total <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((total + 255) / 256));
  auto go = [&](auto tag) {
    using Elem = decltype(tag);
    hipLaunchKernelGGL(perm_weights_kernel<Elem>, grid, dim3(256), 0, s, w, sorted_pair, N,
                       static_cast<const Elem*>(u), r, w_perm, static_cast<Elem*>(wu));
  };
  if (dtype == MOE_BF16) go(bf16_t{});
  else if (dtype == MOE_F16) go(f16_t{});
  else go(float{});
  return hipGetLastError();
}

hipError_t launch_dw_sum(const float* dwp, int slots, const int32_t* inv_pos, int64_t npairs,
                         float* d_topk_w, hipStream_t s) {
  if (npairs <= 0) return hipSuccess;
  hipLaunchKernelGGL(dw_sum_kernel, dim3(static_cast<unsigned>((npairs + 255) / 256)), dim3(256),
                     0, s, dwp, slots, inv_pos, npairs, d_topk_w);
  return hipGetLastError();
}

hipError_t launch_combine(int dtype, const void* y_perm, const int32_t* inv_pos, const float* w,
                          int T, int k, int H, void* y, hipStream_t s, KernelTimer* tm) {
  const int esz = dtype == MOE_F32 ? 4 : 2;
  const int64_t cpr = static_cast<int64_t>(H) * esz / 16;
  const int64_t total = static_cast<int64_t>(T) * cpr;
  dim3 grid(static_cast<unsigned>((total + 255) / 256));
  TimedScope scope(tm, w ? MOE_K_COMBINE : MOE_K_UNPERMUTE, s);
  if (total + 255 > 0xffffffffLL) return hipErrorInvalidValue;  // excluded by the shape limit
  auto go = [&](auto elem) {
    typedef decltype(elem) Elem;
    hipLaunchKernelGGL((combine_kernel<Elem>), grid, dim3(256), 0, s,
                       static_cast<const uint4*>(y_perm), inv_pos, w, T, k,
                       static_cast<uint32_t>(cpr), static_cast<uint4*>(y));
  };
  if (dtype == MOE_BF16) go(bf16_t());
  else if (dtype == MOE_F16) go(f16_t());
  else go(float());
  return hipGetLastError();
}

hipError_t launch_combine_bwd(int dtype, const void* dy, const void* y_exp,
                              const int32_t* inv_pos, const float* w, int T, int k, int H,
                              void* g, float* dw, hipStream_t s, KernelTimer* tm) {
  const int esz = dtype == MOE_F32 ? 4 : 2;
  const int64_t cpr = static_cast<int64_t>(H) * esz / 16;
  TimedScope scope(tm, MOE_K_COMBINE_BWD, s);
  auto go = [&](auto tag, auto kmax) {
    using Elem = decltype(tag);
    hipLaunchKernelGGL((combine_bwd_kernel<Elem, decltype(kmax)::value>), dim3(T), dim3(256), 0, s,
                       static_cast<const uint4*>(dy), static_cast<const uint4*>(y_exp), inv_pos,
                       w, k, cpr, static_cast<uint4*>(g), dw);
  };
  auto by_k = [&](auto tag) {
    if (k <= 8) go(tag, std::integral_constant<int, 8>());
    else go(tag, std::integral_constant<int, 32>());
  };
  if (dtype == MOE_BF16) by_k(bf16_t{});
  else if (dtype == MOE_F16) by_k(f16_t{});
  else by_k(float{});
  return hipGetLastError();
}

}  // namespace moe
