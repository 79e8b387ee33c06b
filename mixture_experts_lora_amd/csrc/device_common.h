// Device helpers shared by the MoE-LoRA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef uint16_t bf16_t;  // raw bfloat16 storage
typedef _Float16 f16_t;   // IEEE half storage
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// Round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(bf16_t, b);
}

// Element conversions for the storage types (16-bit ones round to nearest even).
template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }
template <> __device__ __forceinline__ float to_f32<f16_t>(f16_t v) { return static_cast<float>(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }
template <> __device__ __forceinline__ f16_t from_f32<f16_t>(float v) { return static_cast<f16_t>(v); }

// Four consecutive elements, loaded/stored as one 8-byte (bf16) or 16-byte (f32) access.
template <typename T> struct Vec4;
template <> struct Vec4<bf16_t> {
  typedef uint2 raw;
  __device__ static void load(const bf16_t* p, float (&v)[4]) {
    uint2 r = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(r.x << 16);
    v[1] = __uint_as_float(r.x & 0xffff0000u);
    v[2] = __uint_as_float(r.y << 16);
    v[3] = __uint_as_float(r.y & 0xffff0000u);
  }
  __device__ static void store(bf16_t* p, const float (&v)[4]) {
    uint2 r;
    r.x = static_cast<uint32_t>(f32_to_bf16(v[0])) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
    r.y = static_cast<uint32_t>(f32_to_bf16(v[2])) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
    *reinterpret_cast<uint2*>(p) = r;
  }
};
template <> struct Vec4<float> {
  __device__ static void load(const float* p, float (&v)[4]) {
    float4 r = *reinterpret_cast<const float4*>(p);
    v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
  }
  __device__ static void store(float* p, const float (&v)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

// Logistic function for the SwiGLU epilogues: hardware exp2 and reciprocal
// (each within 1 ulp) instead of an IEEE divide, about ten times fewer
// instructions per element. exp(-z) overflowing to inf gives 0; underflow gives 1.
__device__ __forceinline__ float sigmoidf_(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// SwiGLU forward: act = g * sigmoid(g) * u.
__device__ __forceinline__ float swiglu(float g, float u) { return g * sigmoidf_(g) * u; }

// SwiGLU backward for upstream d = dL/dact: dg = d u s (1 + g (1 - s)), du = d g s.
__device__ __forceinline__ void swiglu_bwd(float g, float u, float d, float& dg, float& du) {
  float s = sigmoidf_(g);
  dg = d * u * s * (1.0f + g * (1.0f - s));
  du = d * g * s;
}

// SwiGLU backward that also returns the forward output g s u (one logistic
// evaluation for both).
__device__ __forceinline__ float swiglu_bwd_act(float g, float u, float d, float& dg, float& du) {
  float s = sigmoidf_(g);
  dg = d * u * s * (1.0f + g * (1.0f - s));
  du = d * g * s;
  return g * s * u;
}

// Cross-lane moves within a row of 16 lanes as DPP operand modifiers of a
// VALU move (no LDS traffic, unlike a shuffle): swap neighbours, swap pairs,
// mirror within 8 lanes, mirror within 16. Every lane of the row must be
// active.
constexpr int kDppSwap1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppSwap2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i within 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i within 16

template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(dpp_i32<CTRL>(__float_as_int(v)));
}

__device__ __forceinline__ float readlane_f32(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Wave-wide sum, every lane getting the total: a butterfly within each row of
// 16 (each step adds the same two values on both lanes of a pair, so a row
// ends uniform), then the four row sums in a fixed order. Deterministic. All
// 64 lanes must be active.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<kDppSwap1>(v);
  v += dpp_f32<kDppSwap2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  v += dpp_f32<kDppMirror>(v);
  return (readlane_f32(v, 0) + readlane_f32(v, 16)) + (readlane_f32(v, 32) + readlane_f32(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<kDppSwap1>(v));
  v = fmaxf(v, dpp_f32<kDppSwap2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppMirror>(v));
  return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)),
               fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
}

}  // namespace moe
