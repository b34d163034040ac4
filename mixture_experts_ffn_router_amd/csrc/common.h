// Shared device helpers for the gfx950 MoE kernels: storage types, bf16/fp8
// conversion, wave64 DPP reductions and launch-error plumbing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // bf16 storage (upper half of an fp32)
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int WAVE = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(((uint32_t)v) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (inputs are finite).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// ---------------------------------------------------------------- wave64 reductions
// Butterfly all-reduce: xor 1 and xor 2 by quad permutes, then the half-row
// and row mirrors (every lane of a quad / half-row already holds the same
// partial, so a mirror reaches the partner group), xor 16 by ds_swizzle, and
// the two 32-lane halves through readlane.  Every lane ends with the result.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t swz_xor16(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);
}

template <typename Op>
__device__ __forceinline__ uint32_t wave_allreduce_u32(uint32_t v, Op op) {
  v = op(v, dpp_u32<0xB1>(v));    // quad_perm [1,0,3,2]
  v = op(v, dpp_u32<0x4E>(v));    // quad_perm [2,3,0,1]
  v = op(v, dpp_u32<0x141>(v));   // row_half_mirror
  v = op(v, dpp_u32<0x140>(v));   // row_mirror
  v = op(v, swz_xor16(v));
  uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  return op(a, b);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_allreduce_u32(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return wave_allreduce_u32(v, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}
__device__ __forceinline__ float wave_max_f32(float v) {
  return __uint_as_float(wave_allreduce_u32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  // same butterfly on the two 32-bit halves of each double
  auto mv = [](double x, auto shuffle) {
    uint64_t u = __double_as_longlong(x);
    uint32_t lo = shuffle((uint32_t)u), hi = shuffle((uint32_t)(u >> 32));
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
  };
  v += mv(v, [](uint32_t a) { return dpp_u32<0xB1>(a); });
  v += mv(v, [](uint32_t a) { return dpp_u32<0x4E>(a); });
  v += mv(v, [](uint32_t a) { return dpp_u32<0x141>(a); });
  v += mv(v, [](uint32_t a) { return dpp_u32<0x140>(a); });
  v += mv(v, [](uint32_t a) { return swz_xor16(a); });
  double a = mv(v, [](uint32_t x) { return (uint32_t)__builtin_amdgcn_readlane((int)x, 0); });
  double b = mv(v, [](uint32_t x) { return (uint32_t)__builtin_amdgcn_readlane((int)x, 32); });
  return a + b;
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  return __uint_as_float(wave_allreduce_u32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}

// Total order on finite fp32 as uint32, with -0.0 mapped onto +0.0.
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);  // -0.0 + 0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f32_from_order_key(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ float act_silu(float a) { return a / (1.0f + expf(-a)); }

// 0.5 a (1 + tanh(c (a + 0.044715 a^3))) written with tanh(u) = 1 - 2/(1 + e^{2u}),
// i.e. a * sigmoid(2u).
__device__ __forceinline__ float act_gelu_tanh(float a) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  float u = c * (a + 0.044715f * a * a * a);
  return a / (1.0f + expf(-2.0f * u));
}

}  // namespace moe
