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

// Round-to-nearest-even fp32 -> bf16: gfx950's v_cvt_pk_bf16_f32 (two values
// per instruction; NaN stays NaN, overflow rounds to infinity).
typedef float f32x2_cvt __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_cvt __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_cvt v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_cvt));
}
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return (bf16_t)(pack_bf16x2(f, 0.f) & 0xFFFFu); }

// ---------------------------------------------------------------- wave64 reductions
// All-reduce over the 64 lanes with DPP moves only (no LDS round trip):
// butterflies over xor 1 and xor 2 (quad permutes), then the half-row and row
// mirrors leave every lane of a 16-lane row with the row's result; row_bcast:15
// folds row 0 into row 1 and row 2 into row 3, row_bcast:31 folds rows 0-1 into
// rows 2-3, so lane 63 ends with the result, which readlane makes uniform.
// Rows a broadcast does not write receive the identity (`old`), so the same
// sequence serves sums as well as max / min.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xF, false);
}

template <typename Op>
__device__ __forceinline__ uint32_t wave_allreduce_u32(uint32_t v, Op op, uint32_t identity) {
  v = op(v, dpp_u32<0xB1>(v, identity));       // quad_perm [1,0,3,2]
  v = op(v, dpp_u32<0x4E>(v, identity));       // quad_perm [2,3,0,1]
  v = op(v, dpp_u32<0x141>(v, identity));      // row_half_mirror
  v = op(v, dpp_u32<0x140>(v, identity));      // row_mirror
  v = op(v, dpp_u32<0x142, 0xA>(v, identity)); // row_bcast:15 into rows 1, 3
  v = op(v, dpp_u32<0x143, 0xC>(v, identity)); // row_bcast:31 into rows 2, 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_allreduce_u32(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; }, 0u);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return wave_allreduce_u32(v, [](uint32_t a, uint32_t b) { return a < b ? a : b; }, 0xFFFFFFFFu);
}
__device__ __forceinline__ float wave_max_f32(float v) {
  return __uint_as_float(wave_allreduce_u32(
      __float_as_uint(v),
      [](uint32_t a, uint32_t b) { return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b))); },
      __float_as_uint(-INFINITY)));
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  return __uint_as_float(wave_allreduce_u32(
      __float_as_uint(v),
      [](uint32_t a, uint32_t b) { return __float_as_uint(__uint_as_float(a) + __uint_as_float(b)); }, 0u));
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  // the same moves on the two 32-bit halves of each double (identity +0.0 = all-zero bits)
  auto mv = [](double x, auto shuffle) {
    uint64_t u = __double_as_longlong(x);
    uint32_t lo = shuffle((uint32_t)u), hi = shuffle((uint32_t)(u >> 32));
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
  };
  v += mv(v, [](uint32_t a) { return dpp_u32<0xB1>(a, 0u); });
  v += mv(v, [](uint32_t a) { return dpp_u32<0x4E>(a, 0u); });
  v += mv(v, [](uint32_t a) { return dpp_u32<0x141>(a, 0u); });
  v += mv(v, [](uint32_t a) { return dpp_u32<0x140>(a, 0u); });
  v += mv(v, [](uint32_t a) { return dpp_u32<0x142, 0xA>(a, 0u); });
  v += mv(v, [](uint32_t a) { return dpp_u32<0x143, 0xC>(a, 0u); });
  return mv(v, [](uint32_t x) { return (uint32_t)__builtin_amdgcn_readlane((int)x, 63); });
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

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float apply_act(int act, float g) {
  return act == 0 ? act_silu(g) : act_gelu_tanh(g);
}

// The same activations for results rounded to bf16 next (8 significant bits):
// both are g * sigmoid(t) (SiLU: t = g; GELU-tanh: t = 2c(g + 0.044715 g^3)),
// and the sigmoid is taken from the hardware base-2 exponential and reciprocal
// (v_exp_f32, v_rcp_f32, about 1 ulp each).  A few fp32 ulps in all, against
// the 2^-9 relative step of the rounding that follows; about a quarter of the
// instructions of the correctly rounded exponential and division.  Limits:
// t -> -inf gives g * 0, t -> +inf gives g.
__device__ __forceinline__ float apply_act_bf16(int act, float g) {
  const float t = act == 0 ? g : 1.5957691216057308f * (g + 0.044715f * g * g * g);  // 2 sqrt(2/pi)
  const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * t);                   // e^-t
  return g * __builtin_amdgcn_rcpf(1.0f + e);
}

// 8 fp8 (E4M3) codes in two dwords -> 8 bf16.  v_cvt_pk_f32_fp8 widens two codes
// (word 0 or word 1 of a dword) to fp32; every E4M3 value has at most 4
// significant bits, so the upper 16 bits of its fp32 pattern are exactly its
// bf16 pattern, and one byte permute packs two of them.
template <bool HI_WORD>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t src) {
  const auto f = __builtin_amdgcn_cvt_pk_f32_fp8(src, HI_WORD);
  return __builtin_amdgcn_perm(__float_as_uint(f[1]), __float_as_uint(f[0]), 0x07060302u);
}
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  u32x4 r;
  r[0] = fp8x2_to_bf16x2<false>(lo);
  r[1] = fp8x2_to_bf16x2<true>(lo);
  r[2] = fp8x2_to_bf16x2<false>(hi);
  r[3] = fp8x2_to_bf16x2<true>(hi);
  return __builtin_bit_cast(bf16x8, r);
}

// Dynamic per-row FP8 quantisation pieces (the "FP8-Dynamic" scheme named on
// the sglang PR #24696 page): a row's scale is its largest magnitude / 448 (1 for
// an all-zero row) and a code is the E4M3 nearest-even of value / scale, with an
// IEEE fp32 division and v_cvt_pk_fp8_f32 (round to nearest even, saturating at
// 448), so a code depends on the fp32 values alone.
__device__ __forceinline__ float absmax8(uint4 x) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  float m = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    m = fmaxf(m, fabsf(__uint_as_float(w[q] << 16)));
    m = fmaxf(m, fabsf(__uint_as_float(w[q] & 0xFFFF0000u)));
  }
  return m;
}

// codes of the 8 bf16 values in x at scale s, in order (two dwords of 4 codes)
__device__ __forceinline__ uint2 codes8(uint4 x, float s) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t out[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float f0 = __uint_as_float(w[2 * h] << 16) / s, f1 = __uint_as_float(w[2 * h] & 0xFFFF0000u) / s;
    const float f2 = __uint_as_float(w[2 * h + 1] << 16) / s, f3 = __uint_as_float(w[2 * h + 1] & 0xFFFF0000u) / s;
    int p = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
    p = __builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, p, true);
    out[h] = (uint32_t)p;
  }
  return make_uint2(out[0], out[1]);
}

__device__ __forceinline__ float scale_of(float amax) {
  const float s = amax / 448.0f;
  return s > 0.f ? s : 1.f;
}

// Buffer resource over [base, base + bytes): loads past the end return 0.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw buffer: stride 0, num_records = bytes (loads past it return 0)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

}  // namespace moe
