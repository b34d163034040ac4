// Row-wise kernels around the grouped GEMMs: the Gemma input norms, the
// per-token combine/finalize and a strided copy of the routing results.
//
// prenorm ("Gemma 4 26B-A4B MoE walkthrough" sections 1 and 3; Gemma4Router in
// the vLLM gemma4 API docs): one pass over each token row x computes
// inv_rms = 1 / sqrt(mean(x^2) + eps) and, only where a learned per-dimension
// weight makes the norm more than a row factor, materialises the rows
//   r   = x * inv_rms * H^-0.5 * router_scale   (router input; RMSNorm without gamma)
//   xn1 = x * inv_rms * gamma_pre               (dense MLP input, pre_feedforward_layernorm)
//   xn2 = x * inv_rms * gamma_pre2              (expert input, pre_feedforward_layernorm_2)
// Without such a weight the GEMM epilogues apply inv_rms to the accumulators.
//
// finalize (section 7 combine, section 1 branch merge): for token t,
//   moe = sum_{j < Kp} ybuf[t, j, :]   in slot order, fp32;
//   out = RMSNorm(dense_out[t]) * gamma_post1 + RMSNorm(moe) * gamma_post2  (dense branch)
//   out = moe                                                              (otherwise)
//   out = x[t] + RMSNorm(out) * gamma_post_ff       (the FFN block's tail, when asked:
//         post_feedforward_layernorm and the residual add of section 1)
// The per-slot rows were already multiplied by their routing weights; out is
// rounded once, at the end.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int NT = 256;

__device__ __forceinline__ float block_sum_f32(float v, float* s_red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_f32(v);
  __syncthreads();
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) t += s_red[w];
  return t;
}

__device__ __forceinline__ double block_sum_f64(double v, double* s_red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_f64(v);
  __syncthreads();
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) t += s_red[w];
  return t;
}

template <typename TIn>
__device__ __forceinline__ float ld(const TIn* p, int64_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<bf16_t>(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

template <typename TOut>
__device__ __forceinline__ void st(TOut* p, int64_t i, float v);
template <>
__device__ __forceinline__ void st<float>(float* p, int64_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void st<bf16_t>(bf16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }

template <typename TX>
__global__ __launch_bounds__(NT) void prenorm_kernel(const TX* __restrict__ x, int H, float eps,
                                                     float* __restrict__ inv_rms,
                                                     const float* __restrict__ router_scale,
                                                     const float* __restrict__ g_pre,
                                                     const float* __restrict__ g_pre2, TX* __restrict__ r_out,
                                                     TX* __restrict__ xn1, TX* __restrict__ xn2) {
  // fp64 throughout: a materialised row is then the exactly rounded normalised
  // value (rounded to fp32, then to the row's type), so any later decision
  // taken on it (an FP8 code) does not depend on the summation order
  __shared__ double s_red[NT / 64];
  const int64_t t = blockIdx.x;
  const TX* xr = x + t * H;
  double ss = 0.0;
  for (int i = threadIdx.x; i < H; i += NT) {
    const double v = ld(xr, i);
    ss += v * v;
  }
  ss = block_sum_f64(ss, s_red);
  const double inv = 1.0 / sqrt(ss / (double)H + (double)eps);
  const double root = 1.0 / sqrt((double)H);
  if (threadIdx.x == 0) inv_rms[t] = (float)inv;
  if (!r_out && !xn1 && !xn2) return;
  for (int i = threadIdx.x; i < H; i += NT) {
    const double n = (double)ld(xr, i) * inv;
    if (r_out) st(r_out, t * H + i, (float)(n * root * (router_scale ? (double)router_scale[i] : 1.0)));
    if (xn1) st(xn1, t * H + i, (float)(n * (g_pre ? (double)g_pre[i] : 1.0)));
    if (xn2) st(xn2, t * H + i, (float)(n * (g_pre2 ? (double)g_pre2[i] : 1.0)));
  }
}

// 8 consecutive elements per access: 16 bytes of bf16 or 32 bytes of fp32.
__device__ __forceinline__ void ld8(const bf16_t* p, float* v) {
  const uint4 u = *(const uint4*)p;
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void ld8(const float* p, float* v) {
  const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void st8(bf16_t* p, const float* v) {
  uint4 u;
  u.x = pack_bf16x2(v[0], v[1]);
  u.y = pack_bf16x2(v[2], v[3]);
  u.z = pack_bf16x2(v[4], v[5]);
  u.w = pack_bf16x2(v[6], v[7]);
  *(uint4*)p = u;
}
__device__ __forceinline__ void st8(float* p, const float* v) {
  *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
  *(float4*)(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// One block per token; thread g owns elements [8g, 8g + 8) (+ NT*8 strides), G
// groups of them (H <= NT * 8 * G).  The dense branch's and the residual's rows
// are loaded first, so their loads are in flight with the slot rows' (one round
// trip per block, not three); the residual stays raw until it is used.
template <typename TY, typename TO, int G>
__global__ __launch_bounds__(NT) void finalize_kernel(const TY* __restrict__ ybuf, int Kp,
                                                      const float* __restrict__ dense_out,
                                                      const float* __restrict__ g1, const float* __restrict__ g2,
                                                      float eps, TO* __restrict__ out,
                                                      float* __restrict__ out_f32, int H, bool tail,
                                                      const TO* __restrict__ resid,
                                                      const float* __restrict__ gff) {
  __shared__ float s_red[NT / 64];
  constexpr bool RB = std::is_same<TO, bf16_t>::value;  // residual rows in bf16 (else fp32)
  const int64_t t = blockIdx.x;
  const int ng = H / 8;
  float d[G][8];
  uint4 rr[G][RB ? 1 : 2];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int idx = threadIdx.x + g * NT;
#pragma unroll
    for (int q = 0; q < 8; ++q) d[g][q] = 0.f;
    if (dense_out && idx < ng) ld8(dense_out + t * H + idx * 8, d[g]);
    if (tail && idx < ng) {
      const uint4* rp = (const uint4*)(resid + t * H + idx * 8);
      rr[g][0] = rp[0];
      if constexpr (!RB) rr[g][RB ? 0 : 1] = rp[1];
    }
  }
  float m[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int q = 0; q < 8; ++q) m[g][q] = 0.f;
  // Sum in slot order; the slot loop is outside so one slot's loads for all of
  // this thread's groups (and, unrolled, the next slots') are in flight together.
#pragma unroll 4
  for (int j = 0; j < Kp; ++j) {
    const TY* yr = ybuf + (t * Kp + j) * H;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int idx = threadIdx.x + g * NT;
      if (idx < ng) {
        float v[8];
        ld8(yr + idx * 8, v);
#pragma unroll
        for (int q = 0; q < 8; ++q) m[g][q] += v[q];
      }
    }
  }
  // o: the layer output of this thread's groups
  float o[G][8];
  if (dense_out == nullptr) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int q = 0; q < 8; ++q) o[g][q] = m[g][q];
  } else {
    float ssm = 0.f, ssd = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int idx = threadIdx.x + g * NT;
      if (idx < ng) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          ssm += m[g][q] * m[g][q];
          ssd += d[g][q] * d[g][q];
        }
      }
    }
    ssm = block_sum_f32(ssm, s_red);
    ssd = block_sum_f32(ssd, s_red);
    const float im = 1.0f / sqrtf(ssm / (float)H + eps);
    const float id = 1.0f / sqrtf(ssd / (float)H + eps);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int idx = threadIdx.x + g * NT;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = idx * 8 + q;
        o[g][q] = idx < ng ? d[g][q] * id * (g1 ? g1[i] : 1.f) + m[g][q] * im * (g2 ? g2[i] : 1.f) : 0.f;
      }
    }
  }
  if (tail) {
    float ss = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int q = 0; q < 8; ++q) ss += o[g][q] * o[g][q];  // zero past H
    ss = block_sum_f32(ss, s_red);
    const float io = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int idx = threadIdx.x + g * NT;
      if (idx < ng) {
        float r[8];
        if constexpr (RB) {
          const uint32_t w[4] = {rr[g][0].x, rr[g][0].y, rr[g][0].z, rr[g][0].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            r[2 * i] = __uint_as_float(w[i] << 16);
            r[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
          }
        } else {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint4 u = rr[g][RB ? 0 : h];
            r[4 * h] = __uint_as_float(u.x);
            r[4 * h + 1] = __uint_as_float(u.y);
            r[4 * h + 2] = __uint_as_float(u.z);
            r[4 * h + 3] = __uint_as_float(u.w);
          }
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) o[g][q] = r[q] + o[g][q] * io * (gff ? gff[idx * 8 + q] : 1.f);
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int idx = threadIdx.x + g * NT;
    if (idx < ng) {
      st8(out + t * H + idx * 8, o[g]);
      if (out_f32) st8(out_f32 + t * H + idx * 8, o[g]);
    }
  }
}

__global__ void gather_topk_kernel(const float* __restrict__ w_in, const int32_t* __restrict__ ids_in,
                                   int in_stride, int K, int64_t T, float* __restrict__ w_out,
                                   int32_t* __restrict__ ids_out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * K) return;
  const int64_t t = i / K;
  const int j = (int)(i % K);
  if (w_out) w_out[i] = w_in[t * in_stride + j];
  if (ids_out) ids_out[i] = ids_in[t * in_stride + j];
}

hipError_t launch_prenorm(const void* x, int elem, int64_t T, int H, float eps, float* inv_rms,
                          const float* router_scale, const float* gamma_pre, const float* gamma_pre2,
                          void* r_out, void* xn1_out, void* xn2_out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (elem == ELEM_F32)
    prenorm_kernel<float><<<dim3((unsigned)T), dim3(NT), 0, s>>>(
        (const float*)x, H, eps, inv_rms, router_scale, gamma_pre, gamma_pre2, (float*)r_out,
        (float*)xn1_out, (float*)xn2_out);
  else
    prenorm_kernel<bf16_t><<<dim3((unsigned)T), dim3(NT), 0, s>>>(
        (const bf16_t*)x, H, eps, inv_rms, router_scale, gamma_pre, gamma_pre2, (bf16_t*)r_out,
        (bf16_t*)xn1_out, (bf16_t*)xn2_out);
  return hipGetLastError();
}

hipError_t launch_finalize(const void* ybuf, int yelem, int Kp, const float* dense_out,
                           const float* gamma_post1, const float* gamma_post2, float eps, void* out,
                           int oelem, float* out_f32, int64_t T, int H, hipStream_t s, const void* resid,
                           const float* gamma_post_ff) {
  if (T == 0) return hipSuccess;
  if (H > NT * 32 || H % 8) return hipErrorInvalidValue;
  const bool tail = resid != nullptr;
  dim3 g((unsigned)T), b(NT);
  // rows up to 4096 elements: two groups of 8 per thread (fewer registers)
  auto go = [&](auto g_tag) -> hipError_t {
    constexpr int G = decltype(g_tag)::value;
    if (yelem == ELEM_F32 && oelem == ELEM_F32)
      finalize_kernel<float, float, G><<<g, b, 0, s>>>((const float*)ybuf, Kp, dense_out, gamma_post1,
                                                       gamma_post2, eps, (float*)out, out_f32, H, tail,
                                                       (const float*)resid, gamma_post_ff);
    else if (yelem == ELEM_BF16 && oelem == ELEM_BF16)
      finalize_kernel<bf16_t, bf16_t, G><<<g, b, 0, s>>>((const bf16_t*)ybuf, Kp, dense_out, gamma_post1,
                                                         gamma_post2, eps, (bf16_t*)out, out_f32, H, tail,
                                                         (const bf16_t*)resid, gamma_post_ff);
    else if (yelem == ELEM_F32 && oelem == ELEM_BF16)
      finalize_kernel<float, bf16_t, G><<<g, b, 0, s>>>((const float*)ybuf, Kp, dense_out, gamma_post1,
                                                        gamma_post2, eps, (bf16_t*)out, out_f32, H, tail,
                                                        (const bf16_t*)resid, gamma_post_ff);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  };
  if (H <= NT * 8 * 2) return go(std::integral_constant<int, 2>{});
  return go(std::integral_constant<int, 4>{});
}

hipError_t launch_gather_topk(const float* w_in, const int32_t* ids_in, int in_stride, int K, int64_t T,
                              float* w_out, int32_t* ids_out, hipStream_t s) {
  const int64_t n = T * K;
  if (n == 0) return hipSuccess;
  gather_topk_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(w_in, ids_in, in_stride, K, T,
                                                                            w_out, ids_out);
  return hipGetLastError();
}

// Zero fill (the atomic combine's fp32 sums start from zero): 16 bytes per lane,
// a grid-stride loop over a few blocks per CU.
__global__ __launch_bounds__(256) void zero_kernel(uint4* __restrict__ p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  if (bytes % 16 || ((uintptr_t)p & 15)) return hipErrorInvalidValue;
  const int64_t n16 = (int64_t)(bytes / 16);
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 4 * 256) blocks = 4 * 256;
  zero_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>((uint4*)p, n16);
  return hipGetLastError();
}

}  // namespace moe
