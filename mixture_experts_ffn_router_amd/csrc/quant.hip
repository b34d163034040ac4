// Dynamic per-row FP8 quantisation of activations (the "FP8-Dynamic" scheme
// named on the sglang PR #24696 page: activations quantised at run time, one
// scale per token row).  For each row r of a bf16 matrix:
//   scale[r] = max_k |a[r,k]| / 448   (1 for an all-zero row)
//   code[r,k] = E4M3 nearest-even of a[r,k] / scale[r]
// The division is IEEE fp32 and the conversion v_cvt_pk_fp8_f32 (round to
// nearest even, saturating at 448), so a code depends on the fp32 values alone.
//
// One 256-thread block per row; the row stays in registers between the maximum
// and the codes (8 bf16 per 16-byte load, up to 8 loads per thread: rows of at
// most 16384 elements, a multiple of 8).
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int QT = 256;
constexpr int QMAXV = 8;  // 16-byte loads per thread

__global__ __launch_bounds__(QT) void quant_rows_fp8_kernel(const bf16_t* __restrict__ in, int C, int64_t ld_in,
                                                            const int32_t* __restrict__ row_map,
                                                            const int32_t* __restrict__ m_dev, int64_t R,
                                                            uint8_t* __restrict__ codes, int64_t ld_out,
                                                            float* __restrict__ scales) {
  __shared__ float s_red[QT / 64];
  const int64_t r = blockIdx.x;
  const int64_t rows = m_dev ? (int64_t)*m_dev : R;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nv = C / 8;  // 16-byte pieces per row
  uint8_t* crow = codes + r * ld_out;
  // rows past the device count are left alone; padding rows (map < 0) get zero codes
  if (r >= rows) return;
  if (row_map && row_map[r] < 0) {
    for (int v = tid; v < nv; v += QT) *(uint2*)(crow + 8 * v) = make_uint2(0u, 0u);
    if (tid == 0) scales[r] = 1.f;
    return;
  }
  const bf16_t* arow = in + r * ld_in;
  uint4 x[QMAXV];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < QMAXV; ++i) {
    const int v = tid + i * QT;
    x[i] = v < nv ? *(const uint4*)(arow + 8 * v) : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t w[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      amax = fmaxf(amax, fabsf(__uint_as_float(w[q] << 16)));
      amax = fmaxf(amax, fabsf(__uint_as_float(w[q] & 0xFFFF0000u)));
    }
  }
  amax = wave_max_f32(amax);
  if (lane == 0) s_red[wave] = amax;
  __syncthreads();
  amax = s_red[0];
#pragma unroll
  for (int w = 1; w < QT / 64; ++w) amax = fmaxf(amax, s_red[w]);
  float s = amax / 448.0f;
  if (!(s > 0.f)) s = 1.f;
  if (tid == 0) scales[r] = s;
#pragma unroll
  for (int i = 0; i < QMAXV; ++i) {
    const int v = tid + i * QT;
    if (v >= nv) break;
    const uint32_t w[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
    uint32_t out[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float f0 = __uint_as_float(w[2 * h] << 16) / s, f1 = __uint_as_float(w[2 * h] & 0xFFFF0000u) / s;
      const float f2 = __uint_as_float(w[2 * h + 1] << 16) / s, f3 = __uint_as_float(w[2 * h + 1] & 0xFFFF0000u) / s;
      int p = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
      p = __builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, p, true);
      out[h] = (uint32_t)p;
    }
    *(uint2*)(crow + 8 * v) = make_uint2(out[0], out[1]);
  }
}
}  // namespace

hipError_t launch_quant_rows_fp8(const void* in, int64_t R, int C, int64_t ld_in, const int32_t* row_map,
                                 const int32_t* m_dev, uint8_t* codes, int64_t ld_out, float* scales,
                                 hipStream_t s) {
  if (R == 0) return hipSuccess;
  if (C % 8 || C > QT * QMAXV * 8 || ld_in % 8 || ld_out % 8) return hipErrorInvalidValue;
  quant_rows_fp8_kernel<<<dim3((unsigned)R), dim3(QT), 0, s>>>((const bf16_t*)in, C, ld_in, row_map, m_dev, R,
                                                                codes, ld_out, scales);
  return hipGetLastError();
}

}  // namespace moe
