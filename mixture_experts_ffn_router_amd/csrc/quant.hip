// Dynamic per-row FP8 quantisation of activations (the "FP8-Dynamic" scheme
// named on the sglang PR #24696 page: activations quantised at run time, one
// scale per token row).  For each row r of a bf16 matrix:
//   scale[r] = max_k |a[r,k]| / 448   (1 for an all-zero row)
//   code[r,k] = E4M3 nearest-even of a[r,k] / scale[r]
// The division is IEEE fp32 and the conversion v_cvt_pk_fp8_f32 (round to
// nearest even, saturating at 448), so a code depends on the fp32 values alone.
//
// The row stays in registers between the maximum and the codes (8 bf16 per
// 16-byte load, up to 8 loads per lane).  Rows of at most 4096 elements: one
// wavefront per row, four rows per block; longer rows (up to 16384): one
// 256-thread block per row.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int QT = 256;
constexpr int QMAXV = 8;  // 16-byte loads per lane

// Rows handled by NTH threads each (64: a wavefront; QT: the block).  Returns
// false for rows that need no work (past the count, or padding set to zeros).
template <int NTH>
__device__ __forceinline__ bool quant_row_prologue(int64_t r, int tid, int nv, const int32_t* row_map,
                                                   uint8_t* crow, float* scales) {
  if (row_map && row_map[r] < 0) {
    for (int v = tid; v < nv; v += NTH) *(uint2*)(crow + 8 * v) = make_uint2(0u, 0u);
    if (tid == 0) scales[r] = 1.f;
    return false;
  }
  return true;
}

__global__ __launch_bounds__(QT) void quant_rows_fp8_wave_kernel(const bf16_t* __restrict__ in, int C, int64_t ld_in,
                                                                 const int32_t* __restrict__ row_map,
                                                                 const int32_t* __restrict__ m_dev, int64_t R,
                                                                 uint8_t* __restrict__ codes, int64_t ld_out,
                                                                 float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * (QT / 64) + (threadIdx.x >> 6);
  const int64_t rows = m_dev ? (int64_t)*m_dev : R;
  if (r >= R || r >= rows) return;  // uniform per wave
  const int nv = C / 8;
  uint8_t* crow = codes + r * ld_out;
  if (!quant_row_prologue<64>(r, lane, nv, row_map, crow, scales)) return;
  const bf16_t* arow = in + r * ld_in;
  uint4 x[QMAXV];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < QMAXV; ++i) {
    const int v = lane + 64 * i;
    x[i] = v < nv ? *(const uint4*)(arow + 8 * v) : make_uint4(0u, 0u, 0u, 0u);
    amax = fmaxf(amax, absmax8(x[i]));
  }
  const float s = scale_of(wave_max_f32(amax));
  if (lane == 0) scales[r] = s;
#pragma unroll
  for (int i = 0; i < QMAXV; ++i) {
    const int v = lane + 64 * i;
    if (v < nv) *(uint2*)(crow + 8 * v) = codes8(x[i], s);
  }
}

__global__ __launch_bounds__(QT) void quant_rows_fp8_block_kernel(const bf16_t* __restrict__ in, int C, int64_t ld_in,
                                                                  const int32_t* __restrict__ row_map,
                                                                  const int32_t* __restrict__ m_dev, int64_t R,
                                                                  uint8_t* __restrict__ codes, int64_t ld_out,
                                                                  float* __restrict__ scales) {
  __shared__ float s_red[QT / 64];
  const int64_t r = blockIdx.x;
  const int64_t rows = m_dev ? (int64_t)*m_dev : R;
  if (r >= rows) return;  // uniform per block
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nv = C / 8;
  uint8_t* crow = codes + r * ld_out;
  if (!quant_row_prologue<QT>(r, tid, nv, row_map, crow, scales)) return;
  const bf16_t* arow = in + r * ld_in;
  uint4 x[QMAXV];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < QMAXV; ++i) {
    const int v = tid + i * QT;
    x[i] = v < nv ? *(const uint4*)(arow + 8 * v) : make_uint4(0u, 0u, 0u, 0u);
    amax = fmaxf(amax, absmax8(x[i]));
  }
  amax = wave_max_f32(amax);
  if (lane == 0) s_red[wave] = amax;
  __syncthreads();
  amax = s_red[0];
#pragma unroll
  for (int w = 1; w < QT / 64; ++w) amax = fmaxf(amax, s_red[w]);
  const float s = scale_of(amax);
  if (tid == 0) scales[r] = s;
#pragma unroll
  for (int i = 0; i < QMAXV; ++i) {
    const int v = tid + i * QT;
    if (v < nv) *(uint2*)(crow + 8 * v) = codes8(x[i], s);
  }
}
}  // namespace

hipError_t launch_quant_rows_fp8(const void* in, int64_t R, int C, int64_t ld_in, const int32_t* row_map,
                                 const int32_t* m_dev, uint8_t* codes, int64_t ld_out, float* scales,
                                 hipStream_t s) {
  if (R == 0) return hipSuccess;
  if (C % 8 || C > QT * QMAXV * 8 || ld_in % 8 || ld_out % 8) return hipErrorInvalidValue;
  if (C <= 64 * QMAXV * 8)
    quant_rows_fp8_wave_kernel<<<dim3((unsigned)((R + QT / 64 - 1) / (QT / 64))), dim3(QT), 0, s>>>(
        (const bf16_t*)in, C, ld_in, row_map, m_dev, R, codes, ld_out, scales);
  else
    quant_rows_fp8_block_kernel<<<dim3((unsigned)R), dim3(QT), 0, s>>>((const bf16_t*)in, C, ld_in, row_map, m_dev,
                                                                        R, codes, ld_out, scales);
  return hipGetLastError();
}

}  // namespace moe
