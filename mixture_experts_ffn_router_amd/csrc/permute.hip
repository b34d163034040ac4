// Dispatch permutation: (token, slot) pairs regrouped expert-major, stable in
// the flat slot index, each expert segment padded to the GEMM's row block
// ("Gemma 4 26B-A4B MoE walkthrough" sections 6-7: dispatch builds a
// permutation map that the grouped GEMM reads indirectly; no token moves).
//
// Two launches, one workgroup (16 waves) per expert in each:
//   count:   expert e counts the slots whose id is e;
//   scatter: expert e sums the padded sizes of experts < e to find its segment,
//            then walks the ids in order, 4096 slots per step, and compacts the
//            matching flat slot indices.  A thread owns 4 consecutive slots;
//            its rank inside the step is an exclusive prefix of per-thread
//            match counts (0..4), taken from three ballots (one per bit of the
//            count) and per-wave totals in LDS, so the order is deterministic
//            and stable without atomics.  Pads get -1 and block_expert gets e.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int PERM_THREADS = 1024;
constexpr int PERM_STEP = PERM_THREADS * 4;

__device__ __forceinline__ int block_sum_i32(int v, int* s_red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // wave all-reduce on the u32 pattern (values are small non-negative ints)
  v = (int)wave_allreduce_u32((uint32_t)v, [](uint32_t a, uint32_t b) { return a + b; }, 0u);
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  int tot = 0;
  for (int w = 0; w < PERM_THREADS / 64; ++w) tot += s_red[w];
  __syncthreads();
  return tot;
}

__global__ __launch_bounds__(PERM_THREADS) void permute_count_kernel(const int32_t* __restrict__ ids,
                                                                     int64_t n, int32_t* __restrict__ counts) {
  __shared__ int s_red[PERM_THREADS / 64];
  const int e = blockIdx.x;
  int c = 0;
  for (int64_t f = (int64_t)threadIdx.x * 4; f < n; f += PERM_STEP) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (f + q < n && ids[f + q] == e) ++c;
  }
  c = block_sum_i32(c, s_red);
  if (threadIdx.x == 0) counts[e] = c;
}

__global__ __launch_bounds__(PERM_THREADS) void permute_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t n, int E, int bm_log2, const int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slots, int32_t* __restrict__ block_expert) {
  __shared__ int s_red[PERM_THREADS / 64];
  __shared__ int s_wtot[PERM_THREADS / 64];
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bm = 1 << bm_log2;
  auto padded_size = [&](int c) { return ((c + bm - 1) >> bm_log2) << bm_log2; };

  int part = 0;
  for (int j = tid; j < e; j += PERM_THREADS) part += padded_size(counts[j]);
  const int start = block_sum_i32(part, s_red);
  const int cnt = counts[e];
  const int padded = padded_size(cnt);
  if (tid == 0) {
    offsets[e] = start;
    if (e == E - 1) offsets[E] = start + padded;
  }

  const uint64_t lt = (1ull << lane) - 1ull;
  int running = 0;
  for (int64_t base = 0; base < n; base += PERM_STEP) {
    const int64_t f0 = base + (int64_t)tid * 4;
    uint32_t bits = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (f0 + q < n && ids[f0 + q] == e) bits |= 1u << q;
    const int c = __popc(bits);
    const uint64_t b0 = __ballot(c & 1), b1 = __ballot(c & 2), b2 = __ballot(c & 4);
    const int wprefix = __popcll(b0 & lt) + 2 * __popcll(b1 & lt) + 4 * __popcll(b2 & lt);
    if (lane == 0) s_wtot[wave] = __popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2);
    __syncthreads();
    int wbase = 0, btot = 0;
    for (int w = 0; w < PERM_THREADS / 64; ++w) {
      int x = s_wtot[w];
      wbase += (w < wave) ? x : 0;
      btot += x;
    }
    int pos = start + running + wbase + wprefix;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if ((bits >> q) & 1u) sorted_slots[pos++] = (int32_t)(f0 + q);
    running += btot;
    __syncthreads();
  }
  for (int i = cnt + tid; i < padded; i += PERM_THREADS) sorted_slots[start + i] = -1;
  for (int b = tid; b < (padded >> bm_log2); b += PERM_THREADS) block_expert[(start >> bm_log2) + b] = e;
}

hipError_t launch_permute(const int32_t* ids, int64_t n, int E, int bm_log2, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_slots, int32_t* block_expert,
                          hipStream_t s) {
  permute_count_kernel<<<E, PERM_THREADS, 0, s>>>(ids, n, counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  permute_scatter_kernel<<<E, PERM_THREADS, 0, s>>>(ids, n, E, bm_log2, counts, offsets, sorted_slots,
                                                    block_expert);
  return hipGetLastError();
}

}  // namespace moe
