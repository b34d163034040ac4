// Dispatch permutation: (token, slot) pairs regrouped expert-major, stable in
// the flat slot index, each expert segment padded to the GEMM's row block
// ("Gemma 4 26B-A4B MoE walkthrough" sections 6-7: dispatch builds a
// permutation map that the grouped GEMM reads indirectly; no token moves).
//
// Two launches, one workgroup (16 waves) per expert in each:
//   count:   expert e counts the slots whose id is e;
//   scatter: expert e sums the padded sizes of experts < e to find its segment,
//            then walks the ids in order, 4096 slots per step (the next step's
//            ids loaded while this one is ranked), and compacts the matching
//            flat slot indices.  A thread owns 4 consecutive slots;
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

// ids f0 .. f0+3 (-1 past n, not read); one 16-byte load when the ids are
// 16-byte aligned and all four exist.
__device__ __forceinline__ int4 load_ids4(const int32_t* __restrict__ ids, int64_t n, int64_t f0, bool vec) {
  if (vec && f0 + 3 < n) return *(const int4*)(ids + f0);
  int4 r;
  r.x = f0 < n ? ids[f0] : -1;
  r.y = f0 + 1 < n ? ids[f0 + 1] : -1;
  r.z = f0 + 2 < n ? ids[f0 + 2] : -1;
  r.w = f0 + 3 < n ? ids[f0 + 3] : -1;
  return r;
}
__device__ __forceinline__ uint32_t match4(int4 v, int e) {
  return (uint32_t)(v.x == e) | ((uint32_t)(v.y == e) << 1) | ((uint32_t)(v.z == e) << 2) | ((uint32_t)(v.w == e) << 3);
}

__global__ __launch_bounds__(PERM_THREADS) void permute_count_kernel(const int32_t* __restrict__ ids,
                                                                     int64_t n, int32_t* __restrict__ counts,
                                                                     bool vec) {
  __shared__ int s_red[PERM_THREADS / 64];
  const int e = blockIdx.x;
  int c = 0;
  // the next step's ids are loaded before this step's are counted
  int64_t f = (int64_t)threadIdx.x * 4;
  int4 cur = load_ids4(ids, n, f, vec);
  for (; f < n; f += PERM_STEP) {
    const int4 nxt = load_ids4(ids, n, f + PERM_STEP, vec);
    c += __popc(match4(cur, e));
    cur = nxt;
  }
  c = block_sum_i32(c, s_red);
  if (threadIdx.x == 0) counts[e] = c;
}

__global__ __launch_bounds__(PERM_THREADS) void permute_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t n, int E, int bm_log2, const int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slots, int32_t* __restrict__ block_expert,
    bool vec) {
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
  int4 cur = load_ids4(ids, n, (int64_t)tid * 4, vec);
  for (int64_t base = 0; base < n; base += PERM_STEP) {
    const int64_t f0 = base + (int64_t)tid * 4;
    const int4 nxt = load_ids4(ids, n, f0 + PERM_STEP, vec);  // next step, in flight meanwhile
    const uint32_t bits = match4(cur, e);
    cur = nxt;
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
  const bool vec = ((uintptr_t)ids & 15) == 0;
  permute_count_kernel<<<E, PERM_THREADS, 0, s>>>(ids, n, counts, vec);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  permute_scatter_kernel<<<E, PERM_THREADS, 0, s>>>(ids, n, E, bm_log2, counts, offsets, sorted_slots,
                                                    block_expert, vec);
  return hipGetLastError();
}

}  // namespace moe
