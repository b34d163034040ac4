// Dispatch permutation: (token, slot) pairs regrouped expert-major, stable in
// the flat slot index, each expert segment padded to the GEMM's row block
// ("Gemma 4 26B-A4B MoE walkthrough" sections 6-7: dispatch builds a
// permutation map that the grouped GEMM reads indirectly; no token moves).
//
// Histogram, prefix scan, stable scatter; every id is read twice in all, so the
// cost is O(T*K + E) however many experts there are.  The ids are cut into
// chunks of CHUNK consecutive flat slots, one 1024-thread block per chunk.
//   hist:    block b counts its chunk's ids per expert in LDS and stores the E
//            counts in slot_row[b*CHUNK .. b*CHUNK + E) (the chunk's own part of
//            that output, free until the scatter writes it); a ragged last chunk,
//            whose part may be shorter than E, stores them in counts[] instead.
//   scan:    one block, a thread per expert: turns the full chunks' counts into
//            exclusive prefixes over the chunks (in place), adds the last
//            chunk's to get counts[e], scans the padded sizes over the experts
//            into offsets[], and writes block_expert[] and the -1 pads.
//   scatter: block b ranks each id among the equal ids before it in its chunk
//            (a wave's equal ids are found with one ballot per bit of the id;
//            waves are ordered through per-wave counts in LDS, so no atomics
//            decide any order), reads its chunk's prefixes into LDS before any
//            of its slot_row entries is overwritten, and writes
//            sorted_slots[pos] = f and slot_row[f] = pos with
//            pos = offsets[e] + (equal ids in earlier chunks) + rank.
// Only block b reads or writes slot_row[b*CHUNK, (b+1)*CHUNK) between the
// launches' boundaries, so the reuse is race-free.  Up to 8192 slots with few
// experts, one block takes the three steps in one launch instead.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int PT = 1024;             // threads per block
constexpr int PW = PT / 64;          // waves per block
constexpr int ROUNDS = 4;            // ids per thread per chunk
constexpr int CHUNK = PT * ROUNDS;   // flat slots per chunk (>= the largest E, 1024)

__device__ __forceinline__ int chunk_id(const int32_t* __restrict__ ids, int64_t n, int64_t f, int E) {
  if (f >= n) return -1;
  const int e = ids[f];
  return (e >= 0 && e < E) ? e : -1;  // ids outside [0, E) belong to no segment
}

// Bits of an id in [0, E): ceil(log2(E)), 0 for E = 1.
__device__ __forceinline__ int id_bits(int E) { return E <= 1 ? 0 : 32 - __clz(E - 1); }

// Lanes of this wave holding the same id as this lane: one ballot per bit of
// the id (nbits = id_bits(E)) and one for validity, so invalid lanes (-1) form
// their own group.
__device__ __forceinline__ uint64_t wave_match(int e, int nbits) {
  uint64_t same = __ballot(e >= 0);
  if (e < 0) same = ~same;
  for (int bit = 0; bit < nbits; ++bit) {
    const bool v = (e >> bit) & 1;
    const uint64_t bal = __ballot(v);
    same &= v ? bal : ~bal;
  }
  return same;
}

// Block-wide exclusive scan of one int per thread (1024 threads); returns the
// thread's exclusive prefix, *total the sum.
__device__ __forceinline__ int block_excl_scan(int v, int* s_w, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // inclusive scan inside the wave with shuffles (log steps)
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) s_w[wave] = incl;
  __syncthreads();
  int wbase = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < PW; ++w) {
    const int x = s_w[w];
    wbase += w < wave ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return wbase + incl - v;
}

// block_expert and pads from the padded segment offsets s_off[0..E] and counts
// s_cnt[E] in LDS: wave w takes experts w, w + PW, ...; its lanes write the
// expert's row blocks and pad rows (sorted_slots = -1) coalesced.  An empty
// expert owns no block.
__device__ __forceinline__ void write_blocks(int E, int bm_log2, const int* s_off, const int* s_cnt,
                                             int32_t* __restrict__ block_expert,
                                             int32_t* __restrict__ sorted_slots, bool pads) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int e = wave; e < E; e += PW) {
    const int o0 = s_off[e], o1 = s_off[e + 1];
    for (int j = (o0 >> bm_log2) + lane; j < (o1 >> bm_log2); j += 64) block_expert[j] = e;
    if (pads)
      for (int q = o0 + s_cnt[e] + lane; q < o1; q += 64) sorted_slots[q] = -1;
  }
}
}  // namespace

__global__ __launch_bounds__(PT) void permute_hist_kernel(const int32_t* __restrict__ ids, int64_t n, int E,
                                                          int32_t* __restrict__ slot_row,
                                                          int32_t* __restrict__ counts) {
  extern __shared__ int s_hist[];  // [E]
  const int b = blockIdx.x, tid = threadIdx.x;
  for (int e = tid; e < E; e += PT) s_hist[e] = 0;
  __syncthreads();
  const int64_t f0 = (int64_t)b * CHUNK;
  int e_r[ROUNDS];  // every id load in flight before the first is used
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) e_r[r] = chunk_id(ids, n, f0 + r * PT + tid, E);
  const uint64_t lt = (1ull << (tid & 63)) - 1ull;
  const int nbits = id_bits(E);
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    // one add per distinct id of the wave (a sum: the order of the adds does not matter)
    const uint64_t same = wave_match(e_r[r], nbits);
    if (e_r[r] >= 0 && (same & lt) == 0) atomicAdd(&s_hist[e_r[r]], __popcll(same));
  }
  __syncthreads();
  const bool full = f0 + CHUNK <= n;
  int32_t* dst = full ? slot_row + f0 : counts;
  for (int e = tid; e < E; e += PT) dst[e] = s_hist[e];
}

__global__ __launch_bounds__(PT) void permute_scan_kernel(int64_t n, int E, int bm_log2,
                                                          int32_t* __restrict__ slot_row,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted_slots,
                                                          int32_t* __restrict__ block_expert,
                                                          int32_t* __restrict__ num_padded) {
  __shared__ int s_w[PW];
  __shared__ int s_off[1025];
  __shared__ int s_cnt[1024];
  const int tid = threadIdx.x;
  const int64_t nfull = n / CHUNK;
  const bool tail = n % CHUNK != 0;
  const int bm = 1 << bm_log2;
  int cnt = 0;
  if (tid < E) {
    // exclusive prefix over the full chunks, in place; four loads in flight
    int32_t* p = slot_row + tid;
    int64_t c = 0;
    for (; c + 4 <= nfull; c += 4) {
      const int v0 = p[(c + 0) * CHUNK], v1 = p[(c + 1) * CHUNK], v2 = p[(c + 2) * CHUNK], v3 = p[(c + 3) * CHUNK];
      p[(c + 0) * CHUNK] = cnt;
      p[(c + 1) * CHUNK] = cnt + v0;
      p[(c + 2) * CHUNK] = cnt + v0 + v1;
      p[(c + 3) * CHUNK] = cnt + v0 + v1 + v2;
      cnt += v0 + v1 + v2 + v3;
    }
    for (; c < nfull; ++c) {
      const int v = p[c * CHUNK];
      p[c * CHUNK] = cnt;
      cnt += v;
    }
    if (tail) cnt += counts[tid];
    counts[tid] = cnt;
  }
  const int padded = ((cnt + bm - 1) >> bm_log2) << bm_log2;
  int total = 0;
  const int start = block_excl_scan(tid < E ? padded : 0, s_w, &total);
  if (tid < E) {
    offsets[tid] = start;
    s_off[tid] = start;
    s_cnt[tid] = cnt;
  }
  if (tid == 0) {
    offsets[E] = total;
    s_off[E] = total;
    if (num_padded) *num_padded = total;
  }
  __syncthreads();
  write_blocks(E, bm_log2, s_off, s_cnt, block_expert, sorted_slots, true);
}

__global__ __launch_bounds__(PT) void permute_scatter_kernel(const int32_t* __restrict__ ids, int64_t n, int E,
                                                             const int32_t* __restrict__ counts,
                                                             const int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ sorted_slots,
                                                             int32_t* __restrict__ slot_row) {
  extern __shared__ int s_dyn[];
  int* s_base = s_dyn;                        // [E] offsets[e] + equal ids before the current round
  uint16_t* s_wcnt = (uint16_t*)(s_dyn + E);  // [PW][E] per-wave counts of the current round (<= 64)
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t f0 = (int64_t)b * CHUNK;
  const bool full = f0 + CHUNK <= n;
  const int nbits = id_bits(E);
  int e_r[ROUNDS];
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) e_r[r] = chunk_id(ids, n, f0 + r * PT + tid, E);
  if (full) {
    for (int e = tid; e < E; e += PT) s_base[e] = offsets[e] + slot_row[f0 + e];
  } else {
    // the ragged last chunk: equal ids in earlier chunks = counts[e] - this chunk's
    for (int e = tid; e < E; e += PT) s_base[e] = offsets[e] + counts[e];
    __syncthreads();
    const uint64_t lt0 = (1ull << lane) - 1ull;
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {  // a count: the order does not matter
      const uint64_t same = wave_match(e_r[r], nbits);
      if (e_r[r] >= 0 && (same & lt0) == 0) atomicSub(&s_base[e_r[r]], __popcll(same));
    }
  }
  const uint64_t lt = (1ull << lane) - 1ull;
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int e = e_r[r];
    const uint64_t same = wave_match(e, nbits);
    for (int i = tid; i < PW * E; i += PT) s_wcnt[i] = 0;
    __syncthreads();  // zeroed; also: the previous round's reads of s_base are done
    const bool leader = (same & lt) == 0;
    if (e >= 0 && leader) s_wcnt[wave * E + e] = (uint16_t)__popcll(same);
    __syncthreads();
    if (e >= 0) {
      int pos = s_base[e] + __popcll(same & lt);
      for (int w = 0; w < wave; ++w) pos += s_wcnt[w * E + e];
      const int64_t f = f0 + r * PT + tid;
      sorted_slots[pos] = (int32_t)f;
      e_r[r] = pos;  // written to slot_row below, once every base read is done
    } else {
      e_r[r] = -1;
    }
    __syncthreads();
    for (int x = tid; x < E; x += PT) {
      int s = 0;
      for (int w = 0; w < PW; ++w) s += s_wcnt[w * E + x];
      s_base[x] += s;
    }
    __syncthreads();  // the sums above have read s_wcnt before the next round clears it
  }
  // every base of this chunk has been read (from slot_row for a full chunk)
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int64_t f = f0 + r * PT + tid;
    if (f < n) slot_row[f] = e_r[r];
  }
}

// Up to SMALL_N slots with few experts: the three steps in one block and one
// launch (the launches cost more than the work), in two passes over the ids
// held in registers.  Pass 1 ranks each id inside its wave and records every
// (round, wave)'s count per expert in an LDS table; parallel prefix steps turn
// the table into exclusive prefixes in (round, wave) order per expert; pass 2
// places each id at offsets[e] + its (round, wave) prefix + its rank.  When the
// padded rows fit in LDS, sorted_slots is assembled there (pads pre-filled) and
// written out in order: one CU's scattered stores to L2 would cost more.
// Round r covers slots [1024 r, 1024 (r + 1)), thread tid slot 1024 r + tid.
// Measured on MI355X: one launch costs about 7 us plus 0.5-1 us per 1024 slots
// (one CU's ballots), the three launches 12-16 us whatever the size; the one
// block wins up to about 8192 slots.
constexpr int SMALL_ROUNDS = 8;
constexpr int64_t SMALL_N = (int64_t)SMALL_ROUNDS * PT;  // 8192
constexpr int SMALL_TABLE = 32768;                       // uint16 table entries: rounds x waves x E
constexpr int SMALL_STAGE = 36864;                       // ints of LDS: table + round prefixes, then rows
static_assert(SMALL_TABLE / 2 + SMALL_TABLE / PW <= SMALL_STAGE, "LDS plan");

__global__ __launch_bounds__(PT) void permute_small_kernel(const int32_t* __restrict__ ids, int64_t n, int E,
                                                           int bm_log2, int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ sorted_slots,
                                                           int32_t* __restrict__ block_expert,
                                                           int32_t* __restrict__ num_padded,
                                                           int32_t* __restrict__ slot_row) {
  __shared__ __align__(16) int s_big[SMALL_STAGE];
  uint16_t* s_tab = reinterpret_cast<uint16_t*>(s_big);  // [round][wave][E]: counts, then exclusive prefixes
  int* s_rpre = s_big + SMALL_TABLE / 2;                   // [round][E]: round totals, then their prefixes
  __shared__ int s_off[1025];
  __shared__ int s_cnt[1024];
  __shared__ int s_w[PW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bm = 1 << bm_log2;
  const int rounds = (int)((n + PT - 1) / PT);
  const int ncell = rounds * PW * E;
  const int nbits = id_bits(E);
  int e_r[SMALL_ROUNDS];  // every id of the call, all loads in flight at once
#pragma unroll
  for (int r = 0; r < SMALL_ROUNDS; ++r) e_r[r] = chunk_id(ids, n, (int64_t)r * PT + tid, E);
  for (int i = tid; i < (ncell + 7) / 8; i += PT) reinterpret_cast<int4*>(s_big)[i] = make_int4(0, 0, 0, 0);
  __syncthreads();
  const uint64_t lt = (1ull << lane) - 1ull;
  int pos[SMALL_ROUNDS];  // rank inside the (round, wave), then the row
#pragma unroll
  for (int r = 0; r < SMALL_ROUNDS; ++r) {
    pos[r] = 0;
    if (r < rounds) {  // uniform
      const uint64_t same = wave_match(e_r[r], nbits);
      pos[r] = __popcll(same & lt);
      if (e_r[r] >= 0 && pos[r] == 0) s_tab[(r * PW + wave) * E + e_r[r]] = (uint16_t)__popcll(same);
    }
  }
  __syncthreads();
  // (1) each round's total per expert
  const int nre = rounds * E;
  for (int i = tid; i < nre; i += PT) {  // (round r, expert e) = (i / E, i % E)
    const int r = i / E, e = i - r * E;
    int tot = 0;
#pragma unroll
    for (int w = 0; w < PW; ++w) tot += s_tab[(r * PW + w) * E + e];
    s_rpre[i] = tot;
  }
  __syncthreads();
  // (2) exclusive prefixes over the rounds: a group of R = 2^lgR >= rounds lanes
  // per expert scans with shuffles; the group's last lane holds the count
  const int lgR = rounds <= 1 ? 0 : 32 - __clz(rounds - 1);
  const int nit = E << lgR;
  for (int base = 0; base < nit; base += PT) {  // uniform trip count: every lane shuffles
    const int i = base + tid;
    const int e = i >> lgR, r = i & ((1 << lgR) - 1);
    const bool ok = i < nit && r < rounds;
    const int v = ok ? s_rpre[r * E + e] : 0;
    int incl = v;
    for (int d = 1; d < (1 << lgR); d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (r >= d) incl += o;
    }
    if (ok) s_rpre[r * E + e] = incl - v;
    if (i < nit && r == (1 << lgR) - 1) s_cnt[e] = incl;
  }
  __syncthreads();
  // (3) exclusive prefixes over the waves inside each round
  for (int i = tid; i < nre; i += PT) {
    const int r = i / E, e = i - r * E;
    int run = s_rpre[i];
#pragma unroll
    for (int w = 0; w < PW; ++w) {
      const int c = (r * PW + w) * E + e;
      const int v = s_tab[c];
      s_tab[c] = (uint16_t)run;  // < SMALL_N: fits
      run += v;
    }
  }
  const int cnt = tid < E ? (rounds ? s_cnt[tid] : 0) : 0;
  const int padded = ((cnt + bm - 1) >> bm_log2) << bm_log2;
  int total = 0;
  const int start = block_excl_scan(tid < E ? padded : 0, s_w, &total);  // also orders step (3)
  if (tid < E) {
    counts[tid] = cnt;
    offsets[tid] = start;
    s_off[tid] = start;
    s_cnt[tid] = cnt;
  }
  if (tid == 0) {
    offsets[E] = total;
    s_off[E] = total;
    if (num_padded) *num_padded = total;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < SMALL_ROUNDS; ++r)
    pos[r] = (r < rounds && e_r[r] >= 0) ? s_off[e_r[r]] + s_tab[(r * PW + wave) * E + e_r[r]] + pos[r] : -1;
  const bool staged = total <= SMALL_STAGE;  // uniform
  write_blocks(E, bm_log2, s_off, s_cnt, block_expert, sorted_slots, !staged);
  if (staged) {
    __syncthreads();  // every table read above is done
    for (int i = tid; i < total; i += PT) s_big[i] = -1;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < SMALL_ROUNDS; ++r)
      if (pos[r] >= 0) s_big[pos[r]] = r * PT + tid;
    __syncthreads();
    for (int i = tid; i < total; i += PT) sorted_slots[i] = s_big[i];
  } else {
#pragma unroll
    for (int r = 0; r < SMALL_ROUNDS; ++r)
      if (pos[r] >= 0) sorted_slots[pos[r]] = r * PT + tid;
  }
#pragma unroll
  for (int r = 0; r < SMALL_ROUNDS; ++r) {
    const int64_t f = (int64_t)r * PT + tid;
    if (r < rounds && f < n) slot_row[f] = pos[r];
  }
}

hipError_t launch_permute(const int32_t* ids, int64_t n, int E, int bm_log2, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_slots, int32_t* block_expert, int32_t* num_padded,
                          int32_t* slot_row, hipStream_t s) {
  if (E < 1 || E > 1024) return hipErrorInvalidValue;
  if (n <= SMALL_N && ((n + PT - 1) / PT) * PW * E <= SMALL_TABLE) {
    permute_small_kernel<<<1, PT, 0, s>>>(ids, n, E, bm_log2, counts, offsets, sorted_slots, block_expert,
                                          num_padded, slot_row);
    return hipGetLastError();
  }
  const int64_t nchunks = (n + CHUNK - 1) / CHUNK;
  if (nchunks > 0) {
    permute_hist_kernel<<<(unsigned)nchunks, PT, E * sizeof(int), s>>>(ids, n, E, slot_row, counts);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  permute_scan_kernel<<<1, PT, 0, s>>>(n, E, bm_log2, slot_row, counts, offsets, sorted_slots, block_expert,
                                       num_padded);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nchunks == 0) return err;
  permute_scatter_kernel<<<(unsigned)nchunks, PT, (size_t)E * sizeof(int) + (size_t)PW * E * sizeof(uint16_t), s>>>(
      ids, n, E, counts, offsets, sorted_slots, slot_row);
  return hipGetLastError();
}

}  // namespace moe
