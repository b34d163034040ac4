// Grouped expert GEMMs for gfx950 ("Gemma 4 26B-A4B MoE walkthrough" sections
// 6-7: grouped GEMM by expert over the permutation map, gated activation,
// weighted combine; "MOE Inference": gated FFN with the merged w13;
// llama.cpp lesson 35: mul_mat_id computes only the selected experts).
//
// C[r, n] = sum_k A[row(r), k] * B_e[n, k] for every row block of the padded,
// expert-major row list; e = the block's expert.  Both operands are
// K-contiguous ("NT"), which is what the MFMA operand layout wants.
//
// MFMA kernel (v_mfma_f32_32x32x16_bf16; FP8 x FP8: 32x32x64), 4 or 8 waves:
//   * BM x BN output tile; every operand tile reaches LDS through buffer loads
//     that write LDS directly (no staging registers), in K tiles of 64.  8 waves
//     ping-pong over 2 A stages and (where LDS holds them) 3 B stages, so the
//     weight tiles stream two K tiles ahead (see pingpong_dma64).  4 waves run a software
//     pipeline over up to 4 stages: tiles kt+1 .. kt+NS-1 are in flight while
//     tile kt computes, and the waits are explicit vmcnt counts, so only the
//     oldest tile is waited for.  Buffer resources bound each operand, so a load
//     past the end returns 0.
//   * LDS rows of 64 / 128 bytes; the 16-byte chunk index is XORed with a
//     function of the row so the 16 lanes of each ds_read_b128 phase hit
//     distinct banks.
//   * Software pipeline: fragments are double-buffered in registers, the LDS
//     reads of the next sub-step (including the first of the next tile, right
//     after the barrier) in flight while the MFMAs of this one run.
//   * A rows are gathered straight from x through the row map (no permuted copy
//     of the activations); B rows come from the block's expert.
//   * The MFMA is issued as B x A, so each lane's accumulator holds 4
//     consecutive output columns of one row (8- or 16-byte direct stores).
//   * Gated epilogue: the B tile holds BN/2 gate rows (w1) and the matching
//     BN/2 up rows (w3), so the gate and up accumulators of a lane cover the
//     same (row, col); h = act(g) * u is formed in registers and stored bf16.
//     The [rows, 2I] product never reaches memory.
//   * Scatter epilogue (down projection): y = acc * routing weight of the row's
//     slot, stored (bf16, or fp32 when the branch is renormalised afterwards)
//     at the slot's row of the per-slot buffer; pad rows are skipped.  The
//     per-token sum happens in the finalize kernel in slot order.  The bf16
//     scatter and the fp32 store epilogues stage the tile in LDS and copy whole
//     rows out with 16-byte stores on consecutive lanes.
//   * Atomic scatter epilogue (the weighted scatter-add combine): the staged
//     rows are added into their token's fp32 row with float atomics, every
//     reduction part into the same row; the sum order then varies between runs.
//   * FP8 B (OCP E4M3 codes, W8A16): B rows are 64 bytes in LDS, widened to bf16
//     in registers (exact), and the per-output-channel scale is applied in the
//     epilogue: sum_k x_k (q_kn s_n) = s_n sum_k x_k q_kn.
//   * FP8 A and B (W8A8, activations quantised per row at run time, the
//     "FP8-Dynamic" scheme of the sglang PR #24696 page): v_mfma_f32_32x32x64_f8f6f4
//     on the 8-wave tiles, 128-deep K tiles (128-byte LDS rows, as bf16), one
//     instruction per half K tile; sum_k (p_tk a_t)(q_kn s_n) = a_t s_n sum_k p_tk q_kn,
//     so the row scale a_t and the channel scale s_n multiply the accumulator.
//   * Per-token row scale: an RMSNorm without a learned weight is a per-row
//     factor, so x_t / rms_t . W = (x_t . W) / rms_t; the epilogue applies it to
//     the accumulator and the normalised rows are never rounded or stored.
//
// fp32 kernel (the fp32 layer): plain LDS-tiled FMA, 64x64 tile, same epilogues.
#include <atomic>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

template <int BELEM>
struct BTraits;
template <>
struct BTraits<ELEM_BF16> {
  static constexpr int ELEM_BYTES = 2;
};
template <>
struct BTraits<ELEM_FP8> {
  static constexpr int ELEM_BYTES = 1;
};
template <>
struct BTraits<ELEM_FP8X8> {
  static constexpr int ELEM_BYTES = 1;
};

typedef __attribute__((address_space(3))) void lds_void;
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x8 __attribute__((ext_vector_type(8)));

// 16 bytes per lane, global -> LDS: lane l's data lands at dst + 16 l (dst wave-uniform).
__device__ __forceinline__ void dma16(rsrc_t r, void* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, (int)voff, (int)soff, 0, 0);
}

// Tile order.  The grid is persistent: block b walks tiles t = b, b + G, ... with
// G a multiple of 8, and blocks are dealt to the 8 XCDs round-robin, so XCD x
// runs the tiles t = x (mod 8).  Renumber so each XCD walks a contiguous range of
// logical tiles.  Logical tiles are laid out segment by segment (a segment is
// the row blocks of one expert, or all row blocks when rows are not grouped by
// expert), each segment cut into near-equal chunks of at most GMAX row blocks,
// and within a chunk the row block runs fastest: the tiles an XCD runs at once
// are the chunk's row blocks times a few column tiles, so each weight tile is
// read from memory once per chunk and the rest come from the XCD's L2.  A fixed
// group height would straddle experts and stream their weights several times.
// Only row blocks that hold rows are counted, so no block idles on padding and
// the XCDs stay balanced.
__device__ __forceinline__ int64_t xcd_logical(int64_t t, int64_t per_xcd, bool xcd_map) {
  constexpr int XCDS = 8;
  return xcd_map ? (t % XCDS) * per_xcd + t / XCDS : t;
}
__device__ __forceinline__ void tile_coords(int64_t lid, int64_t mbn, int64_t nb_cnt, const int32_t* block_expert,
                                            const int32_t* seg_off, int bm, int64_t& mb, int64_t& nb) {
  constexpr int GMAX = 8;
  // A chunk starting at row block s owns logical tiles [s * nb_cnt, (s + h) * nb_cnt),
  // so lid / nb_cnt is a row block of lid's chunk, and of its segment.
  const int64_t r = lid / nb_cnt;
  int64_t f = 0, n = mbn;
  if (block_expert) {
    const int e = block_expert[r];
    f = seg_off[e] / bm;
    n = (seg_off[e + 1] - seg_off[e]) / bm;
  }
  const int64_t j = r - f, q = (n + GMAX - 1) / GMAX;  // block within the segment; chunks
  int64_t c = j * q / n;                                // chunk c: segment blocks [c n / q, (c + 1) n / q)
  while ((c + 1) * n / q <= j) ++c;
  while (c * n / q > j) --c;
  const int64_t c0 = c * n / q, h = (c + 1) * n / q - c0;
  const int64_t local = lid - (f + c0) * nb_cnt;
  mb = f + c0 + local % h;
  nb = local / h;
}

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14])
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// LDS row layout: a K-tile row is 64 or 128 bytes of 16-byte chunks; chunk c of
// row r sits at chunk c ^ swz(r).  A fragment read has 16 consecutive lanes on
// 16 consecutive rows at the same logical chunk, and gfx950 serves a
// ds_read_b128 16 lanes (256 bytes, all 64 banks) per cycle: the swizzle puts
// those 16 reads in 16 distinct 16-byte bank groups (it is also conflict-free
// for 8-lane / 128-byte phases).  With row bits b3..b0:
//   64-byte rows (4 chunks):  swz = (b2, b1 ^ b3)
//   128-byte rows (8 chunks): swz = (b2, b1, b0 ^ b3)
template <int ROW_BYTES>
__device__ __forceinline__ int lds_swz(int row) {
  if constexpr (ROW_BYTES == 128) return (row & 6) | ((row ^ (row >> 3)) & 1);
  else return ((row & 4) >> 1) | (((row >> 1) ^ (row >> 3)) & 1);
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int EPI, int BELEM>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N)
__attribute__((amdgpu_waves_per_eu(WAVES_M * WAVES_N / 4, WAVES_M * WAVES_N / 4)))
void gemm_mfma_kernel(GemmArgs p) {
  constexpr bool FP8 = BELEM == ELEM_FP8;    // FP8 B widened to bf16 (W8A16)
  constexpr bool A8 = BELEM == ELEM_FP8X8;   // FP8 A and B: v_mfma_f32_32x32x64_f8f6f4
  constexpr bool WSC = FP8 || A8;            // per-output-channel weight scales
  constexpr int EA = A8 ? 1 : 2;             // A element bytes
  // All operand tiles reach LDS by DMA (buffer_load ... lds) in 64-deep K tiles,
  // so each lane fetches 16 bytes of a 128-byte bf16 row piece (fp8: 64-byte
  // pieces) and an instruction covers whole cache lines.  8 waves: ping-pong in
  // 2 stages.  4 waves: software pipeline in up to 4 stages (as many as fit).
  constexpr bool PP = WAVES_M * WAVES_N == 8;
  // 64-deep K tiles (128-byte bf16 rows); FP8 x FP8: 128-deep (128-byte rows too)
  constexpr int BK = A8 ? 128 : 64;
  static_assert(!A8 || PP, "FP8 activations run on the 8-wave ping-pong tiles");
  constexpr int STAGE_B = BM * BK * EA + BN * BK * BTraits<BELEM>::ELEM_BYTES;
  constexpr int NS = PP ? 2 : (160 * 1024 / STAGE_B < 4 ? 160 * 1024 / STAGE_B : 4);
  static_assert(PP || NS >= 3, "the pipeline keeps at least two tiles in flight");
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr bool GATED = EPI == EPI_GATED;
  constexpr int EB = BTraits<BELEM>::ELEM_BYTES;
  constexpr int NW = WAVES_M * WAVES_N;  // 4 waves (1 per SIMD) or 8 (2 per SIMD)
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(TM >= 1 && TN >= 1, "wave tile");
  static_assert(!GATED || (TN % 2 == 0), "gated needs gate/up tile pairs");
  constexpr int A_ROW = BK * EA;
  constexpr int B_ROW = BK * EB;
  constexpr int A_BYTES = BM * A_ROW;
  constexpr int B_BYTES = BN * B_ROW;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int A_DMA = A_BYTES / 1024 / NW;  // 1 KiB DMA instructions per wave per stage
  constexpr int B_DMA = B_BYTES / 1024 / NW;
  constexpr int A_CH = A_ROW / 16, B_CH = B_ROW / 16;  // 16-byte chunks per row
  constexpr int A_ROWS_PER_DMA = 1024 / A_ROW, B_ROWS_PER_DMA = 1024 / B_ROW;
  constexpr int D_TILE = A_DMA + B_DMA;
  static_assert(A_DMA >= 1 && B_DMA >= 1 && A_DMA * NW * 1024 == A_BYTES && B_DMA * NW * 1024 == B_BYTES,
                "stage must split into 1 KiB DMA instructions over the waves");
  static_assert(!GATED || ((BN / 2) % B_ROWS_PER_DMA == 0), "DMA groups must not straddle gate/up");
  static_assert(NS * STAGE <= 160 * 1024, "LDS");
  // 8 waves: two A stages and, where LDS holds them, three B stages, so the
  // weight tile of K tile t+2 streams in while tile t computes (weights come
  // from HBM, whose latency under load outlasts the two phases a two-stage
  // ring leaves them); else two B stages.
  constexpr int NBS = PP ? ((2 * A_BYTES + 3 * B_BYTES <= 160 * 1024) ? 3 : 2) : 0;
  constexpr int LDS_MAIN = PP ? 2 * A_BYTES + NBS * B_BYTES : NS * STAGE;
  constexpr int NCOLS = GATED ? BN / 2 : BN;  // output columns per block
  constexpr int OESZ = (GATED || EPI == EPI_SCATTER) ? 2 : 4;  // output element bytes
  constexpr int EROWB = NCOLS * OESZ + 4 * OESZ;  // staged output row (padded)
  constexpr int EPASS = (BM * (EROWB + 4) + 160 * 1024 - 1) / (160 * 1024);
  constexpr int PROWS = BM / EPASS;
  // staged rows + their output row indices (gated and fp32 scatter epilogues
  // store directly)
  constexpr int EPI_LDS = (EPI == EPI_GATED || EPI == EPI_SCATTER_F32) ? 0 : PROWS * EROWB + PROWS * 4;
  static_assert(WAVES_M % EPASS == 0 && EPI_LDS <= 160 * 1024, "epilogue passes of whole wave rows");
  constexpr int SMEM = LDS_MAIN > EPI_LDS ? LDS_MAIN : EPI_LDS;
  constexpr int THREADS = 64 * WAVES_M * WAVES_N;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar) index
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int64_t m_rows = p.m_dev ? (int64_t)(*p.m_dev) : p.M;
  const int64_t mbn = (m_rows + BM - 1) / BM;  // row blocks holding rows
  const int64_t nb_cnt = (p.N + NCOLS - 1) / NCOLS;
  const int KS = p.k_splits;  // reduction parts (scatter and store epilogues), the slowest tile index
  const int64_t ntiles = mbn * nb_cnt * KS;
  const bool xcd_map = gridDim.x % 8 == 0;
  const int64_t per_xcd = (ntiles + 7) / 8;
  const int64_t tend = xcd_map ? per_xcd * 8 : ntiles;
  // Rows whose slot is -1 are padding: their operand loads are issued out of
  // range (zero fill, no memory traffic), a wave whose rows are all padding skips
  // its MFMAs, and nothing is stored for them.
  const int32_t* pad_map = p.a_rows ? p.a_rows : p.c_rows;
  for (int64_t t = blockIdx.x; t < tend; t += gridDim.x) {
  const int64_t lid = xcd_logical(t, per_xcd, xcd_map);
  if (lid >= ntiles) continue;  // uniform per block
  int64_t mb, nbi;
  const int ks = (int)(lid / (mbn * nb_cnt));
  tile_coords(lid % (mbn * nb_cnt), mbn, nb_cnt, p.block_expert, p.seg_off, BM, mb, nbi);
  __syncthreads();  // the previous tile's LDS reads are done in every wave
  const int64_t m0 = mb * BM;
  const int n0 = (int)nbi * NCOLS;
  const int e = p.block_expert ? p.block_expert[mb] : 0;
  const bool routed = e < p.n_routed;
  const int64_t eoff = routed ? (int64_t)e : (int64_t)(e - p.n_routed);
  const uint8_t* Bbase = (const uint8_t*)(routed ? p.B0 : p.B1) + eoff * p.bstride * EB;
  const float* bscale = nullptr;
  if constexpr (WSC) bscale = (routed ? p.bscale0 : p.bscale1) + eoff * p.sstride;
  const bool wave_live = m0 + wm * WM < m_rows && (!pad_map || pad_map[m0 + wm * WM] >= 0);

  const rsrc_t rsA = make_rsrc(p.A, (uint32_t)(p.a_rows_alloc * p.lda * EA));
  const rsrc_t rsB = make_rsrc(Bbase, (uint32_t)((int64_t)(GATED ? 2 * p.N : p.N) * p.Kdim * EB));

  // K tiles [kt0, kt0 + nk) of this reduction part.  FP8 x FP8 with Kdim % 128
  // == 64 ends in a half tile (ktail): its chunks past Kdim load as zeros.
  const int nkt = (p.Kdim + BK - 1) / BK;
  const int ktail = (p.Kdim % BK) ? nkt - 1 : -1;
  const int kt0 = ks * nkt / KS;
  const int nk = (ks + 1) * nkt / KS - kt0;

  // LDS row of the wave's B tile j (output-column tile)
  auto b_lds_row = [&](int j) {
    if constexpr (GATED) {
      constexpr int TH = TN / 2;
      return (j < TH) ? (wn * (WN / 2) + 32 * j) : (BN / 2 + wn * (WN / 2) + 32 * (j - TH));
    } else {
      return wn * WN + 32 * j;
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int l32 = lane & 31, hsel = lane >> 5;
  int a_row_off[TM], b_row_off[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) a_row_off[i] = (wm * WM + 32 * i + l32) * A_ROW;
#pragma unroll
  for (int j = 0; j < TN; ++j) b_row_off[j] = (b_lds_row(j) + l32) * B_ROW;
  // every fragment row of this lane is l32 modulo 32
  const int swa = lds_swz<A_ROW>(l32), swb = lds_swz<B_ROW>(l32);

  // Sub-steps of a K tile: bf16 16 k each; fp8 32 k each (one 16-byte B read
  // feeds two MFMAs, see below).
  constexpr int NA = FP8 ? 2 : 1;
  struct FragsW {
    bf16x8 a[TM][NA];
    u32x4 b[TN];
  };
  // FP8 x FP8 sub-step s (64 deep): each lane holds 32 bytes of its row, bytes
  // [64s + 32hsel, +32) (chunks 4s + 2hsel and 4s + 2hsel + 1), the same bytes
  // for A and B, so the instruction pairs matching k.
  struct Frags8 {
    u32x8 a[TM];
    u32x8 b[TN];
  };
  using Frags = std::conditional_t<A8, Frags8, FragsW>;
  auto load_frags_ab = [&](const uint8_t* sa, const uint8_t* sb, int s, Frags& f) {
    if constexpr (A8) {
      const int c = 4 * s + 2 * hsel;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        f.a[i].lo = *(const u32x4*)(sa + a_row_off[i] + ((c ^ swa) << 4));
        f.a[i].hi = *(const u32x4*)(sa + a_row_off[i] + (((c + 1) ^ swa) << 4));
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        f.b[j].lo = *(const u32x4*)(sb + b_row_off[j] + ((c ^ swb) << 4));
        f.b[j].hi = *(const u32x4*)(sb + b_row_off[j] + (((c + 1) ^ swb) << 4));
      }
      return;
    } else {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if constexpr (!FP8) {
        const int c = 2 * s + hsel;
        f.a[i][0] = *(const bf16x8*)(sa + a_row_off[i] + ((c ^ swa) << 4));
      } else {
        // fp8 sub-step s: B bytes [16c, 16c+16), c = 2s + hsel, hold k in
        // [32s + 16hsel, +16); the first 8 pair with A chunk 4s + 2hsel, the next 8
        // with 4s + 2hsel + 1.  Both MFMAs together cover k in [32s, 32s + 32) once.
        const int ca = 4 * s + 2 * hsel;
        f.a[i][0] = *(const bf16x8*)(sa + a_row_off[i] + ((ca ^ swa) << 4));
        f.a[i][1] = *(const bf16x8*)(sa + a_row_off[i] + (((ca + 1) ^ swa) << 4));
      }
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int c = 2 * s + hsel;
      f.b[j] = *(const u32x4*)(sb + b_row_off[j] + ((c ^ swb) << 4));
    }
    }
  };
  auto load_frags = [&](int buf, int s, Frags& f) {
    load_frags_ab(smem + buf * STAGE, smem + buf * STAGE + A_BYTES, s, f);
  };
  auto mfmas = [&](const Frags& f) {
    if constexpr (A8) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const i32x8 bj = __builtin_bit_cast(i32x8, f.b[j]);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const i32x8 ai = __builtin_bit_cast(i32x8, f.a[i]);
          // E4M3 x E4M3 (format selectors 0), no block scales
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bj, ai, acc[i][j], 0, 0, 0, 0, 0, 0);
        }
      }
      return;
    } else {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      if constexpr (!FP8) {
        const bf16x8 bj = __builtin_bit_cast(bf16x8, f.b[j]);
#pragma unroll
        for (int i = 0; i < TM; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bj, f.a[i][0], acc[i][j], 0, 0, 0);
      } else {
        const bf16x8 b1 = fp8x8_to_bf16x8(f.b[j][0], f.b[j][1]);
        const bf16x8 b2 = fp8x8_to_bf16x8(f.b[j][2], f.b[j][3]);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1, f.a[i][0], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b2, f.a[i][1], acc[i][j], 0, 0, 0);
        }
      }
    }
    }
  };

  // ---- pipeline: tiles kt+1 .. kt+NS-1 are in flight while tile kt computes.
  // A wave whose rows are all padding runs the same DMA / barrier sequence
  // without fragment reads or MFMAs.
  // ---- LDS-DMA source offsets.  Instruction i of this wave fills ROWS_PER_DMA
  // consecutive tile rows; lane l writes row base + l / CH, physical chunk l % CH,
  // which holds logical chunk (l % CH) ^ swz(row).
  struct DmaPlan {
    uint32_t a_off[A_DMA];
    uint32_t b_voff[2];  // by bit 3 of the group's first row (128-byte rows swizzle on it)
    uint32_t b_soff[B_DMA];
  };
  auto dma_plan = [&]() {
    DmaPlan d;
#pragma unroll
    for (int i = 0; i < A_DMA; ++i) {
      const int r = (wave * A_DMA + i) * A_ROWS_PER_DMA + lane / A_CH;
      const int64_t grow = m0 + r;
      const int slot = (pad_map && grow < p.M) ? pad_map[grow] : 0;
      int64_t tok;
      if (p.a_rows) tok = slot >= 0 ? slot / p.row_div : 0;
      else tok = grow < p.M ? grow : p.M - 1;
      d.a_off[i] = (grow >= m_rows || slot < 0)
                       ? 0x80000000u
                       : (uint32_t)(tok * p.lda * EA) + (uint32_t)((((lane % A_CH) ^ lds_swz<A_ROW>(r))) << 4);
    }
    // row within a DMA group (groups of 16 rows of 64 bytes or 8 rows of 128 bytes,
    // starting at multiples of their size: the swizzle of row q0 + bl_row depends
    // on bl_row and, for 128-byte rows, on bit 3 of q0)
    const int bl_row = lane / B_CH;
#pragma unroll
    for (int k = 0; k < 2; ++k)
      d.b_voff[k] = (uint32_t)(bl_row * p.Kdim * EB) +
                    (uint32_t)(((lane % B_CH) ^ lds_swz<B_ROW>(bl_row + 8 * k)) << 4);
#pragma unroll
    for (int i = 0; i < B_DMA; ++i) {
      const int q0 = (wave * B_DMA + i) * B_ROWS_PER_DMA;
      int brow;
      if constexpr (GATED) brow = q0 < BN / 2 ? n0 + q0 : p.N + n0 + (q0 - BN / 2);
      else brow = n0 + q0;
      d.b_soff[i] = (uint32_t)((int64_t)brow * p.Kdim * EB);
    }
    return d;
  };
  // Tile kt into stage buf; tiles past the end are issued with an out-of-range
  // offset, which the buffer bound turns into zero fill without a memory access.
  auto issue_dma = [&](const DmaPlan& d, int kt, int buf) {
    static_assert(B_ROWS_PER_DMA % 8 == 0, "B DMA groups must start at multiples of 8 rows");
    uint8_t* sA = smem + buf * STAGE;
    uint8_t* sB = sA + A_BYTES;
    const bool live = kt < nk;
#pragma unroll
    for (int i = 0; i < A_DMA; ++i)
      dma16(rsA, sA + (wave * A_DMA + i) * 1024, live ? d.a_off[i] : 0x80000000u, live ? (uint32_t)(kt0 + kt) * A_ROW : 0u);
#pragma unroll
    for (int i = 0; i < B_DMA; ++i)
      dma16(rsB, sB + (wave * B_DMA + i) * 1024, live ? d.b_voff[(((wave * B_DMA + i) * B_ROWS_PER_DMA) >> 3) & 1] : 0x80000000u,
            live ? d.b_soff[i] + (uint32_t)(kt0 + kt) * (uint32_t)B_ROW : 0u);
  };

  auto pipeline = [&](auto live_tag) {
    constexpr bool LIVE = decltype(live_tag)::value;
    const DmaPlan dp = dma_plan();
    auto load_frags_l = [&](int b, int s_, Frags& f) {
      if constexpr (LIVE) load_frags(b, s_, f);
    };
    auto mfmas_l = [&](const Frags& f) {
      if constexpr (LIVE) mfmas(f);
    };
  constexpr int R_SUB = TM * NA + TN;             // LDS reads per sub-step
  constexpr int M_SUB = TM * TN * (FP8 ? 2 : 1);  // MFMAs per sub-step
  constexpr int SUBS = BK / (FP8 ? 32 : 16);      // sub-steps per K tile
  static_assert(SUBS == 2 || SUBS == 4, "2 or 4 sub-steps");
#pragma unroll
  for (int t = 0; t < NS - 1; ++t) issue_dma(dp, t, t);
  wait_vmcnt<(NS - 2) * D_TILE>();  // this wave's part of tile 0
  __builtin_amdgcn_s_barrier();      // everyone's part of tile 0
  Frags f[2];
  load_frags_l(0, 0, f[0]);
  int buf = 0;
  for (int kt = 0; kt < nk; ++kt) {
    const int nbuf = buf + 1 == NS ? 0 : buf + 1;
    // Sub-step s < SUBS-1: read the fragments of sub-step s+1 while the MFMAs of
    // sub-step s run.  Sub-step s's fragments were read a sub-step ago; waiting
    // for them first (before new reads) keeps the wait from covering the reads
    // issued next.  Sub-step 0 also refills the stage that held tile kt-1: every
    // wave finished reading it before the barrier of the previous iteration.
    auto sub_step = [&](auto s_c) {
      constexpr int S = decltype(s_c)::value;
      wait_lgkmcnt0();
      load_frags_l(buf, S + 1, f[(S + 1) & 1]);
      if constexpr (S == 0) issue_dma(dp, kt + NS - 1, buf == 0 ? NS - 1 : buf - 1);
      mfmas_l(f[S & 1]);
      // issue order: the reads, then the MFMAs (with the DMAs between the first
      // of them in sub-step 0)
      __builtin_amdgcn_sched_group_barrier(0x100, R_SUB, 0);   // DS read
      if constexpr (S == 0) {
#pragma unroll
        for (int q = 0; q < D_TILE; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM (LDS DMA)
        }
        if (M_SUB > D_TILE) __builtin_amdgcn_sched_group_barrier(0x008, M_SUB - D_TILE, 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, M_SUB, 0);
      }
    };
    sub_step(std::integral_constant<int, 0>{});
    if constexpr (SUBS == 4) {
      sub_step(std::integral_constant<int, 1>{});
      sub_step(std::integral_constant<int, 2>{});
    }
    // Own reads of tile kt done and own DMA of tile kt+1 landed; the barrier
    // extends both to every wave.  Tiles kt+2 .. kt+NS-1 stay in flight.
    wait_lgkmcnt0();
    wait_vmcnt<(NS - 2) * D_TILE>();
    __builtin_amdgcn_s_barrier();
    // last sub-step, with the next tile's sub-step 0 reads between its MFMAs
    load_frags_l(nbuf, 0, f[0]);
    mfmas_l(f[1]);
#pragma unroll
    for (int q = 0; q < R_SUB; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if (M_SUB > R_SUB) __builtin_amdgcn_sched_group_barrier(0x008, M_SUB - R_SUB, 0);
    buf = nbuf;
  }

  };
  // ---- ping-pong (8 waves): the two groups of 4 waves (one wave of each
  // group per SIMD) run offset by one barrier phase.  In a memory phase a wave
  // reads the fragments of half a K tile (32 deep) from LDS and issues its share
  // of a later tile's DMA; in a compute phase it runs that half tile's MFMAs from
  // registers only (fp8 weights: with their conversion to bf16).  While one group
  // computes, the other loads, so each SIMD's
  // matrix pipe alternates between its two waves.  The scheduler may not move
  // anything (MFMAs included) across a phase boundary.
  auto phase_barrier = [] {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // 64-deep K tiles in 2 LDS stages (32-deep tiles in more stages would halve
  // the row pieces each DMA lane fetches and cost L2 bandwidth).  Each K tile
  // takes four phases: group 0 reads half 0 of tile t in phase 4t and half 1 in
  // phase 4t+2, computing each in the next phase; group 1 runs one phase behind.
  // A stage is refilled in parts, each written only when no wave can still read
  // it.  Group 0's wave rows (the lower half of the A tile) are read by group 0
  // alone, last in phase 4t-2 for tile t-1: group 1 refills them for tile t+1 in
  // phase 4t-1, right after its own reads (which never touch those rows), so
  // those loads get four phases.  Group 1's A rows and the B tile are read by
  // group 1 until phase 4t-1: group 0 refills group 1's A rows and the first
  // half of the B rows in phase 4t, group 1 the second half of the B rows in
  // phase 4t+1, each after its fragment reads (of the other stage).  Each wave
  // waits for its own parts in its last phase before phase 4t+4, where tile
  // t+1 is first read (group 0 at the end of its compute phase 4t+3, group 1 at
  // the end of its memory phase 4t+3); the barrier closing phase 4t+3 makes
  // every part visible.
  auto pingpong_dma64 = [&](auto live_tag) {
    constexpr bool LIVE = decltype(live_tag)::value;
    const int grp = wave >> 2, gw = wave & 3;
    constexpr int NA = A_BYTES / 1024, NB = B_BYTES / 1024;  // 1 KiB DMA instructions per stage
    constexpr int AH = NA / 8;   // A instructions per wave for one half of the A tile
    constexpr int BH = NB / 8;   // B instructions per wave for one half of the B tile
    static_assert(AH * 8 == NA && BH * 8 == NB, "DMA parts must split evenly over 4 waves");
    static_assert(AH + BH <= 32, "one bit per DMA instruction");
    static_assert(4 % WAVES_N == 0 && WAVES_M == 2 * (4 / WAVES_N) && (NA / 2) * A_ROWS_PER_DMA == BM / 2,
                  "each group's wave rows are one half of the A tile (group 0 the lower)");
    // This wave's A instructions: group 1 the lower half of the A tile (group
    // 0's wave rows), group 0 the upper half; B instructions: group 0 the first
    // half of the B tile, group 1 the second.
    const int ia0 = (grp == 1 ? 0 : NA / 2) + gw * AH;
    const int ib0 = (grp == 1 ? NB / 2 : 0) + gw * BH;
    uint32_t a_off[AH], b_soff[BH], b_voff[2];
#pragma unroll
    for (int i = 0; i < AH; ++i) {
      const int r = (ia0 + i) * A_ROWS_PER_DMA + lane / A_CH;
      const int64_t grow = m0 + r;
      const int slot = (pad_map && grow < p.M) ? pad_map[grow] : 0;
      int64_t tok;
      if (p.a_rows) tok = slot >= 0 ? slot / p.row_div : 0;
      else tok = grow < p.M ? grow : p.M - 1;
      a_off[i] = (grow >= m_rows || slot < 0)
                     ? 0x80000000u
                     : (uint32_t)(tok * p.lda * EA) + (uint32_t)((((lane % A_CH) ^ lds_swz<A_ROW>(r))) << 4);
    }
    // A half K tile (FP8 x FP8, Kdim % 128 == 64): chunks at or past Kdim load as
    // zeros.  Bit i (A instruction i) / AH + i (B instruction i) of past_k: this
    // lane's global chunk of that instruction lies past Kdim in such a tile.
    uint32_t past_k = 0;
    if constexpr (A8) {
      const int tail_ch = (p.Kdim % BK) * EA / 16;
#pragma unroll
      for (int i = 0; i < AH; ++i)
        if (((lane % A_CH) ^ lds_swz<A_ROW>((ia0 + i) * A_ROWS_PER_DMA + lane / A_CH)) >= tail_ch)
          past_k |= 1u << i;
#pragma unroll
      for (int i = 0; i < BH; ++i)
        if (((lane % B_CH) ^ lds_swz<B_ROW>(lane / B_CH + 8 * ((((ib0 + i) * B_ROWS_PER_DMA) >> 3) & 1))) >= tail_ch)
          past_k |= 1u << (AH + i);
    }
    {
      const int bl_row = lane / B_CH;
#pragma unroll
      for (int k = 0; k < 2; ++k)
        b_voff[k] = (uint32_t)(bl_row * p.Kdim * EB) +
                    (uint32_t)(((lane % B_CH) ^ lds_swz<B_ROW>(bl_row + 8 * k)) << 4);
#pragma unroll
      for (int i = 0; i < BH; ++i) {
        const int q0 = (ib0 + i) * B_ROWS_PER_DMA;
        int brow;
        if constexpr (GATED) brow = q0 < BN / 2 ? n0 + q0 : p.N + n0 + (q0 - BN / 2);
        else brow = n0 + q0;
        b_soff[i] = (uint32_t)((int64_t)brow * p.Kdim * EB);
      }
    }
    // this wave's A part / B part of tile kt into A stage abuf / B stage bbuf (past
    // the end: zero fill).  LDS: A stages [0, 2 A_BYTES), then the B stages.
    auto a_stage = [&](int buf) { return smem + buf * A_BYTES; };
    auto b_stage = [&](int buf) { return smem + 2 * A_BYTES + buf * B_BYTES; };
    auto issue_a = [&](int kt, int buf) {
      uint8_t* sA = a_stage(buf);
      const bool live = kt < nk;
      const bool tail = A8 && kt0 + kt == ktail;
#pragma unroll
      for (int i = 0; i < AH; ++i) {
        const bool on = live && !(tail && ((past_k >> i) & 1u));
        dma16(rsA, sA + (ia0 + i) * 1024, on ? a_off[i] : 0x80000000u, live ? (uint32_t)(kt0 + kt) * A_ROW : 0u);
      }
    };
    auto issue_b = [&](int kt, int buf) {
      uint8_t* sB = b_stage(buf);
      const bool live = kt < nk;
      const bool tail = A8 && kt0 + kt == ktail;
#pragma unroll
      for (int i = 0; i < BH; ++i) {
        const bool on = live && !(tail && ((past_k >> (AH + i)) & 1u));
        dma16(rsB, sB + (ib0 + i) * 1024, on ? b_voff[(((ib0 + i) * B_ROWS_PER_DMA) >> 3) & 1] : 0x80000000u,
              live ? b_soff[i] + (uint32_t)(kt0 + kt) * (uint32_t)B_ROW : 0u);
      }
    };
    // With three B stages the B tile of K tile t+2 is issued during tile t (its
    // stage held tile t-1, read for the last time in phase 4t-1), and the waits
    // leave this wave's BW loads of it in flight; near the end, where it is not
    // issued, they wait for everything.
    constexpr int BAHEAD = NBS - 1;        // B tiles issued ahead of the one computing
    constexpr int BW = NBS == 3 ? BH : 0;  // this wave's B loads left in flight at a wait
    Frags f[2];
    issue_a(0, 0);
    issue_b(0, 0);
    const bool b1 = NBS == 3 && nk > 1;
    if (b1) issue_b(1, 1);
    if (grp == 1) {
      issue_a(1, 1);
      if (b1) wait_vmcnt<AH + BW>();  // this wave's parts of tile 0
      else wait_vmcnt<AH>();
    } else {
      if (b1) wait_vmcnt<BW>();
      else wait_vmcnt<0>();
    }
    phase_barrier();
    if (grp == 1) phase_barrier();
    constexpr int SPH = A8 ? 1 : BK / (FP8 ? 32 : 16) / 2;  // sub-steps per half tile
    int bs = 0;  // B stage of tile t (t % NBS)
    for (int t = 0; t < nk; ++t) {
      const int st = t & 1;
      const int bnext = bs + BAHEAD >= NBS ? bs + BAHEAD - NBS : bs + BAHEAD;  // B stage of tile t + BAHEAD
      const bool bfar = t + BAHEAD < nk;  // B of tile t + BAHEAD is issued this tile
      const uint8_t* sa = a_stage(st);
      const uint8_t* sb = b_stage(bs);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        // memory phase: fragment reads first, so they do not queue behind the
        // DMA's LDS writes
        if constexpr (LIVE) {
#pragma unroll
          for (int q = 0; q < SPH; ++q) load_frags_ab(sa, sb, SPH * hh + q, f[q]);
        }
        if (hh == 0) {
          if (grp == 0 && t + 1 < nk) issue_a(t + 1, st ^ 1);  // group 1's rows of tile t+1
          if (bfar) issue_b(t + BAHEAD, bnext);                 // this group's half of the B rows
        }
        wait_lgkmcnt0();
        if (hh == 1 && grp == 1) {
          // own parts of tile t+1 have landed
          if (NBS == 3 && bfar) wait_vmcnt<BW>();
          else wait_vmcnt<0>();
          if (t + 2 < nk) issue_a(t + 2, st);  // group 0's rows of tile t: read for the last time in phase 4t+2
        }
        phase_barrier();
        // compute phase
        if constexpr (LIVE) {
#pragma unroll
          for (int q = 0; q < SPH; ++q) mfmas(f[q]);
        }
        if (hh == 1 && grp == 0) {  // own parts of tile t+1 have landed
          if (NBS == 3 && bfar) wait_vmcnt<BW>();
          else wait_vmcnt<0>();
        }
        phase_barrier();
      }
      bs = bs + 1 == NBS ? 0 : bs + 1;
    }
    if (grp == 0) phase_barrier();  // same barrier count in both groups
  };

  if constexpr (PP) {
    if (wave_live) pingpong_dma64(std::true_type{});
    else pingpong_dma64(std::false_type{});
  } else {
    if (wave_live) pipeline(std::true_type{});
    else pipeline(std::false_type{});
  }

  // ---- epilogue.  acc[i][j][v]: row = m0 + wm*WM + 32i + l32,
  //      col (tile-local) = 8*(v/4) + 4*hsel + (v%4)
  // Per-row factors of the tile row grow: token factor (row_scale) and, for the
  // scatter epilogue, the routing weight of its slot.
  auto row_factor = [&](int64_t grow) {
    float rs = 1.f;
    if (grow >= m_rows) return rs;  // past the rows: nothing is stored for it
    if (p.row_scale) {
      int64_t tok = grow;
      if (p.a_rows) {
        const int slot = p.a_rows[grow];
        tok = slot >= 0 ? slot / p.row_div : 0;
      }
      rs = p.row_scale[tok];
    }
    if constexpr (EPI == EPI_SCATTER || EPI == EPI_SCATTER_F32 || EPI == EPI_SCATTER_ATOMIC) {
      const int slot = p.c_rows[grow];
      rs *= (slot >= 0 && p.row_weight) ? p.row_weight[slot] : 1.f;  // (x the A row's scale, if any)
    } else if constexpr (EPI == EPI_STORE_F32) {
      rs *= p.c_scale;
    }
    return rs;
  };
  // The 4 output values of acc[i][j][4*g4 .. 4*g4+3] (j < TN/2 for gated)
  // at tile-local column col, with factor rs.
  auto out4 = [&](int i, int j, int g4, int col, float rs, float* v) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (GATED) {
        constexpr int TH = TN / 2;
        float gv = acc[i][j][4 * g4 + q] * rs, uv = acc[i][j + TH][4 * g4 + q] * rs;
        if constexpr (WSC) {
          gv *= bscale[n0 + col + q];
          uv *= bscale[p.N + n0 + col + q];
        }
        v[q] = apply_act_bf16(p.act, gv) * uv;
      } else {
        v[q] = acc[i][j][4 * g4 + q] * rs;
        if constexpr (WSC) v[q] *= bscale[n0 + col + q];
      }
    }
  };
  // Output row of tile row grow, or -1 when nothing is stored for it.
  auto out_row = [&](int64_t grow) -> int64_t {
    if (grow >= m_rows) return -1;
    if constexpr (GATED) return (p.a_rows && p.a_rows[grow] < 0) ? -1 : grow;  // padding: never read back
    else if constexpr (EPI == EPI_SCATTER || EPI == EPI_SCATTER_F32) {
      const int slot = p.c_rows[grow];
      return slot < 0 ? -1 : (int64_t)slot * KS + ks;  // the part's row of this slot
    } else if constexpr (EPI == EPI_SCATTER_ATOMIC) {
      const int slot = p.c_rows[grow];
      return slot < 0 ? -1 : (int64_t)(slot / p.row_div);  // the slot's token: every part adds to it
    } else {
      return (int64_t)ks * p.M + grow;  // part ks's plane of [KS, M, ldc]
    }
  };
  constexpr int CPL = 16 / OESZ;  // output elements per 16 bytes
  // The bf16 scatter and the fp32 store epilogues stage their tile in LDS
  // (below); it needs 16-byte aligned output rows and column groups: always so
  // for the scatter epilogue (checked at launch), not for the router's logits
  // (E columns).  The gated and fp32 scatter epilogues store directly (8 / 16
  // bytes per lane, 16 / 32 contiguous bytes per row): staging them measured
  // no faster.
  bool staged = EPI == EPI_SCATTER || EPI == EPI_STORE_F32 || EPI == EPI_SCATTER_ATOMIC;
  if constexpr (EPI == EPI_STORE_F32 && !PP)
    staged = (p.N % CPL) == 0 && (p.ldc % CPL) == 0 && (((uintptr_t)p.C & 15) == 0);
  if (staged) {
    // Stage the tile's outputs in LDS, row-major (rows padded by 4 elements, so
    // the 32 rows a fragment store spans hit distinct banks), then copy whole
    // rows out with 16-byte stores on consecutive lanes: the MFMA layout would
    // store 32 rows x 16-32 bytes per instruction.  Tiles larger than LDS go
    // in passes of whole wave rows.
    wait_vmcnt<0>();  // no DMA (zero fill past the last K tile) still writing LDS
    __syncthreads();  // every wave done reading the pipeline's stages
#pragma unroll 1
    for (int pass = 0; pass < EPASS; ++pass) {
      if (pass) __syncthreads();  // the previous pass's rows are copied out
      if (wave_live && wm / (WAVES_M / EPASS) == pass) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int rl = wm * WM + 32 * i + l32 - pass * PROWS;  // row in this pass
          const float rs = row_factor(m0 + wm * WM + 32 * i + l32);
#pragma unroll
          for (int j = 0; j < (GATED ? TN / 2 : TN); ++j) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const int col = (GATED ? wn * (WN / 2) : wn * WN) + 32 * j + 8 * g4 + 4 * hsel;
              float v[4] = {0.f, 0.f, 0.f, 0.f};
              if (n0 + col < p.N) out4(i, j, g4, col, rs, v);  // columns past N: not stored
              uint8_t* d = smem + rl * EROWB + col * OESZ;
              if constexpr (OESZ == 2) {
                uint2 pk;
                pk.x = pack_bf16x2(v[0], v[1]);
                pk.y = pack_bf16x2(v[2], v[3]);
                *(uint2*)d = pk;
              } else {
                *(float4*)d = make_float4(v[0], v[1], v[2], v[3]);
              }
            }
          }
        }
      }
      // output row of each staged row (one row-map lookup per row), kept in LDS
      // after the staged rows
      int32_t* s_orow = (int32_t*)(smem + PROWS * EROWB);
      for (int r = tid; r < PROWS; r += THREADS) s_orow[r] = (int32_t)out_row(m0 + pass * PROWS + r);
      __syncthreads();
      if constexpr (EPI == EPI_SCATTER_ATOMIC) {
        // weighted rows added into their token's fp32 row: one element per lane,
        // consecutive lanes on consecutive columns (an instruction covers 256
        // contiguous bytes of one row)
        for (int idx = tid; idx < PROWS * NCOLS; idx += THREADS) {
          const int r = idx / NCOLS, c = idx - r * NCOLS;
          const int col = n0 + c;
          const int32_t orow = s_orow[r];
          if (orow < 0 || col >= p.N) continue;
          unsafeAtomicAdd((float*)p.C + (int64_t)orow * p.ldc + col, *(const float*)(smem + r * EROWB + c * 4));
        }
      } else {
        constexpr int CHR = NCOLS * OESZ / 16;  // 16-byte chunks per row
        for (int idx = tid; idx < PROWS * CHR; idx += THREADS) {
          const int r = idx / CHR, c = idx - r * CHR;
          const int col = n0 + c * CPL;
          const int32_t orow = s_orow[r];
          if (orow < 0 || col >= p.N) continue;
          *(uint4*)((uint8_t*)p.C + ((int64_t)orow * p.ldc + col) * OESZ) = *(const uint4*)(smem + r * EROWB + c * 16);
        }
      }
    }
  } else if constexpr (GATED) {
    // h = act(g) * u, 4 consecutive bf16 outputs (8 bytes) per lane and store
    constexpr int TH = TN / 2;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t grow = m0 + wm * WM + 32 * i + l32;
      if (grow >= m_rows || !wave_live) continue;
      // Padding rows (slot -1) hold zeros (their A rows load as zeros) and are
      // stored like the others, so no row-map lookup waits here unless a
      // per-token factor needs the row's token.
      float rs = 1.f;
      if (p.row_scale) {
        const int slot = p.a_rows ? p.a_rows[grow] : 0;
        if (slot < 0) continue;  // padding: never read back
        rs = p.row_scale[p.a_rows ? slot / p.row_div : grow];
      }
      bf16_t* C = (bf16_t*)p.C + grow * p.ldc;
#pragma unroll
      for (int j = 0; j < TH; ++j) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int col = n0 + wn * (WN / 2) + 32 * j + 8 * g4 + 4 * hsel;
          if (col >= p.N) continue;
          float h[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float gv = acc[i][j][4 * g4 + q] * rs, uv = acc[i][j + TH][4 * g4 + q] * rs;
            if constexpr (WSC) {
              gv *= bscale[col + q];
              uv *= bscale[p.N + col + q];
            }
            h[q] = apply_act_bf16(p.act, gv) * uv;
          }
          uint2 pk;
          pk.x = pack_bf16x2(h[0], h[1]);
          pk.y = pack_bf16x2(h[2], h[3]);
          *(uint2*)(C + col) = pk;
        }
      }
    }
  } else if constexpr (EPI == EPI_SCATTER_F32 || (EPI == EPI_STORE_F32 && !PP)) {
    // Direct fp32 stores: 4 consecutive outputs per lane (16 bytes) when the row
    // is aligned for it (always for the scatter epilogue), else one element at
    // a time (the router's logits).
    const bool vec = EPI == EPI_SCATTER_F32 || ((p.N % 4) == 0 && (p.ldc % 4) == 0 && (((uintptr_t)p.C & 15) == 0));
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t grow = m0 + wm * WM + 32 * i + l32;
      const int64_t orow = wave_live ? out_row(grow) : -1;
      if (orow < 0) continue;
      const float rs = row_factor(grow);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int col = wn * WN + 32 * j + 8 * g4 + 4 * hsel;
          if (n0 + col >= p.N) continue;
          float v[4];
          out4(i, j, g4, col, rs, v);
          float* d = (float*)p.C + orow * p.ldc + n0 + col;
          if (vec) {
            *(float4*)d = make_float4(v[0], v[1], v[2], v[3]);
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (n0 + col + q < p.N) d[q] = v[q];
          }
        }
      }
    }
  }
  }  // tile loop
}

// ------------------------------------------------------------------ fp32 path
// 64x64 output tile (gated: 32 gate + 32 up B rows), BK = 16, 16x16 threads,
// each owning 4 rows x 4 B columns.  Gated threads own 2 gate and the same 2
// up columns, so act(g) * u needs no exchange.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs p) {
  constexpr int BM = 64, BN = 64, BK = 16;
  constexpr bool GATED = EPI == EPI_GATED;
  constexpr int NCOLS = GATED ? BN / 2 : BN;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int64_t mb_cap = (p.M + BM - 1) / BM;
  const int64_t mb = (int64_t)blockIdx.x % mb_cap;
  const int nb = (int)((int64_t)blockIdx.x / mb_cap);
  const int64_t m_rows = p.m_dev ? (int64_t)(*p.m_dev) : p.M;
  const int64_t m0 = mb * BM;
  if (m0 >= m_rows) return;
  const int n0 = nb * NCOLS;
  const int e = p.block_expert ? p.block_expert[mb] : 0;
  const bool routed = e < p.n_routed;
  const int64_t eoff = routed ? (int64_t)e : (int64_t)(e - p.n_routed);
  const float* B = (const float*)(routed ? p.B0 : p.B1) + eoff * p.bstride;

  // loads: thread -> (row = tid/4, k4 = tid%4)
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  int64_t tok;
  {
    const int64_t grow = m0 + lr;
    if (p.a_rows) {
      const int slot = grow < p.M ? p.a_rows[grow] : -1;
      tok = slot >= 0 ? slot / p.row_div : 0;
    } else {
      tok = grow < p.M ? grow : p.M - 1;
    }
  }
  const float* a_src = (const float*)p.A + tok * p.lda + lk;
  int brow;
  if (GATED) {
    const int qq = lr % (BN / 2);
    const int col = min(n0 + qq, p.N - 1);
    brow = lr < BN / 2 ? col : p.N + col;
  } else {
    brow = min(n0 + lr, p.N - 1);
  }
  const float* b_src = B + (int64_t)brow * p.Kdim + lk;

  // B columns owned: gated -> LDS rows {2tx, 2tx+1, 32+2tx, 32+2tx+1}; else 4tx..4tx+3
  int bc[4];
  for (int q = 0; q < 4; ++q) bc[q] = GATED ? ((q < 2) ? 2 * tx + q : 32 + 2 * tx + (q - 2)) : 4 * tx + q;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < p.Kdim; k0 += BK) {
    const float4 av = *(const float4*)(a_src + k0);
    const float4 bv = *(const float4*)(b_src + k0);
    As[lk + 0][lr] = av.x; As[lk + 1][lr] = av.y; As[lk + 2][lr] = av.z; As[lk + 3][lr] = av.w;
    Bs[lk + 0][lr] = bv.x; Bs[lk + 1][lr] = bv.y; Bs[lk + 2][lr] = bv.z; Bs[lk + 3][lr] = bv.w;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      float a[4], b[4];
      for (int r = 0; r < 4; ++r) a[r] = As[k][ty * 4 + r];
      for (int q = 0; q < 4; ++q) b[q] = Bs[k][bc[q]];
      for (int r = 0; r < 4; ++r)
        for (int q = 0; q < 4; ++q) acc[r][q] = fmaf(a[r], b[q], acc[r][q]);
    }
    __syncthreads();
  }
  for (int r = 0; r < 4; ++r) {
    const int64_t grow = m0 + ty * 4 + r;
    if (grow >= m_rows) continue;
    float rs = 1.f;
    if (p.row_scale) {
      int64_t tk = grow;
      if (p.a_rows) {
        const int slot = p.a_rows[grow];
        tk = slot >= 0 ? slot / p.row_div : 0;
      }
      rs = p.row_scale[tk];
    }
    if (GATED) {
      float* C = (float*)p.C + grow * p.ldc;
      for (int q = 0; q < 2; ++q) {
        const int col = n0 + 2 * tx + q;
        if (col < p.N) C[col] = apply_act(p.act, acc[r][q] * rs) * (acc[r][q + 2] * rs);
      }
    } else if (EPI == EPI_SCATTER) {
      const int slot = p.c_rows[grow];
      if (slot < 0) continue;
      const float w = p.row_weight ? p.row_weight[slot] : 1.f;
      float* C = (float*)p.C + (int64_t)slot * p.ldc;
      for (int q = 0; q < 4; ++q) {
        const int col = n0 + 4 * tx + q;
        if (col < p.N) C[col] = acc[r][q] * w;
      }
    } else {
      float* C = (float*)p.C + grow * p.ldc;
      for (int q = 0; q < 4; ++q) {
        const int col = n0 + 4 * tx + q;
        if (col < p.N) C[col] = acc[r][q] * rs * p.c_scale;
      }
    }
  }
}

// ------------------------------------------------------------------ dispatch
// Host-side caches below are atomics: several host threads may launch at once
// (each computes the same value; whichever store lands first is kept).
int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (!v) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
    v = n;
  }
  return v;
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int EPI, int BELEM>
static hipError_t run_mfma(const GemmArgs& a, hipStream_t s) {
  constexpr int NCOLS = EPI == EPI_GATED ? BN / 2 : BN;
  constexpr int THREADS = 64 * WAVES_M * WAVES_N;
  const int64_t mb_cap = (a.M + BM - 1) / BM;
  const int64_t nb = (a.N + NCOLS - 1) / NCOLS;
  const int64_t tiles = mb_cap * nb * a.k_splits;  // upper bound; the kernel counts the real ones
  if (tiles <= 0) return hipSuccess;
  auto kern = gemm_mfma_kernel<BM, BN, WAVES_M, WAVES_N, EPI, BELEM>;
  static std::atomic<int> per_cu_cache{0};  // resident blocks per CU for this instantiation
  int per_cu = per_cu_cache.load(std::memory_order_relaxed);
  if (!per_cu) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, THREADS, 0) != hipSuccess || n <= 0) n = 1;
    per_cu_cache.store(n, std::memory_order_relaxed);
    per_cu = n;
  }
  const int64_t resident = (int64_t)device_cu_count() * per_cu;
  const int64_t grid = tiles < resident ? tiles : resident;
  kern<<<dim3((unsigned)grid), dim3(THREADS), 0, s>>>(a);
  return hipGetLastError();
}

// A tile ncols output columns wide is worth it when its last column block idles
// at most a tenth of N past N, and the tiles still number at least one per CU
// (rows: the row capacity, an upper bound; times the reduction parts).
static bool wide_fits(const GemmArgs& a, int block_m, int ncols) {
  const int64_t N = a.N;
  if (((N + ncols - 1) / ncols * ncols - N) * 10 > N) return false;
  return (a.M + block_m - 1) / block_m * ((N + ncols - 1) / ncols) * a.k_splits >= (int64_t)device_cu_count();
}

template <int EPI, int BELEM>
static hipError_t run_grouped(const GemmArgs& a, int block_m, hipStream_t s) {
  const int N = a.N;
  if (block_m == 256) {
    // 8-wave 256x256 tiles (gated: 128 output columns) unless they would idle
    // too many columns; a ragged last column block reads zeros past the weights
    // and stores nothing past N.
    if (wide_fits(a, 256, EPI == EPI_GATED ? 128 : 256)) return run_mfma<256, 256, 4, 2, EPI, BELEM>(a, s);
    return run_mfma<256, 128, 4, 1, EPI, BELEM>(a, s);
  }
  if (block_m == 128) return run_mfma<128, 512, 2, 4, EPI, BELEM>(a, s);
  if (block_m == 64) {
    if (EPI == EPI_GATED) {
      if (N % 128 == 0) return run_mfma<64, 256, 1, 4, EPI, BELEM>(a, s);
      return run_mfma<64, 128, 2, 2, EPI, BELEM>(a, s);
    }
    if (N % 256 == 0) return run_mfma<64, 256, 1, 4, EPI, BELEM>(a, s);
    return run_mfma<64, 128, 2, 2, EPI, BELEM>(a, s);
  }
  return hipErrorInvalidValue;
}

// The 256-row configurations hold one block per CU (their LDS stages take most
// of it), so a grid round is one tile per CU.  A part must keep at least 32 K
// tiles so the pipeline's fill stays small against it.
int gemm_scatter_k_splits(int64_t rows, int block_m, int N, int Kdim) {
  if (block_m != 256 || rows <= 0) return 1;
  const int bn = N % 256 == 0 ? 256 : 128;
  const int64_t tiles = (rows + block_m - 1) / block_m * ((N + bn - 1) / bn);
  const int64_t slots = device_cu_count();
  int best = 1;
  double best_rounds = 1e300;
  for (int ks = 1; ks <= 4 && (Kdim / 64) / ks >= 32; ++ks) {
    const double rounds = (double)((tiles * ks + slots - 1) / slots) / ks;  // in full-reduction tile times
    if (rounds < best_rounds - 1e-9) {
      best_rounds = rounds;
      best = ks;
    }
  }
  return best;
}

int gemm_scatter_k_splits_max(int block_m, int Kdim) {
  if (block_m != 256) return 1;
  int ks = 1;
  while (ks < 4 && (Kdim / 64) / (ks + 1) >= 32) ++ks;
  return ks;
}

// Reduction parts for a store GEMM over identity rows (the router): enough tiles
// for about two per CU, each part keeping at least 8 K tiles of 32.
int gemm_store_k_splits(int64_t M, int N, int Kdim) {
  if (M <= 0 || N <= 0) return 1;
  const int64_t tiles = (M + 127) / 128 * ((N + (N <= 64 ? 63 : 127)) / (N <= 64 ? 64 : 128));
  int ks = (int)((2 * device_cu_count() + tiles - 1) / tiles);
  ks = ks < 1 ? 1 : (ks > 8 ? 8 : ks);
  while (ks > 1 && (Kdim / 32) / ks < 8) --ks;
  return ks;
}

hipError_t launch_gemm_mfma(const GemmArgs& a, int epi, int belem, int block_m, hipStream_t s) {
  if (a.k_splits < 1 || (a.k_splits > 1 && epi == EPI_GATED)) return hipErrorInvalidValue;
  // Gated and scatter epilogues store groups of 4 or 8 consecutive outputs
  // (8 or 16 bytes), and so does the store epilogue of 256-row blocks (possibly
  // an 8-wave tile); the 4-wave store tiles of 64- and 128-row blocks also take
  // unaligned outputs.
  const int cpl = epi == EPI_GATED || epi == EPI_SCATTER ? 8 : 4;
  const bool aligned = a.N % cpl == 0 && a.ldc % cpl == 0 && ((uintptr_t)a.C & 15) == 0;
  if (!aligned && (epi != EPI_STORE_F32 || block_m == 256)) return hipErrorInvalidValue;
  if (epi == EPI_STORE_F32) {
    if (belem != ELEM_BF16) return hipErrorInvalidValue;
    if (block_m == 128) {
      if (a.N <= 64) return run_mfma<128, 64, 4, 1, EPI_STORE_F32, ELEM_BF16>(a, s);
      return run_mfma<128, 128, 2, 2, EPI_STORE_F32, ELEM_BF16>(a, s);
    }
    return run_grouped<EPI_STORE_F32, ELEM_BF16>(a, block_m, s);
  }
  if (belem == ELEM_FP8X8) {
    // FP8 activations: 8-wave tiles only, K a multiple of 64 (a final half tile is masked)
    if (a.Kdim % 64 || epi == EPI_STORE_F32 || (block_m != 128 && block_m != 256)) return hipErrorInvalidValue;
    if (block_m == 256) {
      if (epi == EPI_GATED) return run_mfma<256, 256, 4, 2, EPI_GATED, ELEM_FP8X8>(a, s);
      if (epi == EPI_SCATTER) return run_mfma<256, 256, 4, 2, EPI_SCATTER, ELEM_FP8X8>(a, s);
      if (epi == EPI_SCATTER_ATOMIC) return run_mfma<256, 256, 4, 2, EPI_SCATTER_ATOMIC, ELEM_FP8X8>(a, s);
      return run_mfma<256, 256, 4, 2, EPI_SCATTER_F32, ELEM_FP8X8>(a, s);
    }
    if (epi == EPI_GATED) return run_mfma<128, 512, 2, 4, EPI_GATED, ELEM_FP8X8>(a, s);
    if (epi == EPI_SCATTER) return run_mfma<128, 512, 2, 4, EPI_SCATTER, ELEM_FP8X8>(a, s);
    if (epi == EPI_SCATTER_ATOMIC) return run_mfma<128, 512, 2, 4, EPI_SCATTER_ATOMIC, ELEM_FP8X8>(a, s);
    return run_mfma<128, 512, 2, 4, EPI_SCATTER_F32, ELEM_FP8X8>(a, s);
  }
  if (epi == EPI_GATED)
    return belem == ELEM_FP8 ? run_grouped<EPI_GATED, ELEM_FP8>(a, block_m, s)
                             : run_grouped<EPI_GATED, ELEM_BF16>(a, block_m, s);
  if (epi == EPI_SCATTER_F32)
    return belem == ELEM_FP8 ? run_grouped<EPI_SCATTER_F32, ELEM_FP8>(a, block_m, s)
                             : run_grouped<EPI_SCATTER_F32, ELEM_BF16>(a, block_m, s);
  if (epi == EPI_SCATTER_ATOMIC)
    return belem == ELEM_FP8 ? run_grouped<EPI_SCATTER_ATOMIC, ELEM_FP8>(a, block_m, s)
                             : run_grouped<EPI_SCATTER_ATOMIC, ELEM_BF16>(a, block_m, s);
  return belem == ELEM_FP8 ? run_grouped<EPI_SCATTER, ELEM_FP8>(a, block_m, s)
                           : run_grouped<EPI_SCATTER, ELEM_BF16>(a, block_m, s);
}

hipError_t launch_gemm_f32(const GemmArgs& a, int epi, hipStream_t s) {
  if (a.k_splits != 1) return hipErrorInvalidValue;
  const int ncols = epi == EPI_GATED ? 32 : 64;
  const int64_t blocks = ((a.M + 63) / 64) * ((a.N + ncols - 1) / ncols);
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (epi == EPI_GATED) gemm_f32_kernel<EPI_GATED><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(a);
  else if (epi == EPI_SCATTER) gemm_f32_kernel<EPI_SCATTER><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(a);
  else gemm_f32_kernel<EPI_STORE_F32><<<dim3((unsigned)blocks), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
