// Decode path of the MoE layer: a handful of tokens (T <= 16), where the layer
// is bound by streaming the weights of the experts the tokens picked ("Gemma 4
// 26B-A4B MoE walkthrough" section 7 tensor flow; llama.cpp lesson 35: only the
// selected experts' weights are read, which is what makes a token cheap, and
// decode is limited by memory bandwidth, not arithmetic).
//
// Every weight row is read once per call and applied to all tokens at once: the
// MFMA v_mfma_f32_16x16x32_bf16 takes 16 weight rows as its A operand and up to
// 16 token rows as its B operand (columns past T, or tokens that did not pick
// the expert, are zero), so each 16x16 accumulator tile is 16 output features x
// 16 tokens.  A block of 8 waves splits the reduction dimension in 8 and sums
// the partial tiles through LDS in a fixed order.
//
// Launches (a fraction of the grouped path's nine):
//   pre   router logits, 16 experts per block (skipped when logits are supplied);
//   up    first the dense MLP's gate/up with its activation (16 hidden units per
//         block; these need no routing, so their weights stream while the other
//         blocks route), then blocks that each recompute the routing of the T
//         tokens (a few hundred instructions per token), build the ascending
//         list of active experts and walk (active expert, 16 hidden units)
//         items: gate/up rows of that expert against the rows of the tokens that
//         picked it, h = act(g) * u times the slot's routing weight, stored per
//         slot in bf16.  Every block normalises the token rows it needs itself
//         while staging them into LDS;
//   down  first the dense MLP's down projection, then blocks of 16 output
//         features (times P parts of the reduction when there are few feature
//         groups): the sum over active experts of W2_e h_e, where h_e already
//         carries each token's weight, so the combine over a token's k slots
//         happens inside the accumulator;
//   finalize (dense branch or P > 1): the sum of the P partial rows in a fixed
//         order, then the two post-norms and the branch sum.
//
// Decode time is mostly chains of dependent memory round trips inside a block,
// so every wave issues all loads of its share of a weight tile in one batch,
// before it stages the token rows when the tile is known in advance, and the
// token rows are read once (into registers) while the routing is computed.
//
// Weights are addressed through buffer resources: a row past the end of the
// tensor (router rows >= E) reads as zero.  FP8 weights are widened to bf16 in
// registers (exact) and their per-output-channel scale is applied once per
// expert to the reduced tile.  MXFP4 weights (4-bit E2M1 codes, one E8M0 scale
// per 32 along the reduction; llama.cpp lesson 35: 4-bit experts for decode
// memory) are widened with their block scale by v_cvt_scalef32_pk_bf16_fp4
// (exact: a power of two times a 4-bit value), half the bytes of FP8.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "route_dev.h"

namespace moe {

// Expert weight kinds of the streaming kernels.
enum : int { WK_BF16 = 0, WK_FP8 = 1, WK_FP4 = 2 };
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Macro steps (64 reduction elements each) per load batch (measured: short
// batches with more resident waves stream bf16 weights best; fp8 prefers longer).
constexpr int DU_PRE = 6;   // router kernel: few blocks, one batch per wave
constexpr int DU_BF16 = 2;  // streaming kernels, bf16 weights
constexpr int DU_FP8 = 6;   // streaming kernels, fp8 weights
constexpr int DU_FP4 = 4;   // MXFP4 weights, whole-item streams: 2 pairs per batch, two batches in flight
constexpr int DU_FP8W = 4;  // fp8 weights, whole-item streams: the bytes of a bf16 batch
constexpr int XCH = 8;  // 16-byte chunks per lane of a token row held in registers (4096 elements)

// Lane l feeds row / token column l & 15 and reduction elements from lane group
// g = l >> 4.  Within macro step m (elements 64m .. 64m + 63) MFMA j reads the
// 8 elements starting at kchunk(m, j, g):
//   bf16 weights: 64m + 32j + 8g   (each 16-byte load is one MFMA's operand)
//   fp8 weights:  64m + 16g + 8j   (one 16-byte load holds both MFMAs' operands)
//   MXFP4:        128(m/2) + 32g + 16(m%2) + 8j
//                 (one 16-byte load holds a pair of macro steps for a lane group:
//                 32 elements, exactly one block of the block scale)
// The assignment of reduction indices to MFMA slots is arbitrary as long as A
// and B agree; these make every load contiguous.
template <int WK>
__device__ __forceinline__ int kchunk(int m, int j, int g) {
  if constexpr (WK == WK_FP4) return 128 * (m >> 1) + 32 * g + 16 * (m & 1) + 8 * j;
  return WK != WK_BF16 ? 64 * m + 16 * g + 8 * j : 64 * m + 32 * j + 8 * g;
}

// Part idx of parts of the macro steps [lo, hi).  MXFP4 ranges are whole pairs
// of steps (lo even), so a 16-byte load never straddles two ranges; an odd step
// count is rounded up to a pair, whose elements past the reduction length the
// stream zeroes (both steps of a pair hold elements below it).
template <int WK>
__device__ __forceinline__ void sub_range(int lo, int hi, int idx, int parts, int& a, int& b) {
  const int n = hi - lo;
  if constexpr (WK == WK_FP4) {
    const int np = (n + 1) / 2;
    a = lo + 2 * (idx * np / parts);
    b = lo + 2 * ((idx + 1) * np / parts);
  } else {
    a = lo + idx * n / parts;
    b = lo + (idx + 1) * n / parts;
  }
}

// Bytes of n weight elements of kind WK.
template <int WK>
__host__ __device__ constexpr int64_t wbytes(int64_t n) {
  return WK == WK_BF16 ? 2 * n : (WK == WK_FP8 ? n : n / 2);
}

// E8M0 block scale -> fp32 (2^(c - 127); c = 0 is the subnormal 2^-127)
__device__ __forceinline__ float e8m0_to_f32(uint32_t c) {
  return __uint_as_float(c ? c << 23 : 0x00400000u);
}

// 8 E2M1 codes (element i in bits 4i..4i+3) times scale s -> 8 bf16, in order
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8(uint32_t w, float s) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  const bf16x2v p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0);
  const bf16x2v p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1);
  const bf16x2v p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2);
  const bf16x2v p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3);
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, p0);
  r[1] = __builtin_bit_cast(uint32_t, p1);
  r[2] = __builtin_bit_cast(uint32_t, p2);
  r[3] = __builtin_bit_cast(uint32_t, p3);
  return __builtin_bit_cast(bf16x8, r);
}

constexpr uint32_t OOB = 0x80000000u;  // a buffer offset past every tensor here: the load returns 0

__device__ __forceinline__ u32x4 bload(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// acc[r] += A_r (16 weight rows) x B (token rows) over macro steps, in batches of DU.
//   ra/aoff: weight tensor and the byte offset of this lane's weight row;
//   BG = false: B rows in LDS (b_lds = this lane's token row, zero if !bvalid);
//   BG = true:  B rows in global memory (rb/boff; boff past the end reads zero).
//   MXFP4: rs/soff: the block-scale tensor and the byte offset of this lane's
//   row of scales (one byte per 32 elements).
//   BQ: B rows in global memory are FP8 codes (boff in bytes), widened to bf16
//   (exact); with fp8 weights one 16-byte load holds both MFMAs' B operands.
template <int WK, int NR, bool BG, int DU, bool BQ = false>
struct Stream {
  static_assert(WK != WK_FP4 || DU % 2 == 0, "MXFP4 batches hold whole pairs of steps");
  static_assert(!BQ || (BG && WK == WK_FP8), "B codes go with fp8 weights and B rows in global memory");
  static constexpr int LA = WK == WK_BF16 ? 2 : 1;  // A loads per row group per macro step
  rsrc_t ra[NR];
  uint32_t aoff[NR];
  rsrc_t rs[NR];
  uint32_t soff[NR];
  int kmax = 1 << 30;  // MXFP4: the reduction length; a pair that ends past it (K % 128 == 64)
                       // gives some lane groups elements >= kmax, which take zero A and B
  rsrc_t rb;
  uint32_t boff;
  int g;
  u32x4 av[NR][DU][LA];
  uint32_t sv[NR][(DU + 1) / 2];  // MXFP4: block scale of each pair of steps
  u32x4 bv[BG ? DU : 1][2];

  __device__ __forceinline__ void load(int m, int m1) {
#pragma unroll
    for (int u = 0; u < DU; ++u) {
      const bool live = m + u < m1;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        if constexpr (WK == WK_FP4) {
          // a pair of steps (m even: batches start on a pair): 32 codes (16 bytes),
          // one 32-element block, and its scale; the odd step reuses them
          if (u % 2 == 0) {
            const int k = kchunk<WK>(m + u, 0, g);
            av[r][u][0] = bload(ra[r], live ? aoff[r] + (uint32_t)(k / 2) : OOB);
            sv[r][u / 2] = __builtin_amdgcn_raw_buffer_load_b8(rs[r], (int)(live ? soff[r] + (uint32_t)(k / 32) : OOB), 0, 0);
          }
        } else {
#pragma unroll
          for (int j = 0; j < LA; ++j)
            av[r][u][j] = bload(ra[r], live ? aoff[r] + (uint32_t)wbytes<WK>(kchunk<WK>(m + u, j, g)) : OOB);
        }
      }
      if constexpr (BQ) {
        bv[u][0] = bload(rb, live ? boff + (uint32_t)kchunk<WK>(m + u, 0, g) : OOB);
      } else if constexpr (BG) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int k = kchunk<WK>(m + u, j, g);
          bv[u][j] = bload(rb, live && (WK != WK_FP4 || k < kmax) ? boff + (uint32_t)(k * 2) : OOB);
        }
      }
    }
  }
  // Steps past m1 run with zero weights (their loads fell outside the buffer)
  // and B re-read from step m1 - 1, so a batch is branch-free (and every load
  // of a batch is consumed, which keeps the next batch's loads from waiting
  // on registers that might still be in flight).
  __device__ __forceinline__ void compute(f32x4 (&acc)[NR], const bf16_t* b_lds, bool bvalid, int m, int m1) {
#pragma unroll
    for (int u = 0; u < DU; ++u) {
      const int mu = m + u < m1 ? m + u : m1 - 1;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bf16x8 b;
        if constexpr (BQ) {
          const u32x4 q = bv[u][0];
          b = fp8x8_to_bf16x8(j ? q[2] : q[0], j ? q[3] : q[1]);
        } else if constexpr (BG) {
          b = __builtin_bit_cast(bf16x8, bv[u][j]);
        } else {
          const int k = kchunk<WK>(mu, j, g);
          const bool kin = WK != WK_FP4 || k < kmax;
          const u32x4 raw = *(const u32x4*)(b_lds + (kin ? k : 0));
          b = __builtin_bit_cast(bf16x8, bvalid && kin ? raw : u32x4{0u, 0u, 0u, 0u});
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          bf16x8 a;
          if constexpr (WK == WK_FP4) {
            // step u of its pair: dwords 2(u % 2) + j; a step past m1 (the second of
            // a pair that straddles the end) contributes zero weights
            const u32x4 q = av[r][u & ~1][0];
            const uint32_t w = m + u < m1 && kchunk<WK>(m + u, j, g) < kmax ? q[2 * (u & 1) + j] : 0u;
            a = fp4x8_to_bf16x8(w, e8m0_to_f32(sv[r][u / 2]));
          } else if constexpr (WK == WK_FP8) {
            const u32x4 q = av[r][u][0];
            a = fp8x8_to_bf16x8(j ? q[2] : q[0], j ? q[3] : q[1]);
          } else {
            a = __builtin_bit_cast(bf16x8, av[r][u][j]);
          }
          acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[r], 0, 0, 0);
        }
      }
    }
  }
  // Macro steps [m0, m1); the first batch was already issued when first_loaded.
  __device__ __forceinline__ void run(f32x4 (&acc)[NR], const bf16_t* b_lds, bool bvalid, int m0, int m1,
                                      bool first_loaded) {
    for (int m = m0; m < m1; m += DU) {
      if (m != m0 || !first_loaded) load(m, m1);
      __builtin_amdgcn_sched_barrier(0);  // the whole batch is issued before the first MFMA waits
      compute(acc, b_lds, bvalid, m, m1);
    }
  }
};

// Split of the reduction over the NW waves of a block.
template <int NW>
__device__ __forceinline__ void wave_range(int ms, int wave, int& m0, int& m1) {
  m0 = wave * ms / NW;
  m1 = (wave + 1) * ms / NW;
}

// Partial tiles of all waves -> LDS.  Tile element (row rho, column t) sits in
// lane t + 16 (rho / 4), register rho % 4 of the 16x16 accumulator.
template <int NR>
__device__ __forceinline__ void partials_to_lds(float* red, const f32x4 (&acc)[NR], int wave, int lane) {
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[((wave * NR + r) * 4 + v) * 64 + lane] = acc[r][v];
}
template <int NW, int NR>
__device__ __forceinline__ float reduced(const float* red, int r, int rho, int t) {
  const int lane = t + 16 * (rho >> 2), v = rho & 3;
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) s += red[((w * NR + r) * 4 + v) * 64 + lane];
  return s;
}

// ---------------------------------------------------------------- token rows -> LDS
// Row pitch H + 8 elements: 16 lanes reading one 16-byte chunk of 16 different
// rows hit distinct banks.  Lane chunk c of pass p covers elements
// (p * XCH + c) * 512 + 8 lane .. + 8.
struct RowRegs {
  u32x4 q[XCH];
};

__device__ __forceinline__ void row_load(RowRegs& r, rsrc_t rx, int t, int H, int pass, int lane) {
#pragma unroll
  for (int c = 0; c < XCH; ++c) {
    const int k = (pass * XCH + c) * 512 + lane * 8;
    r.q[c] = bload(rx, k < H ? (uint32_t)((t * H + k) * 2) : OOB);
  }
}

__device__ __forceinline__ float sumsq8(u32x4 q) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(q[i] << 16), hi = __uint_as_float(q[i] & 0xFFFF0000u);
    s += lo * lo + hi * hi;
  }
  return s;
}

__device__ __forceinline__ double sumsq8_f64(u32x4 q) {
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const double lo = __uint_as_float(q[i] << 16), hi = __uint_as_float(q[i] & 0xFFFF0000u);
    s += lo * lo + hi * hi;
  }
  return s;
}

// Stage token t (one wave).  With norm, f = c / sqrt(mean(x_t^2) + eps):
//   vec given: s[t][k] = bf16(x[t][k] * f * vec[k]), fac[t] = 1
//              (a learned per-dimension weight has to be applied before the dot product);
//   otherwise: s[t] = x[t] unchanged, fac[t] = f, applied in fp32 to the dot products
//              (a norm without a weight is a per-token factor: x_t / rms_t . w = (x_t . w) / rms_t).
// Without norm the row is copied and fac[t] = 1.  r holds pass 0 when preloaded.
// quant (FP8 activations, c = 1): the row the grouped path stores is formed first
// (a normalised row in fp64 throughout, rounded to fp32 and then bf16, so that it
// is the exactly rounded value and its codes do not depend on summation order),
// then replaced by its codes at the row's scale, widened to bf16 (exact), and
// fac[t] = the scale.
__device__ void stage_token(RowRegs& r, bool preloaded, rsrc_t rx, int t, int H, bool norm, float eps, float c,
                            const float* __restrict__ vec, bf16_t* s, int pitch, float* fac, int lane,
                            bool quant = false) {
  const int npass = (H + XCH * 512 - 1) / (XCH * 512);
  bf16_t* sr = s + t * pitch;
  const bool xform = norm && (vec || quant);
  float ss = 0.f;
  double ssd = 0.0;
  for (int p = 0; p < npass; ++p) {
    if (p > 0 || !preloaded) row_load(r, rx, t, H, p, lane);
#pragma unroll
    for (int ch = 0; ch < XCH; ++ch) {
      const int k = (p * XCH + ch) * 512 + lane * 8;
      if (k < H) {
        if (norm) {
          if (quant) ssd += sumsq8_f64(r.q[ch]);
          else ss += sumsq8(r.q[ch]);
        }
        if (!xform) *(u32x4*)(sr + k) = r.q[ch];
      }
    }
  }
  float f = 1.f;
  double fd = 1.0;
  if (norm) {
    if (quant) fd = 1.0 / sqrt(wave_sum_f64(ssd) / (double)H + (double)eps);
    else f = c / sqrtf(wave_sum_f32(ss) / (float)H + eps);
  }
  if (xform) {
    for (int p = 0; p < npass; ++p) {
      if (npass > 1) row_load(r, rx, t, H, p, lane);  // one pass: the row is still in registers
#pragma unroll
      for (int ch = 0; ch < XCH; ++ch) {
        const int k = (p * XCH + ch) * 512 + lane * 8;
        if (k < H) {
          u32x4 o;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float xl = __uint_as_float(r.q[ch][i] << 16), xh = __uint_as_float(r.q[ch][i] & 0xFFFF0000u);
            float lo, hi;
            if (quant) {
              lo = (float)((double)xl * fd * (vec ? (double)vec[k + 2 * i] : 1.0));
              hi = (float)((double)xh * fd * (vec ? (double)vec[k + 2 * i + 1] : 1.0));
            } else {
              lo = xl * f * vec[k + 2 * i];
              hi = xh * f * vec[k + 2 * i + 1];
            }
            o[i] = pack_bf16x2(lo, hi);
          }
          *(u32x4*)(sr + k) = o;
        }
      }
    }
  }
  if (quant) {
    // this lane reads back exactly the chunks it wrote above
    float m = 0.f;
    for (int k = lane * 8; k < H; k += 512) {
      const u32x4 v = *(const u32x4*)(sr + k);
      m = fmaxf(m, absmax8(make_uint4(v[0], v[1], v[2], v[3])));
    }
    const float sc = scale_of(wave_max_f32(m));
    for (int k = lane * 8; k < H; k += 512) {
      const u32x4 v = *(const u32x4*)(sr + k);
      const uint2 q = codes8(make_uint4(v[0], v[1], v[2], v[3]), sc);
      *(bf16x8*)(sr + k) = fp8x8_to_bf16x8(q.x, q.y);
    }
    if (lane == 0) fac[t] = sc;
    return;
  }
  if (lane == 0) fac[t] = xform ? 1.f : f;
}

constexpr int PW = 8;                          // waves per block of the pre and up kernels
constexpr int DW3 = 8;                         // waves per block of the down kernel
constexpr int RED_FLOATS = PW * 2 * 4 * 64;    // partial tiles of up to two row groups

__host__ __device__ __forceinline__ int stage_bytes(int T, int H) { return (T * (H + 8) * 2 + 15) / 16 * 16; }
// up kernel: partial tiles, slot ids and weights, expert flags and list, active
// count, per-token factors, the slot of each (active expert, token) as int16
// (max_active x 16); then the staged rows
__host__ __device__ __forceinline__ int up_small_bytes(int Kp, int Ep, int max_active) {
  return (RED_FLOATS * 4 + (32 * Kp + 2 * Ep + 1 + 16) * 4 + max_active * 16 * 2 + 15) / 16 * 16;
}
__host__ __device__ __forceinline__ int up_max_active(int T, int Kp, int Ep) { return T * Kp < Ep ? T * Kp : Ep; }

// Dense MLP gate/up for 16 hidden units.  It needs no routing: run by the up
// kernel's leading blocks (their weights stream while the expert blocks route)
// when two blocks fit per CU, else by the pre kernel after the router blocks.
__device__ void dense_gate_up_tile(const DecodeArgs& a, uint8_t* dsm, int i0) {
  const int T = a.T, H = a.H, Id = a.Id, pitch = H + 8;
  bf16_t* sx = (bf16_t*)dsm;
  float* red = (float*)(dsm + stage_bytes(T, H));
  float* fac = red + RED_FLOATS;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, col = lane & 15;
  const rsrc_t rx = make_rsrc(a.x, (uint32_t)(T * H * 2));
  const bool bvalid = col < T;
  const bf16_t* brow = sx + (bvalid ? col : 0) * pitch;
  int m0, m1;
  wave_range<PW>(H / 64, wave, m0, m1);
  RowRegs xr;
  if (wave < T) row_load(xr, rx, wave, H, 0, lane);
  Stream<WK_BF16, 2, false, DU_BF16> st;
  st.ra[0] = st.ra[1] = make_rsrc(a.dense_w13, (uint32_t)((int64_t)2 * Id * H * 2));
  st.aoff[0] = (uint32_t)((i0 + col) * H * 2);
  st.aoff[1] = (uint32_t)((Id + i0 + col) * H * 2);
  st.g = g;
  if (m0 < m1) st.load(m0, m1);
  for (int t = wave; t < T; t += PW) stage_token(xr, t == wave, rx, t, H, true, a.eps, 1.f, a.g_pre, sx, pitch, fac, lane);
  __syncthreads();
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  st.run(acc, brow, bvalid, m0, m1, true);
  partials_to_lds<2>(red, acc, wave, lane);
  __syncthreads();
  if (threadIdx.x < 256) {
    const int rho = threadIdx.x >> 4, t = threadIdx.x & 15;
    if (t < T) {
      const float gv = reduced<PW, 2>(red, 0, rho, t) * fac[t], uv = reduced<PW, 2>(red, 1, rho, t) * fac[t];
      ((bf16_t*)a.hd)[t * Id + i0 + rho] = f32_to_bf16(apply_act_bf16(a.dense_act, gv) * uv);
    }
  }
}

// ---------------------------------------------------------------- pre: router logits (+ dense gate/up)
__global__ __launch_bounds__(PW * 64, 2) void decode_pre_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) uint8_t dsm[];
  if ((int)blockIdx.x >= a.n_router_groups) {
    dense_gate_up_tile(a, dsm, (blockIdx.x - a.n_router_groups) * 16);
    return;
  }
  const int T = a.T, H = a.H, pitch = H + 8;
  bf16_t* sx = (bf16_t*)dsm;
  float* red = (float*)(dsm + stage_bytes(T, H));
  float* fac = red + RED_FLOATS;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, col = lane & 15;
  const rsrc_t rx = make_rsrc(a.x, (uint32_t)(T * H * 2));
  const bool bvalid = col < T;
  const bf16_t* brow = sx + (bvalid ? col : 0) * pitch;
  int m0, m1;
  wave_range<PW>(H / 64, wave, m0, m1);
  RowRegs xr;
  if (wave < T) row_load(xr, rx, wave, H, 0, lane);
  const int e0 = blockIdx.x * 16;
  Stream<WK_BF16, 1, false, DU_PRE> st;
  st.ra[0] = make_rsrc(a.w_router, (uint32_t)((int64_t)a.E * H * 2));
  st.aoff[0] = (uint32_t)((e0 + col) * H * 2);  // rows >= E read zero
  st.g = g;
  if (m0 < m1) st.load(m0, m1);
  for (int t = wave; t < T; t += PW)
    stage_token(xr, t == wave, rx, t, H, a.gemma_router != 0, a.eps, a.gemma_router ? 1.0f / sqrtf((float)H) : 1.f,
                a.gemma_router ? a.router_scale : nullptr, sx, pitch, fac, lane);
  __syncthreads();
  f32x4 acc[1] = {{0.f, 0.f, 0.f, 0.f}};
  st.run(acc, brow, bvalid, m0, m1, true);
  partials_to_lds<1>(red, acc, wave, lane);
  __syncthreads();
  if (threadIdx.x < 256) {
    const int rho = threadIdx.x >> 4, t = threadIdx.x & 15;
    if (t < T && e0 + rho < a.E) a.z[t * a.E + e0 + rho] = reduced<PW, 1>(red, 0, rho, t) * fac[t];
  }
}

// ---------------------------------------------------------------- up: dense gate/up, routing + expert gate/up
// Expert gate/up (bf16, fp8 or MXFP4 weights): one wave owns whole (expert, 16
// hidden units) items, so the MFMA accumulator holds each item's complete
// 16 x 16 tiles and the epilogue needs no reduction across waves and no
// barrier.  A wave's items are one flat sequence of batches streamed through
// two register sets: the loads of batch b + 1 are in flight while batch b
// computes.
template <int WK>
__device__ __forceinline__ void up_items_per_wave(const DecodeArgs& a, const int16_t* s_slot, const float* s_w,
                                                  const int* s_active, const float* fac, const bf16_t* sx,
                                                  int pitch, int n_items, int gw, int lane) {
  constexpr int DU = WK == WK_FP4 ? DU_FP4 : (WK == WK_FP8 ? DU_FP8W : DU_BF16);
  using S = Stream<WK, 2, false, DU>;
  const int T = a.T, H = a.H, I = a.I, E = a.E, Kp = a.Kp, RG = I / 16;
  const int g = lane >> 4, col = lane & 15;
  const int nwv = a.n_up_blocks * PW;
  const int it0 = (int)((int64_t)gw * n_items / nwv), it1 = (int)((int64_t)(gw + 1) * n_items / nwv);
  int m0, m1;  // every step of a row (MXFP4: whole pairs, elements past H zeroed by kmax)
  sub_range<WK>(0, H / 64, 0, 1, m0, m1);
  const int BPI = (m1 - m0 + DU - 1) / DU;  // batches per item
  const int NB = (it1 - it0) * BPI;
  S s0, s1;
  // fp8 weights: the per-output-channel scales of each set's item (gate and up
  // rows of hidden units i0 + 4g .. + 3), loaded with every batch of the item
  f32x4 sg0 = {1.f, 1.f, 1.f, 1.f}, su0 = sg0, sg1 = sg0, su1 = sg0;
  // batch b >= NB issues loads outside every buffer (no traffic) so that the
  // loop issues the same loads on every path and each wait covers one batch
  auto issue = [&](S& st, f32x4& sg, f32x4& su, int b) {
    const bool live = b < NB;
    const int bb = live ? b : 0;
    const int item = it0 + bb / BPI;
    const int e = s_active[item / RG], i0 = (item % RG) * 16;
    if constexpr (WK == WK_FP8) {
      const float* sp = a.s13 + (live ? (int64_t)e * 2 * I + i0 + 4 * g : 0);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        sg[v] = sp[v];
        su[v] = sp[(live ? I : 0) + v];
      }
    }
    st.g = g;
    // shared experts (ids E.., bf16 layers only) follow the routed ones
    const uint8_t* wbase = e < E ? (const uint8_t*)a.w13 + wbytes<WK>((int64_t)e * 2 * I * H)
                                 : (const uint8_t*)a.shared_w13 + (int64_t)(e - E) * 2 * I * H * 2;
    st.ra[0] = st.ra[1] = make_rsrc(wbase, (uint32_t)wbytes<WK>((int64_t)2 * I * H));
    st.aoff[0] = (uint32_t)wbytes<WK>((int64_t)(i0 + col) * H);
    st.aoff[1] = (uint32_t)wbytes<WK>((int64_t)(I + i0 + col) * H);
    if constexpr (WK == WK_FP4) {
      st.kmax = H;
      st.rs[0] = st.rs[1] = make_rsrc(a.mx13 + (int64_t)e * 2 * I * (H / 32), (uint32_t)(2 * I * (H / 32)));
      st.soff[0] = (uint32_t)((i0 + col) * (H / 32));
      st.soff[1] = (uint32_t)((I + i0 + col) * (H / 32));
    }
    st.load(live ? m0 + (bb % BPI) * DU : m1, m1);
  };
  f32x4 acc[2];
  // batch b: compute; the last batch of an item runs its epilogue.  Tile element
  // (hidden unit 4g + v, token col) sits in register v of this lane.
  auto step = [&](S& st, const f32x4& sg, const f32x4& su, int b) {
    const int item = it0 + b / BPI, bi = b % BPI;
    const int i0 = (item % RG) * 16;
    const int slot = col < T ? s_slot[(item / RG) * 16 + col] : -1;
    if (bi == 0) acc[0] = acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.compute(acc, sx + (slot >= 0 ? col : 0) * pitch, slot >= 0, m0 + bi * DU, m1);
    if (bi == BPI - 1 && slot >= 0) {
      uint32_t packed[2];
      if constexpr (WK == WK_FP8) {
        // FP8 activations: h is quantised as stored, before the routing weight
        const float w = a.aq ? 1.f : s_w[slot];
#pragma unroll
        for (int v = 0; v < 4; v += 2) {
          const float h0 = apply_act_bf16(a.act, acc[0][v] * fac[col] * sg[v]) * (acc[1][v] * fac[col] * su[v]) * w;
          const float h1 =
              apply_act_bf16(a.act, acc[0][v + 1] * fac[col] * sg[v + 1]) * (acc[1][v + 1] * fac[col] * su[v + 1]) * w;
          packed[v / 2] = (uint32_t)f32_to_bf16(h0) | ((uint32_t)f32_to_bf16(h1) << 16);
        }
      } else {
#pragma unroll
        for (int v = 0; v < 4; v += 2) {
          const float h0 = apply_act_bf16(a.act, acc[0][v] * fac[col]) * (acc[1][v] * fac[col]) * s_w[slot];
          const float h1 = apply_act_bf16(a.act, acc[0][v + 1] * fac[col]) * (acc[1][v + 1] * fac[col]) * s_w[slot];
          packed[v / 2] = (uint32_t)f32_to_bf16(h0) | ((uint32_t)f32_to_bf16(h1) << 16);
        }
      }
      *(u32x2*)((bf16_t*)a.hbuf + (int64_t)slot * I + i0 + 4 * g) = u32x2{packed[0], packed[1]};
    }
  };
  // Two batches ahead: a set is reloaded right after it is consumed, so each
  // wait covers the older set only (sched_barrier keeps the order).
  if (NB > 0) {
    issue(s0, sg0, su0, 0);
    issue(s1, sg1, su1, 1);
  }
  for (int b = 0; b < NB; b += 2) {
    __builtin_amdgcn_sched_barrier(0);
    step(s0, sg0, su0, b);
    issue(s0, sg0, su0, b + 2);
    __builtin_amdgcn_sched_barrier(0);
    if (b + 1 < NB) step(s1, sg1, su1, b + 1);
    issue(s1, sg1, su1, b + 3);
  }
}

template <int VPL, int WK>
__global__ __launch_bounds__(PW * 64, 4) void decode_up_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) uint8_t dsm[];
  if ((int)blockIdx.x < a.n_dense_groups) {
    dense_gate_up_tile(a, dsm, blockIdx.x * 16);
    return;
  }
  const int blk = blockIdx.x - a.n_dense_groups;  // expert block
  const int T = a.T, H = a.H, I = a.I, E = a.E, Kp = a.Kp, Ep = a.Ep, pitch = H + 8;
  // the wave index is the same on every lane of a wave; saying so keeps the
  // streams' buffer resources and step ranges in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, g = lane >> 4, col = lane & 15;
  float* red = (float*)dsm;
  int* s_ids = (int*)(dsm + RED_FLOATS * 4);
  float* s_w = (float*)(s_ids + 16 * Kp);
  int* s_flag = (int*)(s_w + 16 * Kp);
  int* s_active = s_flag + Ep;
  int* s_nact = s_active + Ep;
  float* fac = (float*)(s_nact + 1);
  int16_t* s_slot = (int16_t*)(fac + 16);  // [max_active][16]: slot of (active expert, token), -1: none
  bf16_t* sx = (bf16_t*)(dsm + up_small_bytes(Kp, Ep, a.max_active));
  const rsrc_t rx = make_rsrc(a.x, (uint32_t)(T * H * 2));

  // 1. token rows and logits in flight together, then the routing of the T
  //    tokens (every block computes the same routing).  Up to PW / 2 tokens, wave
  //    w routes token w while wave PW / 2 + w stages its row; more tokens, wave w
  //    routes and stages tokens w and w + PW.
  const bool split = T <= PW / 2;
  const int rt0 = wave, rt1 = split ? T : wave + PW;                 // tokens this wave routes (< T)
  const int st0 = split ? wave - PW / 2 : wave, st1 = split ? T : wave + PW;  // and stages (0 <= t < T)
  RowRegs xr0, xr1;
  if (st0 >= 0 && st0 < T) row_load(xr0, rx, st0, H, 0, lane);
  if (st1 < T) row_load(xr1, rx, st1, H, 0, lane);
  TokenLogits<VPL> z0, z1;
  if (rt0 < T) z0 = load_logits<VPL>(a.z + rt0 * E, E, lane, a.pes);
  if (rt1 < T) z1 = load_logits<VPL>(a.z + rt1 * E, E, lane, a.pes);
  // one token (its Kp <= 64 slots pick distinct experts: the top-k picks, then
  // the shared ids E..): wave 0 ranks them into the ascending active list right
  // after routing, one barrier in all
  const bool one = T == 1;
  if (!one)
    for (int i = threadIdx.x; i < Ep; i += PW * 64) s_flag[i] = 0;
  for (int t = rt0; t < T && t <= rt1; t += PW) {
    float w;
    int id;
    route_logits<VPL>(t == rt0 ? z0 : z1, E, a.K, a.route, a.pes, lane, w, id);
    if (lane < a.K) {
      s_ids[t * Kp + lane] = id;
      s_w[t * Kp + lane] = w;
    } else if (lane < Kp) {
      s_ids[t * Kp + lane] = E + (lane - a.K);
      s_w[t * Kp + lane] = 1.f;
    }
  }
  if (one && wave == 0) {
    const int id = lane < Kp ? s_ids[lane] : 0x7fffffff;
    int rank = 0;
    for (int j = 0; j < Kp; ++j) rank += __shfl(id, j, 64) < id ? 1 : 0;
    if (lane < Kp) {
      s_active[rank] = id;
#pragma unroll
      for (int c = 0; c < 16; ++c) s_slot[rank * 16 + c] = (int16_t)(c == 0 ? lane : -1);
    }
    if (lane == 0) *s_nact = Kp;
  }
  // expert input rows: pre_feedforward_layernorm_2(x) with the dense branch, x otherwise
  if (st0 >= 0 && st0 < T)
    stage_token(xr0, true, rx, st0, H, a.dense != 0, a.eps, 1.f, a.dense ? a.g_pre2 : nullptr, sx, pitch, fac, lane,
                a.aq != 0);
  if (st1 < T)
    stage_token(xr1, true, rx, st1, H, a.dense != 0, a.eps, 1.f, a.dense ? a.g_pre2 : nullptr, sx, pitch, fac, lane,
                a.aq != 0);
  __syncthreads();
  if (!one) {
    for (int i = threadIdx.x; i < T * Kp; i += PW * 64) s_flag[s_ids[i]] = 1;
    __syncthreads();
    if (wave == 0) {  // ascending list of the experts with at least one slot, and each one's place in it
      int base = 0;
      for (int j = 0; j < Ep; j += 64) {
        const int e = j + lane;
        const bool f = e < Ep && s_flag[e];
        const uint64_t mask = __ballot(f);
        if (f) {
          const int u = base + __popcll(mask & ((1ull << lane) - 1ull));
          s_active[u] = e;
          s_flag[e] = u;
        }
        base += __popcll(mask);
      }
      if (lane == 0) *s_nact = base;
    }
    __syncthreads();
    const int na = *s_nact;
    // slot of each (active expert, token): one write per slot through the experts' places
    for (int i = threadIdx.x; i < na * 16; i += PW * 64) s_slot[i] = -1;
    __syncthreads();
    for (int i = threadIdx.x; i < T * Kp; i += PW * 64) s_slot[s_flag[s_ids[i]] * 16 + i / Kp] = (int16_t)i;
    __syncthreads();
  }
  const int n_act = *s_nact;

  // 2. the first expert block publishes the routing for the down kernel and the
  //    caller once its own items are issued (stores then never sit in front of
  //    the weight loads' waits)
  auto publish = [&]() {
    if (blk != 0) return;
    if (threadIdx.x == 0) a.rinfo[0] = n_act;
    for (int i = threadIdx.x; i < n_act; i += PW * 64) a.rinfo[1 + i] = s_active[i];
    for (int i = threadIdx.x; i < n_act * 16; i += PW * 64) a.rinfo[1 + Ep + i] = s_slot[i];
    for (int i = threadIdx.x; i < T * a.K; i += PW * 64) {
      const int t = i / a.K, k = i % a.K;
      if (a.topk_w_out) a.topk_w_out[i] = s_w[t * Kp + k];
      if (a.topk_ids_out) a.topk_ids_out[i] = s_ids[t * Kp + k];
    }
    if (a.aq) {
      for (int i = threadIdx.x; i < T * Kp; i += PW * 64) a.slot_w[i] = s_w[i];
      for (int i = threadIdx.x; i < T; i += PW * 64) a.xscales[i] = fac[i];
      // the staged codes (bf16 values of E4M3 codes, so re-encoding them is exact)
      for (int i = threadIdx.x; i < T * (H / 8); i += PW * 64) {
        const int t = i / (H / 8), k = (i % (H / 8)) * 8;
        const u32x4 v = *(const u32x4*)(sx + t * pitch + k);
        const uint2 q = codes8(make_uint4(v[0], v[1], v[2], v[3]), 1.f);
        *(uint2*)(a.xcodes + (int64_t)t * H + k) = q;
      }
    }
  };

  // 3. (active expert, 16 hidden units) items: a contiguous, balanced range per block
  const int RG = I / 16, n_items = n_act * RG;
  const int it0 = (int)((int64_t)blk * n_items / a.n_up_blocks);
  const int it1 = (int)((int64_t)(blk + 1) * n_items / a.n_up_blocks);
  int m0, m1;
  sub_range<WK>(0, H / 64, wave, PW, m0, m1);
  // Whole items per wave when items are plentiful (every block sees the same
  // n_items): at least one per wave for bf16 and fp8 weights, one per two waves
  // for MXFP4, whose items carry a quarter of the bytes, so that a block-wide
  // reduction per item costs more than the item's stream
  if ((WK == WK_FP4 ? 2 : 1) * n_items >= a.n_up_blocks * PW) {
    up_items_per_wave<WK>(a, s_slot, s_w, s_active, fac, sx, pitch, n_items, blk * PW + wave, lane);
    publish();
    return;
  }
  for (int item = it0; item < it1; ++item) {
    const int u = item / RG, i0 = (item % RG) * 16;
    const int e = s_active[u];
    float sg = 1.f, su = 1.f;  // fp8 per-output-channel scales of the epilogue's row, loaded early
    if constexpr (WK == WK_FP8) {
      if (threadIdx.x < 256) {
        sg = a.s13[(int64_t)e * 2 * I + i0 + (threadIdx.x >> 4)];
        su = a.s13[(int64_t)e * 2 * I + I + i0 + (threadIdx.x >> 4)];
      }
    }
    const int slot_col = col < T ? s_slot[u * 16 + col] : -1;
    const bool bvalid = slot_col >= 0;
    const bf16_t* brow = sx + (bvalid ? col : 0) * pitch;
    const uint8_t* wbase = e < E ? (const uint8_t*)a.w13 + wbytes<WK>((int64_t)e * 2 * I * H)
                                 : (const uint8_t*)a.shared_w13 + (int64_t)(e - E) * 2 * I * H * 2;
    Stream<WK, 2, false, WK == WK_BF16 ? DU_BF16 : DU_FP8> st;
    st.ra[0] = st.ra[1] = make_rsrc(wbase, (uint32_t)wbytes<WK>((int64_t)2 * I * H));
    st.aoff[0] = (uint32_t)wbytes<WK>((int64_t)(i0 + col) * H);
    st.aoff[1] = (uint32_t)wbytes<WK>((int64_t)(I + i0 + col) * H);
    if constexpr (WK == WK_FP4) {  // E8M0 scales [E, 2I, H/32]
      st.kmax = H;
      st.rs[0] = st.rs[1] = make_rsrc(a.mx13 + (int64_t)e * 2 * I * (H / 32), (uint32_t)(2 * I * (H / 32)));
      st.soff[0] = (uint32_t)((i0 + col) * (H / 32));
      st.soff[1] = (uint32_t)((I + i0 + col) * (H / 32));
    }
    st.g = g;
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    st.run(acc, brow, bvalid, m0, m1, false);
    partials_to_lds<2>(red, acc, wave, lane);
    __syncthreads();
    if (threadIdx.x < 256) {
      const int rho = threadIdx.x >> 4, t = threadIdx.x & 15;
      const int slot = t < T ? s_slot[u * 16 + t] : -1;
      if (slot >= 0) {
        const float gv = reduced<PW, 2>(red, 0, rho, t) * fac[t] * sg;
        const float uv = reduced<PW, 2>(red, 1, rho, t) * fac[t] * su;
        // FP8 activations: h is quantised as stored, before the routing weight
        const float h = apply_act_bf16(a.act, gv) * uv * (a.aq ? 1.f : s_w[slot]);
        ((bf16_t*)a.hbuf)[(int64_t)slot * I + i0 + rho] = f32_to_bf16(h);
      }
    }
    __syncthreads();  // red is rewritten by the next item
  }
  publish();
}

// Expert down projection (bf16, fp8 or MXFP4 weights) of one (16 output features,
// part) block: this wave's units (active expert u, split s) for unit = wave,
// wave + DW3, ... as one flat sequence of batches through two register sets
// (the next batch in flight while the current one computes), all summed into
// one 16 x 16 accumulator (the routing weight is already in h').  The routing
// summary is staged in LDS first: max_active entries, read without waiting for
// the active count (entries past it are in bounds and unused), so the first
// weight loads wait for one round trip and one barrier.
constexpr int MAX_ACTIVE_DOWN = 520;  // E <= 512 routed + 8 shared experts
// fp8 weights: each unit's tile is summed in an accumulator of its own, then
// scaled by its expert's channel scales (and, BQ: B are the slots' h codes, by
// the slot's h scale times routing weight) and added.
// s_e [MAX_ACTIVE_DOWN], s_slot [MAX_ACTIVE_DOWN * 16]: the kernel's LDS table.
template <int WK, bool BQ>
__device__ __forceinline__ f32x4 down_units(const DecodeArgs& a, int n_act, int S, int k0, int k1, int n0,
                                            int wave, int lane, int* s_e, int* s_slot) {
  static_assert(!BQ || WK == WK_FP8, "h codes go with fp8 weights");
  // fp8 weights with bf16 h rows: two steps per batch (their B loads take twice
  // the registers of the codes' loads), which keeps two blocks per CU
  constexpr int DU = WK == WK_FP4 ? DU_FP4 : (WK == WK_FP8 ? (BQ ? DU_FP8W : 2) : DU_BF16);
  using St = Stream<WK, 1, true, DU, BQ>;
  const int H = a.H, I = a.I, E = a.E, Ep = a.Ep, g = lane >> 4, col = lane & 15;
  const int MA = a.max_active;
  {  // four loads in flight per thread before their stores (one round trip up to 2048 slots)
    constexpr int NT = DW3 * 64;
    for (int i = threadIdx.x; i < MA; i += NT) s_e[i] = a.rinfo[1 + i];
    for (int base = 0; base < MA * 16; base += 4 * NT) {
      int v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = base + threadIdx.x + j * NT;
        v[j] = i < MA * 16 ? a.rinfo[1 + Ep + i] : 0;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = base + threadIdx.x + j * NT;
        if (i < MA * 16) s_slot[i] = v[j];
      }
    }
  }
  __syncthreads();
  const int n_units = n_act * S;
  const int NJ = n_units > wave ? (n_units - wave + DW3 - 1) / DW3 : 0;  // this wave's units
  // steps per unit, at most (MXFP4: whole pairs)
  const int spu = WK == WK_FP4 ? 2 * (((k1 - k0 + 1) / 2 + S - 1) / S) : (k1 - k0 + S - 1) / S;
  const int BPU = (spu + DU - 1) / DU;  // batches per unit, at most
  const int NB = NJ * BPU;
  const rsrc_t rb = BQ ? make_rsrc(a.hcodes, (uint32_t)((int64_t)a.T * a.Kp * I))
                      : make_rsrc(a.hbuf, (uint32_t)((int64_t)a.T * a.Kp * I * 2));
  St s0, s1;
  int m_0 = 0, e_0 = 0, m_1 = 0, e_1 = 0;  // each set's first step and end step
  f32x4 sc0 = {1.f, 1.f, 1.f, 1.f}, sc1 = sc0;  // fp8: each set's unit's channel scales (rows n0 + 4g ..)
  float cf0 = 1.f, cf1 = 1.f;                   // BQ: each set's unit's slot h scale x routing weight
  // batch b >= NB (and steps past a unit's range) load outside every buffer, so
  // the same loads are issued and consumed on every path
  auto issue = [&](St& st, int& mb, int& me, f32x4& sc, float& cf, int b) {
    const bool live = b < NB;
    const int bb = live ? b : 0;
    const int unit = wave + DW3 * (bb / BPU), bi = bb % BPU;
    const int u = unit / S, sp = unit % S;
    const int e = __builtin_amdgcn_readfirstlane(s_e[u]), slot = s_slot[u * 16 + col];
    int r0, r1;
    sub_range<WK>(k0, k1, sp, S, r0, r1);
    me = r1;
    mb = live ? min(r0 + bi * DU, r1) : r1;
    st.g = g;
    // shared experts (ids E.., bf16 layers only) follow the routed ones
    const uint8_t* wbase = e < E ? (const uint8_t*)a.w2 + wbytes<WK>((int64_t)e * H * I)
                                 : (const uint8_t*)a.shared_w2 + (int64_t)(e - E) * H * I * 2;
    st.ra[0] = make_rsrc(wbase, (uint32_t)wbytes<WK>((int64_t)H * I));
    st.aoff[0] = (uint32_t)wbytes<WK>((int64_t)(n0 + col) * I);
    if constexpr (WK == WK_FP4) {
      st.kmax = I;
      st.rs[0] = make_rsrc(a.mx2 + (int64_t)e * H * (I / 32), (uint32_t)(H * (I / 32)));
      st.soff[0] = (uint32_t)((n0 + col) * (I / 32));
    }
    st.rb = rb;
    st.boff = slot >= 0 ? (uint32_t)((int64_t)slot * I * (BQ ? 1 : 2)) : OOB;
    if constexpr (WK == WK_FP8) {
      const float* sp = a.s2 + (live ? (int64_t)e * H + n0 + 4 * g : 0);
#pragma unroll
      for (int v = 0; v < 4; ++v) sc[v] = sp[v];
      if constexpr (BQ) cf = (live && slot >= 0) ? a.hscales[slot] * a.slot_w[slot] : 0.f;
    }
    st.load(mb, me);
  };
  f32x4 acc[1] = {{0.f, 0.f, 0.f, 0.f}}, uacc[1] = {{0.f, 0.f, 0.f, 0.f}};
  auto comp = [&](St& st, int mb, int me, const f32x4& sc, float cf, int b) {
    if constexpr (WK == WK_FP8) {
      const int bi = b % BPU;
      if (bi == 0) uacc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
      st.compute(uacc, nullptr, false, mb, me);
      if (bi == BPU - 1) {
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[0][v] += sc[v] * uacc[0][v] * cf;
      }
    } else {
      st.compute(acc, nullptr, false, mb, me);
    }
  };
  // sched_barrier: each batch's loads are issued before the other set's MFMAs
  if (NB > 0) issue(s0, m_0, e_0, sc0, cf0, 0);
  for (int b = 0; b < NB; b += 2) {
    issue(s1, m_1, e_1, sc1, cf1, b + 1);
    __builtin_amdgcn_sched_barrier(0);
    comp(s0, m_0, e_0, sc0, cf0, b);
    if (b + 1 >= NB) break;
    issue(s0, m_0, e_0, sc0, cf0, b + 2);
    __builtin_amdgcn_sched_barrier(0);
    comp(s1, m_1, e_1, sc1, cf1, b + 1);
  }
  return acc[0];
}

// Splits per expert of the staged down stream, searched from s_min up (one
// candidate per lane, so s_min .. s_min + 63): the split whose busiest wave
// (units dealt round-robin over DW3 waves) has the fewest batches of DU steps,
// ties to the fewer units.  The same in every wave of every block.
template <int WK>
__device__ __forceinline__ int staged_splits(int n_act, int MS, int s_min, int DU, int lane) {
  const int steps = WK == WK_FP4 ? (MS + 1) / 2 : MS;  // MXFP4: pairs of steps
  const int S = s_min + lane;
  uint32_t key = 0xFFFFFFFFu;
  if (S <= steps) {
    const int spu = WK == WK_FP4 ? 2 * ((steps + S - 1) / S) : (steps + S - 1) / S;
    const int cost = (n_act * S + DW3 - 1) / DW3 * ((spu + DU - 1) / DU);
    key = (uint32_t)cost << 6 | (uint32_t)lane;
  }
  return s_min + (int)(wave_min_u32(key) & 63u);
}

// ---------------------------------------------------------------- down: dense down, expert down + combine
template <int WK>
__global__ __launch_bounds__(DW3 * 64, 4) void decode_down_kernel(DecodeArgs a) {
  __shared__ float red[DW3 * 4 * 64];
  __shared__ int s_e[MAX_ACTIVE_DOWN];          // staged routing summary (down_units)
  __shared__ int s_slot[MAX_ACTIVE_DOWN * 16];
  const int T = a.T, H = a.H, I = a.I, E = a.E, Ep = a.Ep;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, g = lane >> 4, col = lane & 15;

  if ((int)blockIdx.x < a.n_ddown_groups) {
    // dense MLP down projection: 16 output features x T tokens, fp32 out
    const int Id = a.Id, n0 = blockIdx.x * 16;
    Stream<WK_BF16, 1, true, DU_BF16> st;
    st.ra[0] = make_rsrc(a.dense_w2, (uint32_t)((int64_t)H * Id * 2));
    st.aoff[0] = (uint32_t)((n0 + col) * Id * 2);
    st.rb = make_rsrc(a.hd, (uint32_t)(T * Id * 2));
    st.boff = col < T ? (uint32_t)(col * Id * 2) : OOB;
    st.g = g;
    int m0, m1;
    wave_range<DW3>(Id / 64, wave, m0, m1);
    f32x4 acc[1] = {{0.f, 0.f, 0.f, 0.f}};
    st.run(acc, nullptr, false, m0, m1, false);
    partials_to_lds<1>(red, acc, wave, lane);
    __syncthreads();
    if (threadIdx.x < 256) {
      const int rho = threadIdx.x >> 4, t = threadIdx.x & 15;
      if (t < T) a.dsum[t * H + n0 + rho] = reduced<DW3, 1>(red, 0, rho, t);
    }
    return;
  }

  // Block = (16 output features, part): the part takes 1/P of every expert's
  // reduction range, so P blocks share a feature group when there are few groups.
  const int ng = H / 16, gi = blockIdx.x - a.n_ddown_groups;
  const int n0 = (gi % ng) * 16, part = gi / ng, P = a.down_splits;
  // The routing summary of the up kernel; this wave's entries are read in the
  // same round trip as the active count, assuming one unit per active expert
  // (re-read otherwise).  Entries at or past the count are stale but in bounds.
  const int us = wave < a.max_active ? wave : 0;
  const int n_act = a.rinfo[0];
  int e_spec = a.rinfo[1 + us];
  int slot_spec = a.rinfo[1 + Ep + us * 16 + col];
  int k0, k1;  // this part's macro steps
  sub_range<WK>(0, I / 64, part, P, k0, k1);
  const int MS = k1 - k0;
  // further splits per expert over the waves: at least enough units for every wave
  int S = max(1, min((DW3 + n_act - 1) / n_act, WK == WK_FP4 ? (MS + 1) / 2 : MS));
  // More units than waves take the staged stream, whose units are dealt to the
  // waves in turn: there the split is chosen to give the busiest wave the fewest
  // batches (9 experts as 9 units on 8 waves: 2 whole units on one wave)
  if (n_act * S > DW3)
    S = staged_splits<WK>(n_act, MS, S, WK == WK_FP4 ? DU_FP4 : (WK == WK_FP8 ? (a.aq ? DU_FP8W : 2) : DU_BF16), lane);
  const int n_units = n_act * S;
  const rsrc_t rb = make_rsrc(a.hbuf, (uint32_t)((int64_t)T * a.Kp * I * 2));
  f32x4 tot = {0.f, 0.f, 0.f, 0.f};
  // more units than waves: staged routing summary and a two-deep stream over
  // each wave's units (n_units is the same in every wave)
  const bool staged = n_units > DW3;
  if (staged) {
    if (WK == WK_FP8 && a.aq) tot = down_units<WK, WK == WK_FP8>(a, n_act, S, k0, k1, n0, wave, lane, s_e, s_slot);
    else tot = down_units<WK, false>(a, n_act, S, k0, k1, n0, wave, lane, s_e, s_slot);
  }
  for (int unit = wave; !staged && unit < n_units; unit += DW3) {
    const int u = unit / S, s = unit % S;
    const bool spec = u == us && unit == wave;
    const int e = spec ? e_spec : a.rinfo[1 + u];
    const int slot = spec ? slot_spec : a.rinfo[1 + Ep + u * 16 + col];
    const uint8_t* wbase = e < E ? (const uint8_t*)a.w2 + wbytes<WK>((int64_t)e * H * I)
                                 : (const uint8_t*)a.shared_w2 + (int64_t)(e - E) * H * I * 2;
    auto prep = [&](auto& st, rsrc_t rbx, uint32_t bo) {
      st.ra[0] = make_rsrc(wbase, (uint32_t)wbytes<WK>((int64_t)H * I));
      st.aoff[0] = (uint32_t)wbytes<WK>((int64_t)(n0 + col) * I);
      if constexpr (WK == WK_FP4) {  // E8M0 scales [E, H, I/32]
        st.kmax = I;
        st.rs[0] = make_rsrc(a.mx2 + (int64_t)e * H * (I / 32), (uint32_t)(H * (I / 32)));
        st.soff[0] = (uint32_t)((n0 + col) * (I / 32));
      }
      st.rb = rbx;
      st.boff = bo;
      st.g = g;
    };
    f32x4 sc = {1.f, 1.f, 1.f, 1.f};  // fp8 per-output-channel scales of this lane's rows, loaded early
    float cf = 1.f;                    // FP8 activations: this lane's slot's h scale times its routing weight
    if constexpr (WK == WK_FP8) {
#pragma unroll
      for (int v = 0; v < 4; ++v) sc[v] = a.s2[(int64_t)e * H + n0 + 4 * g + v];
      if (a.aq) cf = slot >= 0 ? a.hscales[slot] * a.slot_w[slot] : 0.f;
    }
    f32x4 acc[1] = {{0.f, 0.f, 0.f, 0.f}};
    int s0, s1;
    sub_range<WK>(k0, k1, s, S, s0, s1);
    if (WK == WK_FP8 && a.aq) {
      // B: the slot's h codes (the h scale is in cf)
      Stream<WK, 1, true, DU_FP8, WK == WK_FP8> st;
      prep(st, make_rsrc(a.hcodes, (uint32_t)((int64_t)T * a.Kp * I)), slot >= 0 ? (uint32_t)((int64_t)slot * I) : OOB);
      st.run(acc, nullptr, false, s0, s1, false);
    } else {
      Stream<WK, 1, true, WK == WK_BF16 ? DU_BF16 : DU_FP8> st;
      prep(st, rb, slot >= 0 ? (uint32_t)((int64_t)slot * I * 2) : OOB);
      st.run(acc, nullptr, false, s0, s1, false);
    }
    if constexpr (WK == WK_FP8) {
#pragma unroll
      for (int v = 0; v < 4; ++v) tot[v] += sc[v] * acc[0][v] * cf;
    } else {
      tot += acc[0];
    }
  }
  const f32x4 tile[1] = {tot};
  partials_to_lds<1>(red, tile, wave, lane);
  __syncthreads();
  if (threadIdx.x < 256) {
    const int rho = threadIdx.x >> 4, t = threadIdx.x & 15;
    if (t < T) {
      const float v = reduced<DW3, 1>(red, 0, rho, t);
      if (a.ypart) {
        a.ypart[((int64_t)t * P + part) * H + n0 + rho] = v;
      } else {
        const int64_t o = (int64_t)t * H + n0 + rho;
        ((bf16_t*)a.out)[o] = f32_to_bf16(v);
        if (a.out_f32) a.out_f32[o] = v;
      }
    }
  }
}

// ---------------------------------------------------------------- launches
int decode_up_lds_bytes(int T, int H, int Kp, int Ep) {
  // expert blocks; the dense gate/up blocks need stage_bytes + (RED_FLOATS + 16) * 4, which is less
  return up_small_bytes(Kp, Ep, up_max_active(T, Kp, Ep)) + stage_bytes(T, H);
}
int decode_pre_lds_bytes(int T, int H) { return stage_bytes(T, H) + (RED_FLOATS + 16) * 4; }

template <typename F>
static hipError_t allow_lds(F* f, int bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute((const void*)f, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

hipError_t launch_decode_pre(const DecodeArgs& a, hipStream_t s) {
  const int nb = a.n_router_groups + a.n_pre_dense_groups;
  if (nb == 0) return hipSuccess;
  const int lds = decode_pre_lds_bytes(a.T, a.H);
  hipError_t e = allow_lds(decode_pre_kernel, lds);
  if (e != hipSuccess) return e;
  decode_pre_kernel<<<dim3(nb), dim3(PW * 64), lds, s>>>(a);
  return hipGetLastError();
}

template <int VPL, int WK>
static hipError_t up_vpl(const DecodeArgs& a, int nb, int lds, hipStream_t s) {
  hipError_t e = allow_lds(decode_up_kernel<VPL, WK>, lds);
  if (e != hipSuccess) return e;
  decode_up_kernel<VPL, WK><<<dim3(nb), dim3(PW * 64), lds, s>>>(a);
  return hipGetLastError();
}

int decode_up_blocks_per_cu(int T, int H, int Kp, int Ep) {
  return decode_up_lds_bytes(T, H, Kp, Ep) * 2 <= 160 * 1024 ? 2 : 1;
}

// a.n_up_blocks holds the number of (expert, 16 hidden units) items on entry;
// the expert blocks walk them, sized so that they and the dense blocks are
// resident together.
hipError_t launch_decode_up(const DecodeArgs& args, int wk, hipStream_t s) {
  DecodeArgs a = args;
  const int lds = decode_up_lds_bytes(a.T, a.H, a.Kp, a.Ep);
  const int slots = device_cu_count() * decode_up_blocks_per_cu(a.T, a.H, a.Kp, a.Ep);
  const int room = slots - a.n_dense_groups > slots / 2 ? slots - a.n_dense_groups : slots / 2;
  // as few blocks as keep the item count per block at its minimum, so that every
  // block gets the same number of items when all experts the bound allows are active
  const int per_block = (a.n_up_blocks + room - 1) / room;
  a.n_up_blocks = (a.n_up_blocks + per_block - 1) / per_block;
  const int nb = a.n_dense_groups + a.n_up_blocks;
  const int vpl = a.E <= 64 ? 1 : a.E <= 128 ? 2 : a.E <= 256 ? 4 : 8;
  auto go = [&](auto wk_tag) -> hipError_t {
    constexpr int WK = decltype(wk_tag)::value;
    switch (vpl) {
      case 1: return up_vpl<1, WK>(a, nb, lds, s);
      case 2: return up_vpl<2, WK>(a, nb, lds, s);
      case 4: return up_vpl<4, WK>(a, nb, lds, s);
      default: return up_vpl<8, WK>(a, nb, lds, s);
    }
  };
  if (wk == WK_FP8) return go(std::integral_constant<int, WK_FP8>{});
  if (wk == WK_FP4) return go(std::integral_constant<int, WK_FP4>{});
  return go(std::integral_constant<int, WK_BF16>{});
}

// Parts per output-feature group of the down kernel: enough blocks for about two
// per CU, when a finalize runs anyway (dense branch), when the call has 4+ tokens,
// or when the feature groups leave CUs idle while each streams a long range
// (at most T * Kp experts' 16 rows of I weights of wbits bits: 256 KB or more);
// a finalize launch then costs less than the idle CUs.  At most one part per
// 64-deep step of the reduction.
int decode_down_splits(int T, int H, int I, bool dense, int Kp, int wbits) {
  const int ng = H / 16;
  if (!dense && T < 4) {
    const int64_t block_bytes = (int64_t)T * Kp * 16 * I * wbits / 8;
    if (ng >= device_cu_count() || block_bytes < (256 << 10)) return 1;
  }
  int P = (2 * device_cu_count() + ng - 1) / ng;
  P = P < 1 ? 1 : (P > 4 ? 4 : P);
  return P < I / 64 ? P : I / 64;
}

hipError_t launch_decode_down(const DecodeArgs& a, int wk, hipStream_t s) {
  if (a.down_splits < 1 || (a.down_splits > 1 && !a.ypart)) return hipErrorInvalidValue;
  const dim3 grid(a.n_ddown_groups + a.H / 16 * a.down_splits), block(DW3 * 64);
  if (wk == WK_FP8) decode_down_kernel<WK_FP8><<<grid, block, 0, s>>>(a);
  else if (wk == WK_FP4) decode_down_kernel<WK_FP4><<<grid, block, 0, s>>>(a);
  else decode_down_kernel<WK_BF16><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
