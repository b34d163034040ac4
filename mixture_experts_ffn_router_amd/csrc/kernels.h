// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Routing options.  renorm: divide the selected weights by their sum.  scoring:
// softmax over all experts or a sigmoid per expert.  groups > 1: the experts form
// `groups` equal contiguous ranges and only the topk_groups ranges with the
// largest best logit are candidates.
enum RouteScoring { SCORE_SOFTMAX = 0, SCORE_SIGMOID = 1 };
struct RouteOpts {
  int renorm = 1;
  int scoring = SCORE_SOFTMAX;
  int groups = 1;
  int topk_groups = 1;
};

// logits: nparts planes of [T, E] (part_stride elements apart) summed in order;
// with more than one part, sum_out (if not NULL) receives the summed logits.
hipError_t launch_route(const float* logits, int64_t T, int E, int K, const RouteOpts& o, const float* pes,
                        float* w_out, int32_t* ids_out, int out_stride, int n_shared, hipStream_t s,
                        int nparts = 1, int64_t part_stride = 0, float* sum_out = nullptr);

// slot_row [n] is required (it also holds the per-chunk counts between the
// launches); num_padded may be NULL.  E <= 1024.
hipError_t launch_permute(const int32_t* ids, int64_t n, int E, int bm_log2, int32_t* counts,
                          int32_t* offsets, int32_t* sorted_slots, int32_t* block_expert, int32_t* num_padded,
                          int32_t* slot_row, hipStream_t s);

// Compute units of the current device (256 when it cannot be queried).
int device_cu_count();

// EPI_SCATTER_ATOMIC: fp32 atomic add of each weighted row into row c_rows[r] / row_div
// of C (the slot's token), every reduction part into the same row.
enum GemmEpi { EPI_GATED = 0, EPI_SCATTER = 1, EPI_STORE_F32 = 2, EPI_SCATTER_F32 = 3, EPI_SCATTER_ATOMIC = 4 };
// B element type; ELEM_FP8X8: A and B both FP8 (E4M3), the per-row A scale in row_scale
enum GemmElem { ELEM_F32 = 0, ELEM_BF16 = 1, ELEM_FP8 = 2, ELEM_FP8X8 = 3 };

// One grouped "NT" GEMM: C[r, n] = sum_k A[row(r), k] * B_e[n, k] for the rows r
// of every row block, e = the block's expert.
struct GemmArgs {
  const void* A;              // activation rows, [*, Kdim], row stride lda (elements)
  int64_t lda;
  const int32_t* a_rows;      // row map for A: slot index per row (token = slot / row_div), -1 = pad;
                              // NULL = identity rows
  int32_t row_div;
  int64_t M;                  // identity rows: number of valid rows; mapped rows: capacity
  int64_t a_rows_alloc;       // rows of the A allocation (a_rows_alloc * lda * 2 < 2^31)
  const int32_t* m_dev;       // device count of rows (padded total) or NULL (use M)
  const int32_t* block_expert;  // expert per row block, NULL = expert 0
  const int32_t* seg_off;       // with block_expert: padded row offset of each expert [E + 1]
  const void* B0;             // routed expert weights, expert stride bstride (elements)
  const void* B1;             // weights of experts >= n_routed (shared), same stride
  int64_t bstride;
  int32_t n_routed;
  const float* bscale0;       // FP8 per-output-channel scales, expert stride sstride
  const float* bscale1;
  int64_t sstride;
  int32_t N;                  // output columns (gated: I, reading B rows n and I + n)
  int32_t Kdim;
  void* C;                    // output; row stride ldc (elements)
  int64_t ldc;
  const int32_t* c_rows;      // scatter epilogue: output row = c_rows[r] * k_splits + part (skip if < 0)
  const float* row_weight;    // scatter epilogue: weight per output row (slot), NULL = 1
  int32_t act;                // gated epilogue activation
  const float* row_scale;     // per-token factor on the accumulator (gated: on g and u; store:
                              // on the value), indexed by the A row's token; NULL = 1
  float c_scale = 1.f;        // constant factor on stored values (store epilogue)
  int32_t k_splits = 1;       // MFMA kernel, scatter and store epilogues: the reduction is cut into
                              // this many parts, each stored to its own row (scatter: row slot*KS+part)
                              // or plane (store: C[part][row]); the gated epilogue needs 1
};

// bf16 A; B bf16 or FP8 (ELEM_BF16 / ELEM_FP8).  block_m in {32, 64, 128, 256}.
hipError_t launch_gemm_mfma(const GemmArgs& a, int epi, int belem, int block_m, hipStream_t s);
// Reduction parts for a grouped scatter GEMM of about `rows` rows: the count in
// 1..4 that wastes least of the last round of tiles on this device's CUs.
int gemm_scatter_k_splits(int64_t rows, int block_m, int N, int Kdim);
// The most parts gemm_scatter_k_splits returns for this row block and reduction
// length, whatever the rows (non-decreasing in block_m).
int gemm_scatter_k_splits_max(int block_m, int Kdim);
int gemm_store_k_splits(int64_t M, int N, int Kdim);
// fp32 A and B (the fp32 layer).  block_m = 64.
hipError_t launch_gemm_f32(const GemmArgs& a, int epi, hipStream_t s);

// inv_rms[t] = 1/sqrt(mean(x_t^2) + eps); rows are materialised only where their
// output pointer is non-NULL (router input, dense input, expert input).
hipError_t launch_prenorm(const void* x, int elem, int64_t T, int H, float eps, float* inv_rms,
                          const float* router_scale, const float* gamma_pre, const float* gamma_pre2,
                          void* r_out, void* xn1_out, void* xn2_out, hipStream_t s);

// Dynamic per-row FP8 quantisation: scale[r] = max|in[r,:]| / 448 (1 for a zero
// row), codes[r,:] = E4M3 nearest-even of in[r,:] / scale[r].  in: bf16 rows of C
// elements (C % 8 == 0, C <= 16384), row stride ld_in; rows r >= *m_dev (when
// given) are left alone, rows with row_map[r] < 0 (when given) get zero codes
// and scale 1.
hipError_t launch_quant_rows_fp8(const void* in, int64_t R, int C, int64_t ld_in, const int32_t* row_map,
                                 const int32_t* m_dev, uint8_t* codes, int64_t ld_out, float* scales,
                                 hipStream_t s);

// resid (when given, the layer input in the output type): out = resid +
// RMSNorm(out) * gamma_post_ff (ones when NULL), the FFN block's tail.
hipError_t launch_finalize(const void* ybuf, int yelem, int Kp, const float* dense_out,
                           const float* gamma_post1, const float* gamma_post2, float eps, void* out,
                           int oelem, float* out_f32, int64_t T, int H, hipStream_t s,
                           const void* resid = nullptr, const float* gamma_post_ff = nullptr);

// bytes of zeros at p (16-byte aligned, a multiple of 16)
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

hipError_t launch_gather_topk(const float* w_in, const int32_t* ids_in, int in_stride, int K, int64_t T,
                              float* w_out, int32_t* ids_out, hipStream_t s);

// Decode path (a few tokens, T <= 16): weights streamed once per call, all
// tokens applied to each weight row together.
struct DecodeArgs {
  int T, H, E, K, Kp, Ep, I, Id;
  int act, dense_act, gemma_router, dense;
  RouteOpts route;
  float eps;
  int n_router_groups;  // pre kernel: blocks computing 16 router logits each (0: logits supplied)
  int n_pre_dense_groups;  // pre kernel: trailing blocks computing 16 dense hidden units each
  int n_dense_groups;   // up kernel: leading blocks computing 16 dense hidden units each
  int n_up_blocks;      // up kernel: blocks walking the (expert, 16 hidden units) items
  int n_ddown_groups;   // down kernel: leading blocks computing 16 dense output features each
  int max_active;       // min(Ep, T * Kp): bound on the number of active experts
  const void* x;        // [T, H] bf16
  float* z;             // [T, E] logits: written by the pre kernel or supplied
  const void* w_router;
  const float* router_scale;
  const float* pes;
  const void* w13;
  const void* w2;
  const float* s13;
  const float* s2;
  const uint8_t* mx13;  // MXFP4 experts: E8M0 block scales [E, 2I, H/32] / [E, H, I/32]
  const uint8_t* mx2;
  const void* shared_w13;
  const void* shared_w2;
  const void* dense_w13;
  const void* dense_w2;
  const float* g_pre;
  const float* g_pre2;
  void* hd;             // [T, Id] bf16 dense hidden
  void* hbuf;           // [T * Kp, I] bf16 weighted expert hidden, per slot
  float* dsum;          // [T, H] dense branch output
  float* ypart;         // [T, P, H] partial expert sums when a finalize follows, else NULL
  int down_splits;      // P: parts of the reduction per output-feature group in the down kernel
  int* rinfo;           // active count, active experts [Ep], slot per (active, token) [Ep][16]
  void* out;            // [T, H] bf16 (when ypart is NULL)
  float* out_f32;
  float* topk_w_out;
  int32_t* topk_ids_out;
  // FP8 activations (FP8 expert weights, expert inputs quantised per row): the up
  // kernel stages the codes of each token's expert input (scale = max / 448)
  // widened to bf16 and stores h unweighted; launch_quant_rows_fp8 turns h into
  // hcodes / hscales; the down kernel takes the codes and applies each slot's
  // scale and routing weight to its expert's partial tile.
  int aq;
  uint8_t* xcodes;      // [T, H] x codes and [T] scales, written by the first expert block
  float* xscales;
  const uint8_t* hcodes;  // [T * Kp, I]
  const float* hscales;   // [T * Kp]
  float* slot_w;        // [T * Kp] routing weight of each slot, written by the first expert block
};

int decode_up_lds_bytes(int T, int H, int Kp, int Ep);
int decode_pre_lds_bytes(int T, int H);
int decode_up_blocks_per_cu(int T, int H, int Kp, int Ep);
int decode_down_splits(int T, int H, int I, bool dense, int Kp, int wbits);
hipError_t launch_decode_pre(const DecodeArgs& a, hipStream_t s);
// wk: expert weight kind, 0 bf16, 1 FP8 E4M3, 2 MXFP4
hipError_t launch_decode_up(const DecodeArgs& a, int wk, hipStream_t s);
hipError_t launch_decode_down(const DecodeArgs& a, int wk, hipStream_t s);

}  // namespace moe
