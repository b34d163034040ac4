// C ABI of the MoE FFN layer forward: host-side validation, workspace
// planning and the launch sequence.  Every argument is checked before the
// first launch; errors come back as status codes with a message in
// moe_last_error(), never as a silent skip or an abort.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cmath>
#include <cstring>
#include <algorithm>
#include <mutex>

#include "../../include/moe.h"
#include "kernels.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

moe_status hip_fail(hipError_t e, const char* what) {
  return fail(MOE_HIP_ERROR, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(call, what)                      \
  do {                                           \
    hipError_t _e = (call);                      \
    if (_e != hipSuccess) return hip_fail(_e, what); \
  } while (0)

// A second stream per caller stream, host thread and device, created on first
// use and kept until the process ends: the dense MLP branch of a layer runs on
// it, between a fork event recorded on the caller's stream after the input norms
// and a join event the caller's stream waits for before the finalize, so it fills
// the CUs that routing, permutation and the tails of the grouped GEMMs leave
// idle.  Default priority, non-blocking, ordered only by those events.  Keyed by
// the caller's stream so that layers forwarded on different streams never meet
// on a shared side stream; past SIDE_MAX caller streams on a thread the dense
// branch runs on the caller's stream itself.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int SIDE_MAX = 16;
SideStream* side_stream(hipStream_t caller) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  struct Entry {
    int dev;
    hipStream_t caller;
    bool ok;
    SideStream side;
  };
  thread_local Entry table[SIDE_MAX];
  thread_local int used = 0;
  for (int i = 0; i < used; ++i)
    if (table[i].dev == dev && table[i].caller == caller) return table[i].ok ? &table[i].side : nullptr;
  if (used == SIDE_MAX) return nullptr;
  Entry& x = table[used++];
  x.dev = dev;
  x.caller = caller;
  x.ok = hipStreamCreateWithFlags(&x.side.s, hipStreamNonBlocking) == hipSuccess &&
         hipEventCreateWithFlags(&x.side.fork, hipEventDisableTiming) == hipSuccess &&
         hipEventCreateWithFlags(&x.side.join, hipEventDisableTiming) == hipSuccess;
  return x.ok ? &x.side : nullptr;
}

// Once the dense branch is forked, every way out of the call (errors included)
// makes the caller's stream wait for the side stream, so no work of this call
// outlives it on the side stream (or stays unjoined in a stream capture).
struct SideJoin {
  SideStream* side = nullptr;
  hipStream_t st = nullptr;
  bool armed = false;
  hipError_t join() {
    if (!armed) return hipSuccess;
    armed = false;
    hipError_t e = hipEventRecord(side->join, side->s);
    hipError_t w = hipStreamWaitEvent(st, side->join, 0);
    return e != hipSuccess ? e : w;
  }
  ~SideJoin() { join(); }
};

constexpr size_t ALIGN = 256;
size_t align_up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

int log2_exact(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return (1 << l) == v ? l : -1;
}

int64_t permute_capacity(int64_t n_slots, int E, int bm) {
  return (n_slots + (int64_t)E * (bm - 1)) / bm * bm;
}

// Row-block height of the grouped GEMMs.  Every expert's rows are padded to a
// whole block, so the height follows the rows an expert gets on average: 256
// (256x256 tiles) from 384 rows, 128 (128x512 tiles, the same per-wave shape)
// from 128, else 64; 64 for the fp32 layer.  Measured: per real row the
// 256x256 tiles run about 1.2x faster (their B tiles are half the size and
// fit three LDS stages), which outweighs their extra padding from about 256
// rows per expert when routing is even, but not when a skewed routing leaves
// many experts a few rows each (each then pads a whole block); the host cannot
// see the skew, hence 384.
int choose_block_m(const moe_layer_desc& d, int64_t T) {
  if (d.act_dtype == MOE_DT_F32) return 64;
  const int64_t avg = T * d.top_k / d.num_experts;
  if (d.act_quant) return avg >= 384 ? 256 : 128;  // FP8 activations: 8-wave tiles only
  return avg >= 384 ? 256 : (avg >= 128 ? 128 : 64);
}

// Decode path: at most 16 bf16 tokens (one MFMA tile of token columns) whose
// rows fit the decode kernels' LDS staging (FP8 activations included: FP8
// weights, which have no shared experts).
bool use_decode(const moe_layer_desc& d, int64_t T) {
  if (d.act_dtype != MOE_DT_BF16 || T < 1 || T > 16) return false;
  const int lds_max = 160 * 1024;
  return moe::decode_up_lds_bytes((int)T, d.hidden, d.top_k + d.n_shared, d.num_experts + d.n_shared) <= lds_max &&
         moe::decode_pre_lds_bytes((int)T, d.hidden) <= lds_max;
}

struct Plan {
  bool f32, decode;
  int Kp, Ep, bm;
  int ks;    // reduction parts of the grouped down GEMM (per-slot rows per slot)
  int ks_r;  // reduction parts of the router GEMM (partial logit planes, summed by the route kernel)
  int64_t cap;
  bool need_logits, need_prenorm, gemma_router, dense;
  bool mat_r, mat_xn1, mat_xn2;  // normalised rows that must be materialised (learned weight present)
  bool y_f32;                    // per-slot expert outputs kept in fp32
  bool atomic;                   // atomic combine: y is one fp32 row per token
  bool aq;                       // FP8 activations: x and h quantised per row
  size_t o_xq, o_xs, o_hq, o_hs;  // their codes and scales
  size_t o_slotrow;  // inverse map of the permutation (slot -> padded row)
  size_t o_logits, o_w, o_ids, o_counts, o_offsets, o_sorted, o_bexp, o_rms, o_r, o_xn1, o_xn2, o_h, o_y,
      o_dh, o_dout, total;
  size_t o_rinfo, o_ypart, o_slotw;  // decode path only (o_slotw: FP8 activations)
  size_t path_total;        // bytes the path this call takes lays out (total: the larger of the two)
  int down_splits;
};

// Routing options of a layer or a moe_route call, checked and filled in.
moe_status route_opts(int32_t E, int32_t K, int32_t renorm, int32_t scoring, int32_t n_groups,
                      int32_t topk_groups, moe::RouteOpts& o) {
  if (scoring != MOE_SCORE_SOFTMAX && scoring != MOE_SCORE_SIGMOID)
    return fail(MOE_INVALID_ARG, "unknown scoring %d", scoring);
  if (n_groups < 0) return fail(MOE_INVALID_ARG, "n_groups %d < 0", n_groups);
  if (n_groups > 64) return fail(MOE_UNSUPPORTED, "n_groups %d > 64", n_groups);
  if (n_groups > 1) {
    if (E % n_groups) return fail(MOE_INVALID_ARG, "n_groups %d does not divide num_experts %d", n_groups, E);
    if (topk_groups < 1 || topk_groups > n_groups)
      return fail(MOE_INVALID_ARG, "topk_groups %d outside [1, n_groups = %d]", topk_groups, n_groups);
    if ((int64_t)topk_groups * (E / n_groups) < K)
      return fail(MOE_INVALID_ARG, "top_k %d exceeds the %d experts of the picked groups", K,
                  topk_groups * (E / n_groups));
  }
  o.renorm = renorm != 0;
  o.scoring = scoring;
  o.groups = n_groups > 1 ? n_groups : 1;
  o.topk_groups = n_groups > 1 ? topk_groups : 1;
  return MOE_OK;
}

moe_status validate_desc(const moe_layer_desc* d) {
  if (!d) return fail(MOE_INVALID_ARG, "desc is NULL");
  if (d->hidden <= 0 || d->num_experts <= 0 || d->top_k <= 0 || d->inter <= 0)
    return fail(MOE_INVALID_ARG, "hidden, num_experts, top_k and inter must be positive");
  if (d->num_experts > 512) return fail(MOE_UNSUPPORTED, "num_experts %d > 512", d->num_experts);
  if (d->top_k > d->num_experts) return fail(MOE_INVALID_ARG, "top_k %d > num_experts %d", d->top_k, d->num_experts);
  if (d->n_shared < 0 || d->n_shared > 8) return fail(MOE_INVALID_ARG, "n_shared %d outside [0, 8]", d->n_shared);
  if (d->top_k + d->n_shared > 64) return fail(MOE_UNSUPPORTED, "top_k + n_shared > 64");
  if (d->hidden % 64 || d->inter % 64)
    return fail(MOE_UNSUPPORTED, "hidden (%d) and inter (%d) must be multiples of 64", d->hidden, d->inter);
  if (d->hidden > 8192) return fail(MOE_UNSUPPORTED, "hidden %d > 8192", d->hidden);
  if (d->inter_dense < 0 || d->inter_dense % 64)
    return fail(d->inter_dense < 0 ? MOE_INVALID_ARG : MOE_UNSUPPORTED, "inter_dense %d must be a multiple of 64", d->inter_dense);
  if (d->act != MOE_ACT_SILU && d->act != MOE_ACT_GELU_TANH) return fail(MOE_INVALID_ARG, "unknown activation %d", d->act);
  if (d->inter_dense && d->dense_act != MOE_ACT_SILU && d->dense_act != MOE_ACT_GELU_TANH)
    return fail(MOE_INVALID_ARG, "unknown dense activation %d", d->dense_act);
  if (d->act_dtype != MOE_DT_F32 && d->act_dtype != MOE_DT_BF16)
    return fail(MOE_INVALID_ARG, "act_dtype must be F32 or BF16");
  if (d->act_dtype == MOE_DT_F32 && d->weight_dtype != MOE_DT_F32)
    return fail(MOE_UNSUPPORTED, "an fp32 layer needs fp32 expert weights");
  if (d->act_dtype == MOE_DT_BF16 && d->weight_dtype != MOE_DT_BF16 && d->weight_dtype != MOE_DT_FP8_E4M3 &&
      d->weight_dtype != MOE_DT_MXFP4)
    return fail(MOE_UNSUPPORTED, "a bf16 layer needs bf16, fp8 or mxfp4 expert weights");
  if ((d->weight_dtype == MOE_DT_FP8_E4M3 || d->weight_dtype == MOE_DT_MXFP4) && d->n_shared)
    return fail(MOE_UNSUPPORTED, "shared experts with fp8 / mxfp4 routed experts");
  if (d->router_mode != MOE_ROUTER_PLAIN && d->router_mode != MOE_ROUTER_GEMMA)
    return fail(MOE_INVALID_ARG, "unknown router mode %d", d->router_mode);
  if (!(d->eps >= 0.f)) return fail(MOE_INVALID_ARG, "eps must be >= 0");
  if (d->block_tail != 0 && d->block_tail != 1) return fail(MOE_INVALID_ARG, "block_tail must be 0 or 1");
  if (d->combine != MOE_COMBINE_SLOT_ORDER && d->combine != MOE_COMBINE_ATOMIC)
    return fail(MOE_INVALID_ARG, "unknown combine %d", d->combine);
  if (d->combine == MOE_COMBINE_ATOMIC && d->act_dtype == MOE_DT_F32)
    return fail(MOE_UNSUPPORTED, "the atomic combine serves bf16 layers");
  if (d->act_quant != MOE_ACT_QUANT_NONE && d->act_quant != MOE_ACT_QUANT_FP8_DYNAMIC)
    return fail(MOE_INVALID_ARG, "unknown act_quant %d", d->act_quant);
  if (d->act_quant) {
    if (d->weight_dtype != MOE_DT_FP8_E4M3 || d->act_dtype != MOE_DT_BF16)
      return fail(MOE_UNSUPPORTED, "FP8 activations need FP8 expert weights and bf16 x");
    if (d->inter > 16384) return fail(MOE_UNSUPPORTED, "FP8 activations need inter <= 16384");
  }
  moe::RouteOpts o;
  return route_opts(d->num_experts, d->top_k, d->renormalize, d->scoring, d->n_groups, d->topk_groups, o);
}

// The routing options of a validated layer.
moe::RouteOpts layer_route_opts(const moe_layer_desc& d) {
  moe::RouteOpts o;
  route_opts(d.num_experts, d.top_k, d.renormalize, d.scoring, d.n_groups, d.topk_groups, o);
  return o;
}

// The decode path's buffers for T tokens (offsets into the workspace, set in p,
// and the parts of its down kernel); returns the bytes they span.  Needs p's
// Kp, Ep, need_logits, dense and aq.
size_t decode_layout(const moe_layer_desc& d, int64_t T, Plan& p) {
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t r = o;
    o = align_up(o + bytes);
    return r;
  };
  const size_t H = d.hidden;
  const int64_t slots = T * p.Kp;
  p.o_logits = take(p.need_logits ? (size_t)T * d.num_experts * 4 : 0);
  p.o_rinfo = take((size_t)(1 + 17 * p.Ep) * 4);
  p.o_h = take((size_t)slots * d.inter * 2);
  p.o_dh = take(p.dense ? (size_t)T * d.inter_dense * 2 : 0);
  p.o_dout = take(p.dense ? (size_t)T * H * 4 : 0);
  const int wbits = d.weight_dtype == MOE_DT_FP8_E4M3 ? 8 : (d.weight_dtype == MOE_DT_MXFP4 ? 4 : 16);
  p.down_splits = moe::decode_down_splits((int)T, d.hidden, d.inter, p.dense, p.Kp, wbits);
  p.o_ypart = take(p.dense || p.down_splits > 1 || d.block_tail ? (size_t)T * p.down_splits * H * 4 : 0);
  // FP8 activations: x codes and scales, h codes and scales per slot, slot weights
  p.o_xq = take(p.aq ? (size_t)T * H : 0);
  p.o_xs = take(p.aq ? (size_t)T * 4 : 0);
  p.o_hq = take(p.aq ? (size_t)slots * d.inter : 0);
  p.o_hs = take(p.aq ? (size_t)slots * 4 : 0);
  p.o_slotw = take(p.aq ? (size_t)slots * 4 : 0);
  return o;
}

moe_status make_plan(const moe_layer_desc& d, const moe_tensors* t, int64_t T, Plan& p) {
  p.f32 = d.act_dtype == MOE_DT_F32;
  p.Kp = d.top_k + d.n_shared;
  p.Ep = d.num_experts + d.n_shared;
  p.bm = choose_block_m(d, T);
  const int64_t slots = T * p.Kp;
  if (slots >= (int64_t)1 << 31) return fail(MOE_UNSUPPORTED, "T * (top_k + n_shared) >= 2^31");
  p.cap = permute_capacity(slots, p.Ep, p.bm);
  // Every GEMM operand is addressed through a buffer resource with 32-bit offsets.
  const int64_t lim = (int64_t)1 << 31;
  const int64_t wb = d.weight_dtype == MOE_DT_FP8_E4M3 ? 1 : (d.weight_dtype == MOE_DT_F32 ? 4 : 2);
  if (T * d.hidden * 4 >= lim || T * (int64_t)d.inter_dense * 4 >= lim)
    return fail(MOE_UNSUPPORTED, "T = %lld too large: an activation buffer would exceed 2 GiB", (long long)T);
  // The padding alone (up to block_m - 1 rows per expert) can pass the limit for
  // layers with very many wide experts, at any T.
  if (p.cap * d.inter * 4 >= lim)
    return fail(MOE_UNSUPPORTED,
                "T = %lld too large for this layer: the expert intermediate of %lld padded rows x inter %d "
                "would exceed 2 GiB",
                (long long)T, (long long)p.cap, d.inter);
  if ((int64_t)2 * d.inter * d.hidden * wb >= lim || (int64_t)2 * d.inter_dense * d.hidden * 4 >= lim ||
      (int64_t)d.num_experts * d.hidden * 4 >= lim)
    return fail(MOE_UNSUPPORTED, "one expert's weights exceed 2 GiB");
  p.need_logits = !(t && t->logits);
  p.gemma_router = p.need_logits && d.router_mode == MOE_ROUTER_GEMMA;
  p.dense = d.inter_dense > 0;
  p.need_prenorm = p.gemma_router || p.dense;
  // Without a tensor set (workspace query) size for the case that materialises every row.
  p.mat_r = p.gemma_router && (!t || t->router_scale);
  p.mat_xn1 = p.dense && (!t || t->gamma_pre);
  p.aq = d.act_quant != MOE_ACT_QUANT_NONE;
  // FP8 activations quantise the normalised expert input as stored: always materialised
  p.mat_xn2 = p.dense && (!t || t->gamma_pre2 || p.aq);
  const size_t ae = p.f32 ? 4 : 2;  // activation element bytes
  // With the dense branch the MoE sum is RMS-normalised afterwards, which turns
  // its relative error into error at output scale: keep the per-slot rows fp32.
  p.y_f32 = p.f32 || p.dense;
  p.atomic = d.combine == MOE_COMBINE_ATOMIC;
  // Split the down GEMM's reduction when its tiles would fill the CUs in few
  // rounds (long reductions over few rows: the Mixtral-style layer); rows are
  // estimated with half a block of padding per expert.
  p.ks = p.f32 ? 1 : moe::gemm_scatter_k_splits(slots + (int64_t)p.Ep * (p.bm / 2), p.bm, d.hidden, d.inter);
  // The per-slot rows are sized for the most parts this row block allows, not for
  // the parts this T picks (which can fall as T grows): the reported workspace size
  // must not decrease with T.
  const int ks_room = p.f32 ? 1 : moe::gemm_scatter_k_splits_max(p.bm, d.inter);
  const size_t H = d.hidden;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t r = o;
    o = align_up(o + bytes);
    return r;
  };
  p.o_logits = take(p.need_logits ? (size_t)T * d.num_experts * 4 : 0);
  p.o_w = take((size_t)slots * 4);
  p.o_ids = take((size_t)slots * 4);
  p.o_counts = take((size_t)p.Ep * 4);
  p.o_offsets = take((size_t)(p.Ep + 1) * 4);
  p.o_sorted = take((size_t)p.cap * 4);
  p.o_bexp = take((size_t)(p.cap / p.bm) * 4);
  p.o_slotrow = take((size_t)slots * 4);
  p.o_rms = take(p.need_prenorm ? (size_t)T * 4 : 0);
  p.o_r = take(p.mat_r ? (size_t)T * H * ae : 0);
  p.o_xn1 = take(p.mat_xn1 ? (size_t)T * H * ae : 0);
  p.o_xn2 = take(p.mat_xn2 ? (size_t)T * H * ae : 0);
  p.o_h = take((size_t)p.cap * d.inter * ae);
  p.o_y = take(p.atomic ? (size_t)T * H * 4 : (size_t)slots * ks_room * H * (p.y_f32 ? 4 : ae));
  p.o_dh = take(p.dense ? (size_t)T * d.inter_dense * ae : 0);
  p.o_dout = take(p.dense ? (size_t)T * H * 4 : 0);
  p.o_xq = take(p.aq ? (size_t)T * H : 0);
  p.o_xs = take(p.aq ? (size_t)T * 4 : 0);
  p.o_hq = take(p.aq ? (size_t)p.cap * d.inter : 0);
  p.o_hs = take(p.aq ? (size_t)p.cap * 4 : 0);
  p.total = o;
  // The router GEMM has few output tiles (T/128 x E/128) and a reduction over all
  // of H: split it so the tiles cover the CUs.  Its partial planes live in the
  // expert hidden buffer h, which is first written after routing.
  p.ks_r = 1;
  if (p.need_logits && !p.f32) {
    p.ks_r = moe::gemm_store_k_splits(T, d.num_experts, d.hidden);
    const size_t h_bytes = (size_t)p.cap * d.inter * ae;
    while (p.ks_r > 1 && (size_t)p.ks_r * T * d.num_experts * 4 > h_bytes) --p.ks_r;
  }
  // The decode path lays out its own buffers over the same workspace.  The size
  // reported covers both layouts, and past the decode range still the largest
  // decode layout: for small layers the decode path's fp32 partial rows can
  // outweigh the grouped path's buffers, and the size must not fall where a call
  // leaves the decode path.
  p.path_total = p.total;
  p.decode = use_decode(d, T);
  if (p.decode) {
    p.path_total = decode_layout(d, T, p);
    if (p.path_total > p.total) p.total = p.path_total;
  } else {
    int64_t td = std::min<int64_t>(T, 16);  // decode-eligible T form a prefix: LDS needs grow with T
    while (td >= 1 && !use_decode(d, td)) --td;
    if (td >= 1) {
      Plan q = p;
      const size_t bytes = decode_layout(d, td, q);
      if (bytes > p.total) p.total = bytes;
    }
  }
  return MOE_OK;
}

moe_status validate_tensors(const moe_layer_desc& d, const moe_tensors* t) {
  if (!t) return fail(MOE_INVALID_ARG, "tensors is NULL");
  if (!t->x || !t->w13 || !t->w2 || !t->out) return fail(MOE_INVALID_ARG, "x, w13, w2 and out are required");
  if (!t->logits && !t->w_router) return fail(MOE_INVALID_ARG, "either logits or w_router is required");
  if ((d.weight_dtype == MOE_DT_FP8_E4M3 || d.weight_dtype == MOE_DT_MXFP4) && (!t->w13_scale || !t->w2_scale))
    return fail(MOE_INVALID_ARG, "fp8 / mxfp4 weights need w13_scale and w2_scale");
  if (d.n_shared && (!t->shared_w13 || !t->shared_w2))
    return fail(MOE_INVALID_ARG, "n_shared > 0 needs shared_w13 and shared_w2");
  if (d.inter_dense && (!t->dense_w13 || !t->dense_w2))
    return fail(MOE_INVALID_ARG, "inter_dense > 0 needs dense_w13 and dense_w2");
  // Matrix operands are moved in 16-byte pieces (LDS DMA, vector loads and stores).
  const struct {
    const void* p;
    const char* name;
  } mats[] = {{t->x, "x"},          {t->w_router, "w_router"},     {t->w13, "w13"},
              {t->w2, "w2"},        {t->shared_w13, "shared_w13"}, {t->shared_w2, "shared_w2"},
              {t->dense_w13, "dense_w13"}, {t->dense_w2, "dense_w2"}, {t->out, "out"},
              {t->out_f32, "out_f32"}};
  for (const auto& m : mats)
    if ((uintptr_t)m.p % 16) return fail(MOE_INVALID_ARG, "%s must be 16-byte aligned", m.name);
  return MOE_OK;
}

}  // namespace

MOE_API const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_INVALID_ARG: return "MOE_INVALID_ARG";
    case MOE_UNSUPPORTED: return "MOE_UNSUPPORTED";
    case MOE_WORKSPACE_TOO_SMALL: return "MOE_WORKSPACE_TOO_SMALL";
    case MOE_HIP_ERROR: return "MOE_HIP_ERROR";
  }
  return "MOE_UNKNOWN_STATUS";
}

MOE_API const char* moe_last_error(void) { return g_err; }

MOE_API moe_status moe_route(const float* logits, int64_t T, int32_t E, int32_t K, int32_t renorm,
                             int32_t scoring, int32_t n_groups, int32_t topk_groups,
                             const float* per_expert_scale, float* topk_w, int32_t* topk_ids, void* stream) {
  g_err[0] = 0;
  if (T < 0) return fail(MOE_INVALID_ARG, "T < 0");
  if (E < 1 || K < 1 || K > E) return fail(MOE_INVALID_ARG, "need 1 <= K <= E (K=%d, E=%d)", K, E);
  if (E > 512 || K > 64) return fail(MOE_UNSUPPORTED, "E <= 512 and K <= 64 are supported");
  moe::RouteOpts o;
  if (moe_status st = route_opts(E, K, renorm, scoring, n_groups, topk_groups, o)) return st;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_w || !topk_ids) return fail(MOE_INVALID_ARG, "logits, topk_w and topk_ids are required");
  if (T > ((int64_t)1 << 32)) return fail(MOE_UNSUPPORTED, "T too large");
  HIP_TRY(moe::launch_route(logits, T, E, K, o, per_expert_scale, topk_w, topk_ids, K, 0,
                            (hipStream_t)stream),
          "route launch");
  return MOE_OK;
}

MOE_API int64_t moe_permute_capacity(int64_t T, int32_t K, int32_t E, int32_t block_m) {
  if (T < 0 || K < 1 || E < 1 || log2_exact(block_m) < 4 || block_m > 256) return -1;
  return permute_capacity(T * K, E, block_m);
}

MOE_API moe_status moe_permute(const int32_t* topk_ids, int64_t T, int32_t K, int32_t E, int32_t block_m,
                               int32_t* counts, int32_t* offsets, int32_t* sorted_slots, int32_t* block_expert,
                               int32_t* num_padded, int32_t* slot_row, void* stream) {
  g_err[0] = 0;
  if (T < 0) return fail(MOE_INVALID_ARG, "T < 0");
  if (K < 1 || K > 64) return fail(MOE_INVALID_ARG, "K %d outside [1, 64]", K);
  if (E < 1 || E > 1024) return fail(MOE_INVALID_ARG, "E %d outside [1, 1024]", E);
  const int l2 = log2_exact(block_m);
  if (l2 < 4 || block_m > 256) return fail(MOE_INVALID_ARG, "block_m %d must be a power of two in [16, 256]", block_m);
  if (T * K >= ((int64_t)1 << 31)) return fail(MOE_UNSUPPORTED, "T*K >= 2^31");
  if (!counts || !offsets || !sorted_slots || !block_expert || (T > 0 && (!topk_ids || !slot_row)))
    return fail(MOE_INVALID_ARG, "null output pointer");
  HIP_TRY(moe::launch_permute(topk_ids, T * K, E, l2, counts, offsets, sorted_slots, block_expert, num_padded,
                              slot_row, (hipStream_t)stream),
          "permute launch");
  return MOE_OK;
}

MOE_API int32_t moe_forward_path(const moe_layer_desc* desc, int64_t T) {
  if (validate_desc(desc) != MOE_OK || T < 0) return -1;
  return use_decode(*desc, T) ? MOE_PATH_DECODE : MOE_PATH_GROUPED;
}

MOE_API int32_t moe_decode_dense_gate_up_stage(const moe_layer_desc* desc, int64_t T) {
  if (validate_desc(desc) != MOE_OK || T < 0 || !use_decode(*desc, T) || desc->inter_dense == 0) return -1;
  const int kp = desc->top_k + desc->n_shared, ep = desc->num_experts + desc->n_shared;
  return moe::decode_up_blocks_per_cu((int)T, desc->hidden, kp, ep) == 2 ? MOE_STAGE_GATE_UP : MOE_STAGE_ROUTER;
}

MOE_API moe_status moe_forward_workspace_size(const moe_layer_desc* desc, int64_t T, size_t* bytes) {
  g_err[0] = 0;
  moe_status s = validate_desc(desc);
  if (s != MOE_OK) return s;
  if (T < 0) return fail(MOE_INVALID_ARG, "T < 0");
  if (!bytes) return fail(MOE_INVALID_ARG, "bytes is NULL");
  Plan p;
  // Size for computed logits (the larger case); supplied logits need less.
  s = make_plan(*desc, nullptr, T, p);
  if (s != MOE_OK) return s;
  *bytes = p.total;
  return MOE_OK;
}

MOE_API moe_status moe_forward_workspace_layout(const moe_layer_desc* desc, const moe_tensors* t, int64_t T,
                                                moe_workspace_layout* out) {
  g_err[0] = 0;
  moe_status s = validate_desc(desc);
  if (s != MOE_OK) return s;
  if ((s = validate_tensors(*desc, t)) != MOE_OK) return s;
  if (T < 1) return fail(MOE_INVALID_ARG, "T must be >= 1");
  if (!out) return fail(MOE_INVALID_ARG, "layout is NULL");
  Plan p;
  if ((s = make_plan(*desc, t, T, p)) != MOE_OK) return s;
  moe_workspace_layout L;
  L.path = p.decode ? MOE_PATH_DECODE : MOE_PATH_GROUPED;
  L.block_m = p.bm;
  L.slots_per_token = p.Kp;
  L.y_parts = p.atomic ? 0 : p.ks;
  L.y_f32 = p.y_f32 || p.atomic;
  L.capacity = p.cap;
  auto off = [&](bool has, size_t o) { return (!p.decode && has) ? (int64_t)o : (int64_t)-1; };
  if (p.decode) {
    // the decode path's h rows are per slot (row t * slots_per_token + k); with FP8
    // activations also the codes and scales it takes
    L.y_parts = 0;
    L.y_f32 = 0;
    L.capacity = T * p.Kp;
    auto doff = [&](bool has, size_t o) { return has ? (int64_t)o : (int64_t)-1; };
    L.topk_w = L.topk_ids = L.counts = L.offsets = L.sorted_slots = L.block_expert = L.slot_row = -1;
    L.inv_rms = L.x_expert = L.y = -1;
    L.h = doff(true, p.o_h);
    L.x_codes = doff(p.aq, p.o_xq);
    L.x_scales = doff(p.aq, p.o_xs);
    L.h_codes = doff(p.aq, p.o_hq);
    L.h_scales = doff(p.aq, p.o_hs);
    *out = L;
    return MOE_OK;
  }
  L.topk_w = off(true, p.o_w);
  L.topk_ids = off(true, p.o_ids);
  L.counts = off(true, p.o_counts);
  L.offsets = off(true, p.o_offsets);
  L.sorted_slots = off(true, p.o_sorted);
  L.block_expert = off(true, p.o_bexp);
  L.slot_row = off(true, p.o_slotrow);
  L.inv_rms = off(p.need_prenorm, p.o_rms);
  L.x_expert = off(p.mat_xn2, p.o_xn2);
  L.h = off(true, p.o_h);
  L.y = off(true, p.o_y);
  L.x_codes = off(p.aq, p.o_xq);
  L.x_scales = off(p.aq, p.o_xs);
  L.h_codes = off(p.aq, p.o_hq);
  L.h_scales = off(p.aq, p.o_hs);
  *out = L;
  return MOE_OK;
}

// noalloc: the workspace is the library's static scratch, sized for the path this
// call takes, and the dense branch runs on the caller's stream (no side stream or
// events are created).
static moe_status forward_impl(const moe_layer_desc* desc, const moe_tensors* t, int64_t T, void* workspace,
                               size_t workspace_bytes, void* stream, void* const* events, bool noalloc = false) {
  g_err[0] = 0;
  moe_status s = validate_desc(desc);
  if (s != MOE_OK) return s;
  const moe_layer_desc& d = *desc;
  s = validate_tensors(d, t);
  if (s != MOE_OK) return s;
  if (T < 0) return fail(MOE_INVALID_ARG, "T < 0");
  if (T == 0) return MOE_OK;
  Plan p;
  s = make_plan(d, t, T, p);
  if (s != MOE_OK) return s;
  if (d.weight_dtype == MOE_DT_MXFP4 && !p.decode)
    return fail(MOE_UNSUPPORTED, "mxfp4 expert weights serve the decode path only (T <= 16, rows within its LDS staging)");
  const size_t need = noalloc ? p.path_total : p.total;
  if (!workspace || workspace_bytes < need)
    return fail(MOE_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", workspace_bytes, need);
  if ((uintptr_t)workspace % ALIGN) return fail(MOE_INVALID_ARG, "workspace must be 256-byte aligned");

  hipStream_t st = (hipStream_t)stream;
  uint8_t* ws = (uint8_t*)workspace;
  auto mark = [&](int stage) -> hipError_t {
    return events ? hipEventRecord((hipEvent_t)events[stage], st) : hipSuccess;
  };
#define STAGE(i) HIP_TRY(mark(i), "event record")
  if (p.decode) {
    moe::DecodeArgs a{};
    a.T = (int)T;
    a.H = d.hidden;
    a.E = d.num_experts;
    a.K = d.top_k;
    a.Kp = p.Kp;
    a.Ep = p.Ep;
    a.I = d.inter;
    a.Id = d.inter_dense;
    a.act = d.act;
    a.dense_act = d.dense_act;
    a.route = layer_route_opts(d);
    a.gemma_router = d.router_mode == MOE_ROUTER_GEMMA;
    a.dense = p.dense;
    a.eps = d.eps;
    a.n_router_groups = p.need_logits ? (d.num_experts + 15) / 16 : 0;
    // The dense gate/up runs in the up kernel while two of its blocks fit per CU
    // (its weights then stream while the expert blocks route), else with the router.
    const bool dense_in_up = moe::decode_up_blocks_per_cu((int)T, d.hidden, p.Kp, p.Ep) == 2;
    a.n_dense_groups = p.dense && dense_in_up ? d.inter_dense / 16 : 0;
    a.n_pre_dense_groups = p.dense && !dense_in_up ? d.inter_dense / 16 : 0;
    a.max_active = (int)std::min<int64_t>(p.Ep, T * p.Kp);
    a.n_up_blocks = a.max_active * (d.inter / 16);  // items; capped at launch
    a.n_ddown_groups = p.dense ? d.hidden / 16 : 0;
    a.x = t->x;
    a.z = p.need_logits ? (t->logits_out ? t->logits_out : (float*)(ws + p.o_logits)) : const_cast<float*>(t->logits);
    a.w_router = t->w_router;
    a.router_scale = t->router_scale;
    a.pes = t->per_expert_scale;
    a.w13 = t->w13;
    a.w2 = t->w2;
    const bool mx = d.weight_dtype == MOE_DT_MXFP4;
    a.s13 = mx ? nullptr : t->w13_scale;
    a.s2 = mx ? nullptr : t->w2_scale;
    a.mx13 = mx ? (const uint8_t*)t->w13_scale : nullptr;
    a.mx2 = mx ? (const uint8_t*)t->w2_scale : nullptr;
    a.shared_w13 = t->shared_w13;
    a.shared_w2 = t->shared_w2;
    a.dense_w13 = t->dense_w13;
    a.dense_w2 = t->dense_w2;
    a.g_pre = t->gamma_pre;
    a.g_pre2 = t->gamma_pre2;
    a.hd = p.dense ? ws + p.o_dh : nullptr;
    a.hbuf = ws + p.o_h;
    a.dsum = p.dense ? (float*)(ws + p.o_dout) : nullptr;
    a.down_splits = p.down_splits;
    a.ypart = p.dense || p.down_splits > 1 || d.block_tail ? (float*)(ws + p.o_ypart) : nullptr;
    a.rinfo = (int*)(ws + p.o_rinfo);
    a.out = t->out;
    a.out_f32 = t->out_f32;
    a.topk_w_out = t->topk_w_out;
    a.topk_ids_out = t->topk_ids_out;
    a.aq = p.aq;
    if (p.aq) {
      a.xcodes = ws + p.o_xq;
      a.xscales = (float*)(ws + p.o_xs);
      a.hcodes = ws + p.o_hq;
      a.hscales = (float*)(ws + p.o_hs);
      a.slot_w = (float*)(ws + p.o_slotw);
    }
    const int wk = d.weight_dtype == MOE_DT_FP8_E4M3 ? 1 : (d.weight_dtype == MOE_DT_MXFP4 ? 2 : 0);
    // the down kernel stages the routing summary in a 520-entry LDS table; E <= 512
    // and at most 8 shared experts keep max_active within it
    if (a.max_active > 520)
      return fail(MOE_UNSUPPORTED, "decode: %d active experts exceed the routing table", a.max_active);
    STAGE(MOE_STAGE_PRENORM);
    STAGE(MOE_STAGE_ROUTER);
    // router logits
    HIP_TRY(moe::launch_decode_pre(a, st), "decode pre launch");
    if (!p.need_logits && t->logits_out)
      HIP_TRY(hipMemcpyAsync(t->logits_out, t->logits, (size_t)T * d.num_experts * 4, hipMemcpyDeviceToDevice, st),
              "logits copy");
    STAGE(MOE_STAGE_ROUTE);
    STAGE(MOE_STAGE_PERMUTE);
    STAGE(MOE_STAGE_QUANT_X);
    STAGE(MOE_STAGE_GATE_UP);
    // dense gate/up, routing + expert gate/up
    HIP_TRY(moe::launch_decode_up(a, wk, st), "decode up launch");
    STAGE(MOE_STAGE_QUANT_H);
    // FP8 activations: the h row of every slot quantised (all T * Kp rows are written)
    if (p.aq)
      HIP_TRY(moe::launch_quant_rows_fp8(a.hbuf, T * p.Kp, d.inter, d.inter, nullptr, nullptr, (uint8_t*)a.hcodes,
                                         d.inter, (float*)a.hscales, st),
              "decode h quantisation launch");
    STAGE(MOE_STAGE_DOWN);
    // dense down, expert down + combine
    HIP_TRY(moe::launch_decode_down(a, wk, st), "decode down launch");
    STAGE(MOE_STAGE_DENSE_GATE_UP);
    STAGE(MOE_STAGE_DENSE_DOWN);
    STAGE(MOE_STAGE_FINALIZE);
    if (a.ypart)
      HIP_TRY(moe::launch_finalize(a.ypart, moe::ELEM_F32, p.down_splits, a.dsum, t->gamma_post1, t->gamma_post2,
                                   d.eps, t->out, moe::ELEM_BF16, t->out_f32, T, d.hidden, st,
                                   d.block_tail ? t->x : nullptr, t->gamma_post_ff),
              "finalize launch");
    STAGE(MOE_STAGE_COUNT);
    return MOE_OK;
  }
  const int H = d.hidden, E = d.num_experts, K = d.top_k, I = d.inter;
  const int act_elem = p.f32 ? moe::ELEM_F32 : moe::ELEM_BF16;
  const int b_elem = p.aq ? moe::ELEM_FP8X8 : (d.weight_dtype == MOE_DT_FP8_E4M3 ? moe::ELEM_FP8 : moe::ELEM_BF16);
  uint8_t* xq = p.aq ? (uint8_t*)(ws + p.o_xq) : nullptr;
  float* xs = p.aq ? (float*)(ws + p.o_xs) : nullptr;
  uint8_t* hq = p.aq ? (uint8_t*)(ws + p.o_hq) : nullptr;
  float* hs = p.aq ? (float*)(ws + p.o_hs) : nullptr;
  float* w = (float*)(ws + p.o_w);
  int32_t* ids = (int32_t*)(ws + p.o_ids);
  int32_t* counts = (int32_t*)(ws + p.o_counts);
  int32_t* offsets = (int32_t*)(ws + p.o_offsets);
  int32_t* sorted = (int32_t*)(ws + p.o_sorted);
  int32_t* bexp = (int32_t*)(ws + p.o_bexp);
  float* inv_rms = p.need_prenorm ? (float*)(ws + p.o_rms) : nullptr;
  void* r_in = p.mat_r ? ws + p.o_r : nullptr;
  void* xn1 = p.mat_xn1 ? ws + p.o_xn1 : nullptr;
  void* xn2 = p.mat_xn2 ? ws + p.o_xn2 : nullptr;
  void* h = ws + p.o_h;
  void* y = ws + p.o_y;
  void* dh = p.dense ? ws + p.o_dh : nullptr;
  float* dout = p.dense ? (float*)(ws + p.o_dout) : nullptr;

  auto gemm_on = [&](const moe::GemmArgs& a, int epi, int belem, int bm, hipStream_t s) -> hipError_t {
    return p.f32 ? moe::launch_gemm_f32(a, epi, s) : moe::launch_gemm_mfma(a, epi, belem, bm, s);
  };
  auto gemm = [&](const moe::GemmArgs& a, int epi, int belem, int bm) -> hipError_t {
    return gemm_on(a, epi, belem, bm, st);
  };
  // parallel dense MLP (Gemma): dense_out = MLP(xn1) in fp32, on stream s
  auto dense_branch = [&](hipStream_t s, bool marks) -> moe_status {
    const int dbm = T >= 1024 ? 256 : 64;
    moe::GemmArgs a{};
    a.A = p.mat_xn1 ? xn1 : t->x;
    if (!p.mat_xn1) a.row_scale = inv_rms;
    a.lda = H;
    a.M = T;
    a.a_rows_alloc = T;
    a.B0 = t->dense_w13;
    a.n_routed = 1;
    a.N = d.inter_dense;
    a.Kdim = H;
    a.C = dh;
    a.ldc = d.inter_dense;
    a.act = d.dense_act;
    HIP_TRY(gemm_on(a, moe::EPI_GATED, moe::ELEM_BF16, dbm, s), "dense gate/up gemm launch");
    if (marks) STAGE(MOE_STAGE_DENSE_DOWN);
    moe::GemmArgs b{};
    b.A = dh;
    b.lda = d.inter_dense;
    b.M = T;
    b.a_rows_alloc = T;
    b.B0 = t->dense_w2;
    b.n_routed = 1;
    b.N = H;
    b.Kdim = d.inter_dense;
    b.C = dout;
    b.ldc = H;
    HIP_TRY(gemm_on(b, moe::EPI_STORE_F32, moe::ELEM_BF16, dbm, s), "dense down gemm launch");
    return MOE_OK;
  };
  // Overlap the dense branch with the MoE path unless stages are being timed.
  SideStream* side = p.dense && !events && !noalloc ? side_stream(st) : nullptr;
  SideJoin side_join;

  STAGE(MOE_STAGE_PRENORM);
  // 1. input norms (Gemma router preprocessing, pre_feedforward_layernorm / _2):
  //    1/rms per token; normalised rows only where a learned weight is given.
  if (p.need_prenorm)
    HIP_TRY(moe::launch_prenorm(t->x, act_elem, T, H, d.eps, inv_rms, t->router_scale, t->gamma_pre,
                                t->gamma_pre2, r_in, xn1, xn2, st),
            "prenorm launch");
  if (side) {
    HIP_TRY(hipEventRecord(side->fork, st), "fork event");
    HIP_TRY(hipStreamWaitEvent(side->s, side->fork, 0), "fork wait");
    side_join.side = side;
    side_join.st = st;
    side_join.armed = true;
    s = dense_branch(side->s, false);
    if (s != MOE_OK) return s;
  }

  STAGE(MOE_STAGE_ROUTER);
  // 2. router logits (fp32)
  const float* z = t->logits;
  if (p.need_logits) {
    float* zo = t->logits_out ? t->logits_out : (float*)(ws + p.o_logits);
    if (p.ks_r > 1) zo = (float*)h;  // [ks_r, T, E] partial planes
    moe::GemmArgs a{};
    a.A = p.mat_r ? r_in : t->x;
    a.lda = H;
    a.M = T;
    a.a_rows_alloc = T;
    if (p.gemma_router && !p.mat_r) {  // RMSNorm without gamma and H^-0.5 as epilogue factors
      a.row_scale = inv_rms;
      a.c_scale = 1.0f / sqrtf((float)H);
    }
    a.B0 = t->w_router;
    a.n_routed = 1;
    a.N = E;
    a.Kdim = H;
    a.C = zo;
    a.ldc = E;
    a.k_splits = p.ks_r;
    HIP_TRY(gemm(a, moe::EPI_STORE_F32, moe::ELEM_BF16, 128), "router gemm launch");
    z = zo;
  } else if (t->logits_out) {
    HIP_TRY(hipMemcpyAsync(t->logits_out, t->logits, (size_t)T * E * 4, hipMemcpyDeviceToDevice, st),
            "logits copy");
  }

  STAGE(MOE_STAGE_ROUTE);
  // 3. routing weights and ids (shared experts appended as ids E.., weight 1)
  HIP_TRY(moe::launch_route(z, T, E, K, layer_route_opts(d), t->per_expert_scale, w, ids, p.Kp, d.n_shared, st,
                            p.ks_r, T * E, t->logits_out),
          "route launch");

  STAGE(MOE_STAGE_PERMUTE);
  // 4. permutation map
  HIP_TRY(moe::launch_permute(ids, T * p.Kp, p.Ep, log2_exact(p.bm), counts, offsets, sorted, bexp, nullptr,
                              (int32_t*)(ws + p.o_slotrow), st),
          "permute launch");

  STAGE(MOE_STAGE_QUANT_X);
  // 5. grouped gate/up GEMM + gated activation -> h [cap, I]
  //    (FP8 activations: x quantised per token first, its scale a row factor)
  if (p.aq)
    HIP_TRY(moe::launch_quant_rows_fp8(p.mat_xn2 ? xn2 : t->x, T, H, H, nullptr, nullptr, xq, H, xs, st),
            "x quantisation launch");
  STAGE(MOE_STAGE_GATE_UP);
  {
    moe::GemmArgs a{};
    a.A = p.mat_xn2 ? xn2 : t->x;
    if (p.dense && !p.mat_xn2) a.row_scale = inv_rms;
    if (p.aq) {
      a.A = xq;
      a.row_scale = xs;
    }
    a.lda = H;
    a.a_rows = sorted;
    a.row_div = p.Kp;
    a.M = p.cap;
    a.a_rows_alloc = T;
    a.m_dev = offsets + p.Ep;
    a.block_expert = bexp;
    a.seg_off = offsets;
    a.B0 = t->w13;
    a.B1 = t->shared_w13;
    a.bstride = (int64_t)2 * I * H;
    a.n_routed = E;
    a.bscale0 = t->w13_scale;
    a.sstride = 2 * I;
    a.N = I;
    a.Kdim = H;
    a.C = h;
    a.ldc = I;
    a.act = d.act;
    HIP_TRY(gemm(a, moe::EPI_GATED, b_elem, p.bm), "gate/up gemm launch");
  }
  STAGE(MOE_STAGE_QUANT_H);
  // 6. grouped down GEMM, scaled by the routing weight, scattered to per-slot rows
  //    (FP8 activations: h quantised per padded row, padding rows to zeros)
  if (p.aq)
    HIP_TRY(moe::launch_quant_rows_fp8(h, p.cap, I, I, sorted, offsets + p.Ep, hq, I, hs, st),
            "h quantisation launch");
  STAGE(MOE_STAGE_DOWN);
  if (p.atomic) HIP_TRY(moe::launch_zero(y, (size_t)T * H * 4, st), "zero fill launch");
  {
    moe::GemmArgs a{};
    a.A = p.aq ? (const void*)hq : h;
    a.row_scale = hs;
    a.lda = I;
    a.M = p.cap;
    a.a_rows_alloc = p.cap;
    a.m_dev = offsets + p.Ep;
    a.block_expert = bexp;
    a.seg_off = offsets;
    a.B0 = t->w2;
    a.B1 = t->shared_w2;
    a.bstride = (int64_t)H * I;
    a.n_routed = E;
    a.bscale0 = t->w2_scale;
    a.sstride = H;
    a.N = H;
    a.Kdim = I;
    a.C = y;
    a.ldc = H;
    a.c_rows = sorted;
    a.row_weight = w;
    a.k_splits = p.ks;
    a.row_div = p.Kp;  // atomic combine: a slot's token
    const int epi = p.atomic ? moe::EPI_SCATTER_ATOMIC
                             : ((p.y_f32 && !p.f32) ? moe::EPI_SCATTER_F32 : moe::EPI_SCATTER);
    HIP_TRY(gemm(a, epi, b_elem, p.bm), "down gemm launch");
  }
  STAGE(MOE_STAGE_DENSE_GATE_UP);
  // 7. parallel dense MLP (Gemma), here when it did not run on the side stream
  if (p.dense && !side) {
    s = dense_branch(st, true);
    if (s != MOE_OK) return s;
  } else {
    STAGE(MOE_STAGE_DENSE_DOWN);
  }
  HIP_TRY(side_join.join(), "join of the dense branch");
  STAGE(MOE_STAGE_FINALIZE);
  // 8. per-token combine in slot order (+ Gemma post-norms and branch sum)
  HIP_TRY(moe::launch_finalize(y, p.y_f32 || p.atomic ? moe::ELEM_F32 : act_elem, p.atomic ? 1 : p.Kp * p.ks, dout,
                               t->gamma_post1, t->gamma_post2, d.eps, t->out, act_elem,
                               t->out_f32, T, H, st, d.block_tail ? t->x : nullptr, t->gamma_post_ff),
          "finalize launch");
  // 9. optional copies of the routing result
  if (t->topk_w_out || t->topk_ids_out)
    HIP_TRY(moe::launch_gather_topk(w, ids, p.Kp, K, T, t->topk_w_out, t->topk_ids_out, st), "topk copy");
  STAGE(MOE_STAGE_COUNT);
#undef STAGE
  return MOE_OK;
}

MOE_API moe_status moe_forward(const moe_layer_desc* desc, const moe_tensors* t, int64_t T, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return forward_impl(desc, t, T, workspace, workspace_bytes, stream, nullptr);
}

// ---- moe_forward for callers that cannot allocate: the workspace is a static
// device array of MOE_NOALLOC_SCRATCH_BYTES, one copy per GPU, held until the
// process ends.  In host code `scratch` names a host-side stand-in, never device
// memory: its device address is looked up once per device with
// hipGetSymbolAddress and only that address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

static moe_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(MOE_UNSUPPORTED, "device index %d >= 64", dev);
  static std::mutex mu;
  static void* addr[64] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || (uintptr_t)ptr % ALIGN) return fail(MOE_HIP_ERROR, "static scratch at an unusable address");
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return MOE_OK;
}

MOE_API moe_status moe_forward_noalloc(const moe_layer_desc* desc, const moe_tensors* t, int64_t T, void* stream) {
  g_err[0] = 0;
  moe_status s = validate_desc(desc);
  if (s != MOE_OK) return s;
  if ((s = validate_tensors(*desc, t)) != MOE_OK) return s;
  if (T < 0) return fail(MOE_INVALID_ARG, "T < 0");
  if (T == 0) return MOE_OK;
  Plan p;
  if ((s = make_plan(*desc, t, T, p)) != MOE_OK) return s;
  if (p.path_total > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_WORKSPACE_TOO_SMALL,
                "T = %lld needs %zu bytes of scratch; the static scratch holds %zu (call moe_forward with a "
                "workspace instead)",
                (long long)T, p.path_total, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((s = scratch_address(&ws)) != MOE_OK) return s;
  return forward_impl(desc, t, T, ws, MOE_NOALLOC_SCRATCH_BYTES, stream, nullptr, true);
}

MOE_API moe_status moe_forward_profiled(const moe_layer_desc* desc, const moe_tensors* t, int64_t T,
                                        void* workspace, size_t workspace_bytes, void* stream,
                                        void* const* events) {
  if (!events) return fail(MOE_INVALID_ARG, "events is NULL");
  for (int i = 0; i <= MOE_STAGE_COUNT; ++i)
    if (!events[i]) return fail(MOE_INVALID_ARG, "events[%d] is NULL", i);
  return forward_impl(desc, t, T, workspace, workspace_bytes, stream, events);
}
