/*
 * moe.h - C ABI of libmoe_mi355x.so, the MoE FFN layer forward for one
 * AMD Instinct MI355X (gfx950).
 *
 * Conventions for every entry point:
 *   - All tensors are dense, row-major, contiguous device pointers (HIP device
 *     memory the caller owns).  The library allocates no device memory and keeps
 *     no data between calls; calls on different streams are independent.  The
 *     one thing it keeps: moe_forward creates, on first need per caller stream,
 *     host thread and device (up to 16 caller streams per thread), a second
 *     stream (default priority, non-blocking) and two events, held until the
 *     process ends; a layer's dense branch runs on that stream, ordered with the
 *     caller's stream by those events (see moe_forward).  Every return after the
 *     fork, errors included, first makes the caller's stream wait for it.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Work
 *     is enqueued asynchronously on it; the call returns once it is enqueued.
 *   - Arguments are validated on the host before anything is launched.  A bad
 *     argument returns an error status and launches nothing; nothing is ever
 *     skipped silently and no call aborts the process.  moe_last_error() gives
 *     a description of the last failure on the calling thread.
 *   - T = 0 is a valid no-op.
 *   - bf16 is stored as uint16_t (the upper half of an IEEE fp32); fp8 weights are
 *     OCP E4M3 ("fn": finite, max 448) codes stored as uint8_t; MXFP4 weights are
 *     OCP MXFP4: E2M1 codes, two per byte (the even element in the low nibble),
 *     with one E8M0 scale byte (2^(s-127)) per 32 consecutive elements along the
 *     reduction dimension.
 *
 * Citations name the web pages that describe each operation:
 *   [G4] "Gemma 4 26B-A4B MoE walkthrough" (yeyulingfeng.com/587419)
 *   [VD] vLLM API docs, vllm.model_executor.models.gemma4 (Gemma4MoE, Gemma4Router)
 *   [MI] "MOE Inference" (gaohongy.github.io), gated FFN
 *   [LC] llama.cpp visual guide, lesson 35 (MoE)
 *   [SG] sglang PR #24696 summary (per-expert FP8 weights with weight_scale)
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_INVALID_ARG = 1,          /* null pointer, bad size, bad enum value */
  MOE_UNSUPPORTED = 2,          /* valid request the kernels do not cover (e.g. H % 64 != 0) */
  MOE_WORKSPACE_TOO_SMALL = 3,  /* workspace smaller than moe_forward_workspace_size() */
  MOE_HIP_ERROR = 4             /* a HIP launch or runtime call failed */
} moe_status;

typedef enum { MOE_ACT_SILU = 0, MOE_ACT_GELU_TANH = 1 } moe_act;
typedef enum { MOE_DT_F32 = 0, MOE_DT_BF16 = 1, MOE_DT_FP8_E4M3 = 2, MOE_DT_MXFP4 = 3 } moe_dtype;
typedef enum { MOE_ROUTER_PLAIN = 0, MOE_ROUTER_GEMMA = 1 } moe_router_mode;
/* How the router turns logits into routing probabilities ([LC] routing: a
 * softmax, or in some models a sigmoid). */
typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_scoring;
/* Activation quantisation of the routed experts' GEMM inputs ([SG]: the
 * "FP8-Dynamic" checkpoints quantise activations at run time, per token). */
typedef enum { MOE_ACT_QUANT_NONE = 0, MOE_ACT_QUANT_FP8_DYNAMIC = 1 } moe_act_quant;
/* The weighted combine ([G4] section 7: a weighted scatter-add of the expert
 * outputs into their tokens' rows).  SLOT_ORDER: each (token, slot) row is
 * stored and a token's rows are summed in slot order: deterministic, bit for
 * bit.  ATOMIC: the down GEMM adds each weighted row (every part of a split
 * reduction) into its token's fp32 row with float atomics: less memory
 * traffic, but the summation order, and so the last bits, vary between runs. */
typedef enum { MOE_COMBINE_SLOT_ORDER = 0, MOE_COMBINE_ATOMIC = 1 } moe_combine;

/* Human-readable name of a status code (static storage). */
const char* moe_status_string(moe_status s);
/* Description of the last error on the calling thread ("" if none). */
const char* moe_last_error(void);

/*
 * moe_route - softmax over all experts (or a sigmoid per expert), top-k,
 * renormalisation and the per-expert scale fold, one token per wavefront.
 *
 * Defined by [G4] section 4 (routing maths) and section 5 (per-expert scale),
 * and the routing function of Gemma4MoE in [VD]; [LC] routing (softmax ->
 * argsort_top_k -> get_rows -> normalise) is the same with unit scales, and
 * [LC] names the two variants taken here: sigmoid scoring, and expert groups
 * (groups picked first, then experts inside the picked groups).
 * For each token t:
 *   candidates      = all E experts; with n_groups > 1, the experts form n_groups
 *                     equal contiguous ranges, a range scores its largest logit,
 *                     and only the topk_groups best ranges (ties to the lower
 *                     range) are candidates;
 *   ids[t, 0..K-1]  = the K largest candidate logits, largest first; ties go to
 *                     the lower expert index and -0.0 equals +0.0;
 *   p_e             = softmax over all E at e (scoring SOFTMAX), or
 *                     1 / (1 + exp(-z_e)) (scoring SIGMOID);
 *   renorm != 0:     w[t, j] = p_ids_j / sum_{i<K} p_ids_i
 *                    (softmax: = exp(z_ids_j) / sum_{i<K} exp(z_ids_i));
 *   renorm == 0:     w[t, j] = p_ids_j;
 *   then             w[t, j] *= per_expert_scale[ids_j]   (1 when NULL).
 *
 *   logits            [T, E] fp32, finite (non-finite logits give undefined ids).
 *   scoring           moe_scoring.
 *   n_groups          0 or 1: no groups; else 2..64, dividing E.
 *   topk_groups       with n_groups > 1: 1..n_groups, and topk_groups * E / n_groups >= K.
 *   per_expert_scale  [E] fp32 or NULL.
 *   topk_w            [T, K] fp32 out.   topk_ids [T, K] int32 out.
 * Limits: 1 <= K <= E <= 512, K <= 64.  T >= 0.
 */
moe_status moe_route(const float* logits, int64_t T, int32_t E, int32_t K, int32_t renorm,
                     int32_t scoring, int32_t n_groups, int32_t topk_groups,
                     const float* per_expert_scale, float* topk_w, int32_t* topk_ids,
                     void* stream);

/*
 * Capacity (number of int32 entries) sorted_slots must hold for moe_permute:
 * floor((T*K + E*(block_m-1)) / block_m) * block_m.  Returns -1 on bad arguments.
 */
int64_t moe_permute_capacity(int64_t T, int32_t K, int32_t E, int32_t block_m);

/*
 * moe_permute - the dispatch permutation map: (token, slot) pairs regrouped
 * expert-major without copying any token data ([G4] sections 6-7: dispatch
 * builds a permutation map that the grouped GEMM reads indirectly; section 7
 * walks the token -> (expert, row) map both ways).
 *
 * Flat slot f = t*K + j refers to topk_ids[t, j].  Expert e's segment is
 * sorted_slots[offsets[e] .. offsets[e] + counts[e]) and lists its flat slots
 * in ascending order (a stable sort by expert); the segment is then padded with
 * -1 up to a multiple of block_m, so offsets[e+1] - offsets[e] =
 * ceil(counts[e] / block_m) * block_m and offsets[E] is the padded total.
 * block_expert[b] = expert owning rows [b*block_m, (b+1)*block_m) for
 * b < offsets[E] / block_m.  slot_row is the inverse map: slot_row[f] = the
 * padded row r with sorted_slots[r] == f.  Entries of sorted_slots and
 * block_expert past the padded total are left untouched.
 *
 * Work: a histogram per chunk of 4096 slots, one scan over the experts, and a
 * stable scatter: every id is read twice, however many experts there are.
 *
 *   topk_ids      [T, K] int32, each in [0, E).
 *   counts        [E] int32 out.          offsets [E+1] int32 out.
 *   sorted_slots  [moe_permute_capacity(T,K,E,block_m)] int32 out.
 *   block_expert  [capacity / block_m] int32 out.
 *   num_padded    [1] int32 out (= offsets[E]), or NULL.
 *   slot_row      [T*K] int32 out (also holds per-chunk counts while the call's
 *                 work runs on `stream`; may be NULL only when T == 0).
 * Limits: block_m a power of two in [16, 256]; 1 <= K <= 64; 1 <= E <= 1024;
 * T*K < 2^31.  Expert ids outside [0, E) are a precondition violation: those
 * slots are dropped from every segment (the counts then sum to less than T*K)
 * and their slot_row entries are -1.
 */
moe_status moe_permute(const int32_t* topk_ids, int64_t T, int32_t K, int32_t E, int32_t block_m,
                       int32_t* counts, int32_t* offsets, int32_t* sorted_slots,
                       int32_t* block_expert, int32_t* num_padded, int32_t* slot_row, void* stream);

/* Layer description (host memory, read during the call only).  Besides the
 * per-field rules below, the kernels address each operand with 32-bit byte
 * offsets: one routed expert's w13 (2 * inter * hidden elements, counted at 1
 * byte for fp8, 2 for bf16 and MXFP4, 4 for fp32), the dense w13 (2 *
 * inter_dense * hidden * 4 bytes) and the router (num_experts * hidden * 4
 * bytes) must each stay under 2 GiB, else MOE_UNSUPPORTED. */
typedef struct {
  int32_t hidden;        /* H, multiple of 64 */
  int32_t num_experts;   /* E routed experts, 1..512 */
  int32_t top_k;         /* K, 1..min(E, 64) */
  int32_t inter;         /* I of every routed expert, multiple of 64 */
  int32_t act;           /* moe_act of the routed / shared experts */
  int32_t act_dtype;     /* MOE_DT_F32 or MOE_DT_BF16: x, out, router / shared / dense weights */
  int32_t weight_dtype;  /* routed expert weights: F32 (needs act F32), BF16, FP8_E4M3 (needs BF16), or
                            MXFP4 (needs BF16; decode path only, see moe_forward) */
  int32_t renormalize;   /* non-zero: renormalise the top-k weights (see moe_route) */
  int32_t router_mode;   /* moe_router_mode, used when logits are computed */
  int32_t n_shared;      /* always-on shared experts (weight 1, same I), 0..8 */
  int32_t inter_dense;   /* > 0: parallel dense MLP of this I with Gemma post-norms; 0: none */
  int32_t dense_act;     /* moe_act of the dense MLP */
  float eps;             /* RMSNorm epsilon (router preprocessing and Gemma norms) */
  int32_t scoring;       /* moe_scoring (see moe_route) */
  int32_t n_groups;      /* expert groups for group-limited routing: 0 or 1 = none, else 2..64 */
  int32_t topk_groups;   /* groups picked per token when n_groups > 1 */
  int32_t act_quant;     /* moe_act_quant: MOE_ACT_QUANT_FP8_DYNAMIC needs FP8 weights, bf16 x
                            and inter <= 16384; the dense branch stays bf16 (see moe_forward) */
  int32_t block_tail;    /* 1: also the FFN block's tail, out = x + RMSNorm(out) * gamma_post_ff
                            ([G4] section 1); 0: the layer output alone */
  int32_t combine;       /* moe_combine, grouped bf16 path: how a token's weighted expert outputs
                            are summed (the decode path sums in its accumulators either way) */
} moe_layer_desc;

/* Tensors of one forward call (device pointers unless noted).  The matrix
 * tensors (x, w_router, w13, w2, shared and dense weights, out, out_f32) must be
 * 16-byte aligned, else MOE_INVALID_ARG; the vectors and routing outputs need
 * only their element alignment. */
typedef struct {
  const void* x;                  /* [T, H] act_dtype */
  const float* logits;            /* [T, E] fp32 router logits, or NULL: computed from x */
  const void* w_router;           /* [E, H] act_dtype (needed when logits == NULL) */
  const float* router_scale;      /* [H] learned per-dimension router scale, NULL = ones (Gemma mode) */
  const float* per_expert_scale;  /* [E], NULL = ones */
  const void* w13;                /* [E, 2I, H]: rows [0,I) gate (w1), rows [I,2I) up (w3) */
  const void* w2;                 /* [E, H, I] down projection */
  const float* w13_scale;         /* FP8: [E, 2I] per-output-channel fp32 scales; MXFP4: uint8 E8M0
                                     block scales [E, 2I, H/32] (one per 32 along H) */
  const float* w2_scale;          /* FP8: [E, H] fp32; MXFP4: uint8 [E, H, I/32] */
  const void* shared_w13;         /* [n_shared, 2I, H] act_dtype, or NULL when n_shared == 0 */
  const void* shared_w2;          /* [n_shared, H, I] */
  const void* dense_w13;          /* [2*inter_dense, H] act_dtype (gate rows first) */
  const void* dense_w2;           /* [H, inter_dense] */
  const float* gamma_pre;         /* [H] pre_feedforward_layernorm weight (dense input), NULL = ones */
  const float* gamma_pre2;        /* [H] pre_feedforward_layernorm_2 weight (expert input), NULL = ones */
  const float* gamma_post1;       /* [H] post norm of the dense branch, NULL = ones */
  const float* gamma_post2;       /* [H] post norm of the MoE branch, NULL = ones */
  void* out;                      /* [T, H] act_dtype, overwritten */
  float* logits_out;              /* optional [T, E]: the logits the routing used */
  float* topk_w_out;              /* optional [T, K] */
  int32_t* topk_ids_out;          /* optional [T, K] */
  float* out_f32;                 /* optional [T, H] fp32: the output before its final rounding to act_dtype */
  const float* gamma_post_ff;     /* [H] post_feedforward_layernorm weight (block_tail), NULL = ones */
} moe_tensors;

/*
 * Bytes of workspace moe_forward needs for T tokens (*bytes set on MOE_OK).
 * Non-decreasing in T: a workspace sized for T serves every smaller T.
 * MOE_UNSUPPORTED when one of the layout's buffers would pass 2 GiB (the kernels
 * address them with 32-bit offsets): from some T on, and then for every larger
 * T; from T = 0 for layers whose row padding alone (up to block_m - 1 rows per
 * expert, times inter) passes it.
 */
moe_status moe_forward_workspace_size(const moe_layer_desc* desc, int64_t T, size_t* bytes);

/*
 * moe_forward - the MoE FFN layer forward.
 *
 *   z      = logits if given, else r . W_router^T in fp32, where r = x (plain
 *            router) or r = RMSNorm_without_gamma(x) * H^-0.5 * router_scale
 *            (Gemma router: [G4] section 3, Gemma4Router.forward in [VD]);
 *   w, ids = moe_route(z)                       ([G4] sections 4-5);
 *   dispatch by moe_permute, no token copies    ([G4] sections 6-7);
 *   per expert e and routed row: h = act(x_e W1_e^T) * (x_e W3_e^T), y = h W2_e^T
 *            (gated FFN, [MI]; activation SiLU [LC] or GELU-tanh [G4] section 6);
 *            x_e = RMSNorm(x) * gamma_pre2 when the dense branch is present, else x;
 *            FP8 weights: W = decode_e4m3(q) * scale[e, n] ([SG]);
 *            MXFP4 weights: W[n, k] = decode_e2m1(q[n, k]) * 2^(s[n, k/32] - 127) ([LC]:
 *            4-bit experts for decode memory); these run on the decode path only,
 *            other T return MOE_UNSUPPORTED;
 *            FP8 activations (act_quant, [SG] FP8-Dynamic): the routed experts' GEMM
 *            inputs x_e and h are each quantised per row first, scale = max|row| / 448
 *            (1 for a zero row), code = E4M3 nearest-even of value / scale (fp32),
 *            both as stored in bf16; the products run on FP8 x FP8 MFMAs and the row
 *            and channel scales multiply the accumulators;
 *   moe_t  = sum_j w[t,j] y_{t,j}              (weighted combine, [G4] section 7);
 *   shared experts: moe_t += sum_s FFN_s(x_t) with weight 1 ([LC] shared expert);
 *   dense branch (inter_dense > 0, [G4] section 1):
 *            out = RMSNorm(MLP(RMSNorm(x)*gamma_pre))*gamma_post1 + RMSNorm(moe)*gamma_post2;
 *   otherwise out = moe.
 *   block_tail (the rest of the FFN block, [G4] section 1): out = x + RMSNorm(out) * gamma_post_ff,
 *   computed in fp32 before the single output rounding.
 *
 * Precision: bf16 operands with fp32 accumulation (fp32 throughout for
 * act_dtype F32); the gated intermediate and the per-slot expert outputs are
 * rounded to bf16 in the bf16 path; logits are fp32.
 *
 * On the grouped path the dense branch runs on the library's second stream
 * between an event recorded on `stream` after the input norms and a wait of
 * `stream` before the finalize, so it overlaps routing, permutation and the
 * grouped GEMMs; moe_forward_profiled keeps it on `stream`.
 *
 * Two execution paths compute this same operation (moe_forward_path tells which
 * one a call takes).  The grouped path permutes the routed rows and runs grouped
 * GEMMs.  The decode path (T <= 16 bf16 tokens) streams each selected expert's
 * weights once and applies them to all tokens together; it folds the routing
 * weight into the gated intermediate before its bf16 rounding (with FP8
 * activations: into the slot's h scale, after the quantisation of the
 * unweighted h) and sums the expert outputs of a token in fp32 before the
 * single output rounding.  Its FP8 activation codes equal the grouped path's;
 * its products take the codes widened to bf16 (exact) on bf16 MFMAs.
 *
 * workspace: device memory of at least moe_forward_workspace_size() bytes,
 * 256-byte aligned, owned by the caller; contents on entry do not matter and
 * are clobbered.  Two calls that share a workspace must be stream-ordered.
 */
moe_status moe_forward(const moe_layer_desc* desc, const moe_tensors* tensors, int64_t T,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_forward_noalloc - moe_forward (same operation, results, arguments and
 * errors) for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  It takes no
 * workspace: the library's own static device scratch of
 * MOE_NOALLOC_SCRATCH_BYTES serves as one (each GPU the library runs on holds
 * its copy until the process ends), and the call allocates nothing and creates
 * no stream or event (the dense branch runs on `stream`).  The first call on a
 * device looks up that device's scratch address once.
 *
 * A call whose layout needs more than MOE_NOALLOC_SCRATCH_BYTES returns
 * MOE_WORKSPACE_TOO_SMALL before launching anything (the decode path and
 * moderate token counts fit; large prefill batches need moe_forward with a
 * workspace).  Every call on one GPU shares that GPU's scratch: calls that
 * overlap on one GPU (on different streams, or from several threads without
 * stream ordering) race and give undefined results.  The scratch keeps the
 * last call's contents; nothing in it needs to start at zero.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_forward_noalloc(const moe_layer_desc* desc, const moe_tensors* tensors, int64_t T, void* stream);

/* Execution path moe_forward takes for T tokens ([LC] lesson 35: a decode
 * token touches only its experts' weights, so the layer is bound by reading
 * them).  Returns MOE_PATH_GROUPED, MOE_PATH_DECODE, or -1 for an invalid
 * descriptor or T < 0. */
typedef enum { MOE_PATH_GROUPED = 0, MOE_PATH_DECODE = 1 } moe_path;
int32_t moe_forward_path(const moe_layer_desc* desc, int64_t T);

/* Stage (MOE_STAGE_ROUTER or MOE_STAGE_GATE_UP) whose launch runs the dense
 * MLP's gate/up on the decode path for T tokens: the gate/up launch while two of
 * its blocks fit per CU with the staged token rows, else the router launch.
 * -1 for an invalid descriptor, a layer without the dense branch, or a T that
 * takes the grouped path.  For measurement (bytes per stage). */
int32_t moe_decode_dense_gate_up_stage(const moe_layer_desc* desc, int64_t T);

/* Where one moe_forward call keeps its intermediates in the workspace, for
 * inspection (tests, debugging): byte offsets into the workspace, -1 for a
 * buffer the call does not have.  Contents are those the call left once its
 * work on the stream has completed, until the workspace is used again.  On the
 * decode path (path == MOE_PATH_DECODE) only h, as [T * slots_per_token, I] rows
 * in slot order (capacity = T * slots_per_token), and with FP8 activations
 * x_codes, x_scales, h_codes and h_scales (per slot row) are given; every other
 * offset is -1 and y_parts is 0.
 *   topk_w, topk_ids  [T, slots_per_token] fp32 / int32 (shared experts appended
 *                     as ids E.., weight 1)
 *   counts [E+S], offsets [E+S+1], sorted_slots [capacity], block_expert
 *   [capacity / block_m], slot_row [T * slots_per_token]  (as moe_permute)
 *   inv_rms           [T] fp32, 1/sqrt(mean(x^2) + eps) (router or dense branch present)
 *   x_expert          [T, H] act dtype: the normalised expert input, where stored
 *   h                 [capacity, I] act dtype: the gated intermediate per padded row
 *   y                 [T * slots_per_token * y_parts, H] (fp32 when y_f32, else act
 *                     dtype): row (slot * y_parts + part) holds the routing-weighted
 *                     expert output of flat slot `slot`, summed over the parts;
 *                     with the atomic combine y_parts is 0 and y is [T, H] fp32,
 *                     each token's combined MoE row
 *   x_codes [T, H] u8, x_scales [T] fp32, h_codes [capacity, I] u8,
 *   h_scales [capacity] fp32: FP8 activations (E4M3 codes, per-row scales) */
typedef struct {
  int32_t path, block_m, slots_per_token, y_parts, y_f32;
  int64_t capacity;
  int64_t topk_w, topk_ids, counts, offsets, sorted_slots, block_expert, slot_row, inv_rms, x_expert, h, y,
      x_codes, x_scales, h_codes, h_scales;
} moe_workspace_layout;
moe_status moe_forward_workspace_layout(const moe_layer_desc* desc, const moe_tensors* tensors, int64_t T,
                                        moe_workspace_layout* layout);

/* Stages of moe_forward, in launch order (indices into the event array below). */
typedef enum {
  MOE_STAGE_PRENORM = 0,        /* 1/rms per token (+ rows with learned norm weights) */
  MOE_STAGE_ROUTER = 1,         /* router logits GEMM */
  MOE_STAGE_ROUTE = 2,          /* moe_route */
  MOE_STAGE_PERMUTE = 3,        /* moe_permute */
  MOE_STAGE_QUANT_X = 4,        /* FP8 activations: per-token quantisation of x */
  MOE_STAGE_GATE_UP = 5,        /* grouped gate/up GEMM + gated activation */
  MOE_STAGE_QUANT_H = 6,        /* FP8 activations: per-row quantisation of h */
  MOE_STAGE_DOWN = 7,           /* grouped down GEMM + routing-weight scatter */
  MOE_STAGE_DENSE_GATE_UP = 8,  /* dense MLP gate/up GEMM */
  MOE_STAGE_DENSE_DOWN = 9,     /* dense MLP down GEMM */
  MOE_STAGE_FINALIZE = 10,      /* per-token combine, post-norms, output rounding */
  MOE_STAGE_COUNT = 11
} moe_stage;

/*
 * moe_forward_profiled - moe_forward (same operation, arguments and errors)
 * that also records caller-created HIP events (hipEvent_t passed as void*) on
 * `stream`: events[i] just before stage i and events[MOE_STAGE_COUNT] after the
 * last one, so hipEventElapsedTime(events[i], events[i+1]) is the time of stage
 * i.  A stage that does not run for this layer gets two back-to-back records.
 * On the decode path the gate/up stage also runs the dense gate/up and the
 * routing, and the down stage also runs the dense down and the combine.
 * It only records: nothing is synchronised.  For measurement.
 */
moe_status moe_forward_profiled(const moe_layer_desc* desc, const moe_tensors* tensors, int64_t T,
                                void* workspace, size_t workspace_bytes, void* stream,
                                void* const* events);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
