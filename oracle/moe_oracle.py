"""Plain, slow CPU oracle for the MoE FFN layer forward (float64, numpy).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this module: only the tests, the smoke check and the CPU-baseline leg
of the benchmark do.  It shares no code, table or constant generator with the
HIP library; inputs reach both sides from the seeded generator as exact
stored values (bf16 and fp32 widen exactly to float64; fp8 codes are decoded
here from the OCP E4M3 definition).

Every step is written as the plain definition of what the layer computes, in
the order and notation of the pages it follows:

* "Gemma 4 26B-A4B MoE walkthrough" (yeyulingfeng.com/587419):
  §1 (MoE branch inside the decoder layer), §3 (Gemma4Router input
  preprocessing), §4 (routing maths: top-k on logits, softmax over all
  experts, indicator mask, renormalisation, gather), §5 (per-expert scale
  folded into the routing weights), §6 (gated MLP / GELU-tanh), §7 (tensor
  flow: dispatch, grouped expert FFN, weighted combine).
* vLLM API docs, "vllm.model_executor.models.gemma4": Gemma4MoE (routing
  function), Gemma4Router.forward, load_weights (w13 = [gate; up] rows of
  shape [I, H], w2 of shape [H, I]).
* "MOE Inference" (gaohongy.github.io): gated FFN (Act(x w1) * (x w3)) w2 with
  the merged w13.
* llama.cpp visual guide, lesson 35 (MoE): softmax / argsort_top_k / get_rows /
  normalise routing, sigmoid scoring, expert groups; mul_mat_id sparse expert
  matmuls; shared experts.
* sglang PR #24696 summary: per-expert FP8 weights with a weight_scale per
  projection; "FP8-Dynamic" checkpoints (activations quantised at run time).

Readings where the pages are silent are listed in the repository's design
notes and repeated at the function that takes them.  Every function here is
pinned by the CPU tests (worked example, closed forms, brute force, library
routines); none is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

RMS_EPS = 1e-6  # reading: the pages print no epsilon; 1e-6 is the Gemma fused-norm default


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------
# Elementwise pieces
# ----------------------------------------------------------------------------

def silu(a):
    """SiLU(a) = a * sigmoid(a) ("MOE Inference", gated FFN: Act is usually SiLU;
    llama.cpp lesson 35: silu(gate) * up)."""
    a = _f64(a)
    return a / (1.0 + np.exp(-a))


def gelu_tanh(a):
    """GELU with the tanh approximation, 0.5 a (1 + tanh(sqrt(2/pi) (a + 0.044715 a^3)))
    (Gemma 4 walkthrough §6, the gelu_pytorch_tanh activation)."""
    a = _f64(a)
    return 0.5 * a * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (a + 0.044715 * a ** 3)))


ACTIVATIONS = {"silu": silu, "gelu_tanh": gelu_tanh}


def activation(name):
    """Gated activation by name.  Any other name is an error, never a fallback
    (Gemma 4 walkthrough §6: the MLP raises on an activation it does not know)."""
    if name not in ACTIVATIONS:
        raise ValueError(f"unsupported activation {name!r}")
    return ACTIVATIONS[name]


def rmsnorm(x, gamma=None, eps=RMS_EPS):
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * gamma.

    gamma=None is the weightless form the router uses (Gemma 4 walkthrough §3,
    RMSNorm(has_weight=False)).  Reading: gamma multiplies directly (the pages
    show y = (x / RMS(x)) * gamma)."""
    x = _f64(x)
    y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    if gamma is not None:
        y = y * _f64(gamma)
    return y


def decode_e4m3fn(codes):
    """Decode OCP FP8 E4M3 ("fn": finite, no infinities) codes to float64.

    Bit layout s eeee mmm, exponent bias 7.  e == 0 is subnormal:
    (-1)^s * 2^-6 * m/8.  Otherwise (-1)^s * 2^(e-7) * (1 + m/8), except
    e == 15, m == 7, which is NaN.  Written from the format's definition; the
    per-expert FP8 checkpoints on the sglang PR page store weights this way with
    a separate weight_scale."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    val = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, val)


def decode_e2m1(codes):
    """Decode FP4 E2M1 codes (low 4 bits) to float64: bit 3 sign, bits 2-1
    exponent (bias 1), bit 0 mantissa; exponent 0 is subnormal, m * 2^-1;
    otherwise 2^(e-1) * (1 + m/2).  No infinities or NaN.  Written from the
    format's definition (OCP microscaling formats, the element type of MXFP4)."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where(s == 1, -mag, mag)


def decode_e8m0(codes):
    """Decode E8M0 scale codes: 2^(c - 127), c = 255 is NaN (the MX block scale)."""
    c = np.asarray(codes).astype(np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


def decode_mxfp4(packed, scales):
    """MXFP4 weights to float64.  packed [..., K/2] uint8 holds two E2M1 codes per
    byte, element 2i in the low nibble and 2i+1 in the high nibble; scales
    [..., K/32] uint8 holds one E8M0 scale per block of 32 consecutive elements
    along K (readings: the pages name 4-bit expert weights, not a format; MXFP4
    is the 4-bit format with hardware support on the target, and K, the
    reduction dimension, is the blocked one, as for the activations' rows)."""
    packed = np.asarray(packed).astype(np.int64)
    lo, hi = packed & 0xF, packed >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(packed.shape[:-1] + (2 * packed.shape[-1],))
    vals = decode_e2m1(codes)
    sc = decode_e8m0(scales)
    return vals * np.repeat(sc, 32, axis=-1)


def _e4m3fn_values():
    """The 127 non-negative finite E4M3 values, by code 0..126, ascending."""
    return decode_e4m3fn(np.arange(127, dtype=np.uint8))


def encode_e4m3fn(x):
    """Nearest OCP E4M3 ("fn") code of each float32 value, ties to the even code
    (the one whose last mantissa bit is 0), magnitudes beyond 448 saturating to
    448, the sign kept (negative values that round to zero give -0).  Written
    from the format's definition: a search over the ascending table of the
    representable magnitudes."""
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("values to encode must be finite")
    vals = _e4m3fn_values()
    mag = np.minimum(np.abs(x).astype(np.float64), vals[-1])
    hi = np.clip(np.searchsorted(vals, mag, side="left"), 0, 126)  # first value >= mag
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = mag - vals[lo], vals[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)  # -0 for negatives rounding to 0


def quantize_rows_fp8(a):
    """Dynamic per-row FP8 quantisation of an activation matrix, the scheme of
    the "FP8-Dynamic" checkpoints named on the sglang PR page (activations
    quantised at run time, one scale per token row).

    Readings (the page names the scheme, not its arithmetic): scale = the row's
    largest magnitude / 448 (the largest E4M3 value), 1 for an all-zero row;
    code = nearest E4M3 of value / scale.  Both steps in float32, the precision
    the kernel takes these decisions in, so that the codes are a function of
    the float32 inputs alone.  Returns (codes uint8 [R, C], scales float32 [R])."""
    a = np.asarray(a, dtype=np.float32)
    amax = np.abs(a).max(axis=-1)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    scale = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    codes = encode_e4m3fn((a / scale[:, None]).astype(np.float32))
    return codes, scale


def fp8_roundtrip_rows(a):
    """The activation a GEMM sees after dynamic FP8 quantisation: codes x scale."""
    codes, scale = quantize_rows_fp8(a)
    return decode_e4m3fn(codes) * scale.astype(np.float64)[:, None]


def round_bf16(a):
    """Round float64 values to the nearest bfloat16 (ties to even), returned as
    float64: the storage precision of the gated intermediate in the bf16 layer."""
    f = np.asarray(a, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# Router (Gemma 4 walkthrough §3; vLLM Gemma4Router.forward)
# ----------------------------------------------------------------------------

def router_input(x, mode="plain", router_scale=None, eps=RMS_EPS):
    """What the router projection sees.

    plain (Mixtral / DeepSeek / llama.cpp lesson 35): the token vector itself.
    gemma: RMSNorm without gamma, times hidden_size**-0.5, times the learned
    per-dimension scale (ones when None)."""
    x = _f64(x)
    if mode == "plain":
        return x
    if mode != "gemma":
        raise ValueError(f"unknown router mode {mode!r}")
    H = x.shape[-1]
    r = rmsnorm(x, None, eps) * (H ** -0.5)
    if router_scale is not None:
        r = r * _f64(router_scale)
    return r


def router_logits(x, w_router, mode="plain", router_scale=None, eps=RMS_EPS):
    """Router logits z = r . W_r^T, shape [T, E] (GateLinear, fp32 output on the
    pages; float64 here)."""
    r = router_input(x, mode, router_scale, eps)
    return r @ _f64(w_router).T


# ----------------------------------------------------------------------------
# Routing maths (Gemma 4 walkthrough §4-§5; vLLM Gemma4MoE routing function)
# ----------------------------------------------------------------------------

def select_topk(z, k, allowed=None):
    """Indices of the k largest logits per row, largest first.

    Selection is on the logits, not on probabilities (§4: top-k only touches
    the raw logits).  Slot order is descending value, as in the worked example
    whose ids come out as [3, 2].  Reading for ties (unstated on the pages):
    the lower expert index wins, and -0.0 equals +0.0.  A stable argsort of -z
    gives exactly that order.

    `allowed` (bool [T, E], optional) restricts the candidates of each row
    (group-limited routing); each row must allow at least k experts."""
    z = _f64(z)
    if not np.all(np.isfinite(z)):
        raise ValueError("router logits must be finite")
    E = z.shape[-1]
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    if allowed is None:
        return np.argsort(-z, axis=-1, kind="stable")[..., :k]
    allowed = np.asarray(allowed, dtype=bool)
    if np.any(allowed.sum(axis=-1) < k):
        raise ValueError("fewer than k experts allowed")
    # masked experts sort after every allowed one; the stable sort keeps index order
    return np.argsort(np.where(allowed, -z, np.inf), axis=-1, kind="stable")[..., :k]


def softmax_all(z):
    """Softmax over ALL experts (§4 step 2): exp(z - max) / sum exp(z - max)."""
    z = _f64(z)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def sigmoid_scores(z):
    """Sigmoid scoring, 1 / (1 + exp(-z)) per expert, each independent of the
    others (llama.cpp lesson 35: some models turn the router scores into
    probabilities with a sigmoid in place of the softmax)."""
    z = _f64(z)
    return 1.0 / (1.0 + np.exp(-z))


def group_mask(z, n_groups, topk_groups):
    """Experts each token may select under group-limited routing (llama.cpp
    lesson 35: with very many experts they are split into groups; a token first
    picks groups, then its experts inside the picked groups).

    Readings (the page names the two counts, n_expert_groups and n_group_used,
    and nothing more): the groups are n_groups equal, contiguous ranges of
    expert ids; a group's score is the largest logit among its experts (the
    same group order as the largest probability, since both scorings are
    increasing); the topk_groups groups with the largest scores are picked,
    ties to the lower group index.  Returns bool [T, E]."""
    z = _f64(z)
    T, E = z.shape
    if n_groups < 1 or E % n_groups:
        raise ValueError("n_groups must divide E")
    if not 1 <= topk_groups <= n_groups:
        raise ValueError("need 1 <= topk_groups <= n_groups")
    gsz = E // n_groups
    gscore = z.reshape(T, n_groups, gsz).max(axis=-1)
    picked = np.argsort(-gscore, axis=-1, kind="stable")[:, :topk_groups]
    gallowed = np.zeros((T, n_groups), dtype=bool)
    np.put_along_axis(gallowed, picked, True, axis=-1)
    return np.repeat(gallowed, gsz, axis=-1)


def route(z, k, renormalize=True, per_expert_scale=None, scoring="softmax", n_groups=1,
          topk_groups=1):
    """Routing weights and ids, in the order of §4-§5:

    1. ids = top-k of the logits (with n_groups > 1: among the experts of the
       picked groups, see group_mask);
    2. p = softmax over all E, or the per-expert sigmoid (scoring="sigmoid");
    3. indicator [T, E] with exactly k ones per row;
    4. gate = indicator * p;
    5. renormalise by the row sum (a non-positive sum is replaced by 1);
       without renormalisation (DeepSeek-style reading) gate is used as is;
    6. gather the k selected weights in slot order;
    7. multiply by per_expert_scale[ids] (ones when None).

    Both scorings are strictly increasing in the logit, so selecting on the
    logits selects the k largest probabilities (llama.cpp lesson 35 sorts the
    probabilities; the Gemma walkthrough §4 the logits).

    Returns (weights [T, k] float64, ids [T, k] int64)."""
    z = _f64(z)
    T, E = z.shape
    if scoring not in ("softmax", "sigmoid"):
        raise ValueError(f"unknown scoring {scoring!r}")
    allowed = group_mask(z, n_groups, topk_groups) if n_groups > 1 else None
    ids = select_topk(z, k, allowed)
    p = softmax_all(z) if scoring == "softmax" else sigmoid_scores(z)
    indicator = np.zeros((T, E))
    np.put_along_axis(indicator, ids, 1.0, axis=-1)
    gate = indicator * p
    if renormalize:
        s = gate.sum(axis=-1, keepdims=True)
        s = np.where(s > 0.0, s, 1.0)
        gate = gate / s
    w = np.take_along_axis(gate, ids, axis=-1)
    if per_expert_scale is not None:
        w = w * _f64(per_expert_scale)[ids]
    return w, ids


# ----------------------------------------------------------------------------
# Dispatch (Gemma 4 walkthrough §6-§7: a permutation map, no token copies)
# ----------------------------------------------------------------------------

def permutation(ids, E):
    """Expert-major ordering of the T*k (token, slot) pairs.

    Canonical form (reading): experts ascending; inside one expert, flat slot
    index f = t*k + j ascending.  Returns (counts [E], offsets [E+1],
    order [T*k]) where order lists flat slot indices."""
    flat = np.asarray(ids).reshape(-1)
    counts = np.zeros(E, dtype=np.int64)
    buckets = [[] for _ in range(E)]
    for f, e in enumerate(flat.tolist()):
        if not 0 <= e < E:
            raise ValueError("expert id out of range")
        counts[e] += 1
        buckets[e].append(f)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    order = np.array([f for b in buckets for f in b], dtype=np.int64)
    return counts, offsets, order


# ----------------------------------------------------------------------------
# Expert FFN ("MOE Inference" gated FFN; Gemma 4 walkthrough §6)
# ----------------------------------------------------------------------------

def gated_ffn(xrows, w13, w2, act, act_quant=None, h_fp8=None):
    """(Act(x w1) * (x w3)) w2 for a block of rows.

    w13 has shape [2I, H]: rows [0, I) are the gate projection w1, rows
    [I, 2I) the up projection w3 (vLLM load_weights: gate_proj is shard w1,
    up_proj shard w3, both [I, H]); w2 has shape [H, I] (down_proj).

    act_quant="fp8_dynamic": each projection's input rows are quantised as in
    quantize_rows_fp8 first: x before gate/up, and h, as stored (rounded to
    bf16), before the down projection.  h_fp8 = (codes [n, I] uint8, scales
    [n] float32), when given, are the quantised h rows to project instead of
    this function's own quantisation of h: the codes are integers that
    floating point decides, so parity checks them as it checks top-k ids, on
    the other side's own h, and takes them as given for the rest of the layer
    (as routing parity takes the logits)."""
    xrows = _f64(xrows)
    w13 = _f64(w13)
    I = w13.shape[0] // 2
    if act_quant == "fp8_dynamic":
        xrows = fp8_roundtrip_rows(xrows)
    elif act_quant is not None:
        raise ValueError(f"unknown activation quantisation {act_quant!r}")
    g = xrows @ w13[:I].T
    u = xrows @ w13[I:].T
    h = activation(act)(g) * u
    if act_quant == "fp8_dynamic":
        if h_fp8 is None:
            h = fp8_roundtrip_rows(round_bf16(h))
        else:
            codes, scales = h_fp8
            h = decode_e4m3fn(codes) * np.asarray(scales, dtype=np.float32).astype(np.float64)[:, None]
    elif h_fp8 is not None:
        raise ValueError("h_fp8 needs act_quant='fp8_dynamic'")
    return h @ _f64(w2).T


def moe_combine(xe, weights, ids, w13, w2, act, rows=None, w13_scale=None, w2_scale=None,
                act_quant=None, h_fp8=None):
    """Sparse MoE output for the selected rows: out_t = sum_j w[t,j] * FFN_{ids[t,j]}(xe_t).

    Only the selected experts are evaluated (llama.cpp lesson 35: mul_mat_id
    touches only the chosen experts); the result equals computing every expert
    and masking (checked by brute force in the tests).  The k expert outputs of
    a token are summed in slot order.  Rows of one expert are evaluated
    together (a matmul per expert) to bound memory; each (t, j) output is
    independent of the grouping.

    w13 / w2 are indexable per expert (array [E, 2I, H] / [E, H, I], any real
    dtype holding the exact stored values, or FP8 codes with per-output-channel
    scales w13_scale [E, 2I] and w2_scale [E, H]: W = decode(q) * s[n], or MXFP4:
    packed codes [E, 2I, H/2] / [E, H, I/2] with uint8 E8M0 block scales
    [E, 2I, H/32] / [E, H, I/32]).

    h_fp8 = (codes [T, k, I] uint8, scales [T, k] float32): quantised expert
    intermediates per (token, slot) to use instead of the oracle's own (see
    gated_ffn); FP8 activations only."""
    xe = _f64(xe)
    weights = _f64(weights)
    ids = np.asarray(ids)
    T, k = ids.shape
    rows = np.arange(T) if rows is None else np.asarray(rows)
    H = xe.shape[1]
    y = np.zeros((len(rows), k, H))
    sel_ids = ids[rows]
    for e in np.unique(sel_ids):
        ri, ji = np.nonzero(sel_ids == e)
        if len(ri) == 0:
            continue
        W13 = _expert_weight(w13, w13_scale, e)
        W2 = _expert_weight(w2, w2_scale, e)
        hq = None if h_fp8 is None else (h_fp8[0][rows[ri], ji], h_fp8[1][rows[ri], ji])
        y[ri, ji] = gated_ffn(xe[rows[ri]], W13, W2, act, act_quant, hq)
    out = np.zeros((len(rows), H))
    for j in range(k):  # slot order
        out += weights[rows, j][:, None] * y[:, j]
    return out


def _expert_weight(w, scale, e):
    if scale is None:
        return _f64(w[e])
    if np.asarray(scale).dtype == np.uint8:  # MXFP4: packed codes, E8M0 block scales
        return decode_mxfp4(w[e], scale[e])
    return decode_e4m3fn(w[e]) * _f64(scale[e])[:, None]


# ----------------------------------------------------------------------------
# The whole layer
# ----------------------------------------------------------------------------

def moe_layer(x, layer, rows=None, logits=None, h_fp8=None):
    """The MoE FFN layer forward for token rows `rows` (all when None).

    `layer` is a dict with:
      E, K, act, renorm, router_mode ('plain'|'gemma'),
      scoring ('softmax'|'sigmoid'), n_groups, topk_groups (group-limited routing),
      act_quant (None | 'fp8_dynamic': routed experts' inputs quantised per row),
      block_tail (True: the FFN block's tail, post_feedforward_layernorm with weight
      gamma_post_ff (ones when None) and the residual add),
      w_router [E,H] or None (then `logits` must be given),
      router_scale [H] or None, per_expert_scale [E] or None,
      w13 [E,2I,H], w2 [E,H,I] (+ w13_scale [E,2I], w2_scale [E,H] for FP8 codes),
      shared: None or (w13 [S,2Is,H], w2 [S,H,Is])   - always-on experts, weight 1,
      dense: None or dict(w13 [2Id,H], w2 [H,Id], gamma_pre, gamma_pre2,
             gamma_post1, gamma_post2)               - Gemma parallel branch,
      eps.

    Steps (Gemma 4 walkthrough §1, §3-§7; llama.cpp lesson 35):
      z      = router logits (supplied, or computed from x)
      w, ids = route(z)
      xe     = pre_feedforward_layernorm_2(x) when the Gemma dense branch is
               present, else x
      moe    = sum_j w_j FFN_{ids_j}(xe)
      shared experts: out = moe + sum_s FFN_s(x)            (DeepSeek reading)
      Gemma: out = post_norm_1(MLP(pre_norm(x))) + post_norm_2(moe)
      others: out = moe
    The decoder layer's final post_feedforward_layernorm and residual add are
    outside the FFN layer (reading) unless block_tail asks for them:
      out = x + post_feedforward_layernorm(out).

    h_fp8 (FP8 activations only): quantised expert intermediates (codes
    [T, K, I] uint8, scales [T, K] float32) taken as given, like `logits`; see
    gated_ffn.

    Returns dict(out [len(rows),H], logits [T,E], weights [T,K], ids [T,K],
    counts [E], offsets [E+1], order [T*K])."""
    x = _f64(x)
    T, H = x.shape
    E, K = layer["E"], layer["K"]
    eps = layer.get("eps", RMS_EPS)
    rows = np.arange(T) if rows is None else np.asarray(rows)
    if logits is None:
        logits = router_logits(x, layer["w_router"], layer.get("router_mode", "plain"),
                               layer.get("router_scale"), eps)
    z = _f64(logits)
    w, ids = route(z, K, layer.get("renorm", True), layer.get("per_expert_scale"),
                   layer.get("scoring", "softmax"), layer.get("n_groups", 1),
                   layer.get("topk_groups", 1))
    counts, offsets, order = permutation(ids, E)
    dense = layer.get("dense")
    if dense is not None:
        xe = rmsnorm(x, dense.get("gamma_pre2"), eps)
        if layer.get("act_quant"):
            # reading: the normalised expert input is stored (bf16) and quantised as stored
            xe = round_bf16(xe)
    else:
        xe = x
    moe = moe_combine(xe, w, ids, layer["w13"], layer["w2"], layer["act"], rows,
                      layer.get("w13_scale"), layer.get("w2_scale"), layer.get("act_quant"), h_fp8)
    shared = layer.get("shared")
    if shared is not None:
        sw13, sw2 = shared
        for s in range(len(sw13)):
            moe = moe + gated_ffn(x[rows], sw13[s], sw2[s], layer["act"])
    if dense is not None:
        d = gated_ffn(rmsnorm(x[rows], dense.get("gamma_pre"), eps), dense["w13"], dense["w2"],
                      layer.get("dense_act", layer["act"]))
        out = rmsnorm(d, dense.get("gamma_post1"), eps) + rmsnorm(moe, dense.get("gamma_post2"), eps)
    else:
        out = moe
    if layer.get("block_tail"):
        # the rest of the FFN block (Gemma 4 walkthrough §1): post_feedforward_layernorm
        # of the merged branches, then the residual add (the layer input is the residual)
        out = x[rows] + rmsnorm(out, layer.get("gamma_post_ff"), eps)
    return dict(out=out, logits=z, weights=w, ids=ids, counts=counts, offsets=offsets,
                order=order)
