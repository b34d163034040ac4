"""Seeded synthetic MoE layers, shaped like the models the pages discuss.

This module only draws random numbers and stores them in the dtypes the
layer consumes; it holds none of the layer's arithmetic.  Tests hand the same
tensors to the HIP library and (widened exactly to float64) to the oracle.

Every tensor comes from its own numpy stream, keyed by (seed, tensor id,
expert), so a tensor does not change when the token count T or another tensor
changes, and weight sets can be drawn per expert in parallel threads.

Distributions: x ~ N(0, 1); every projection ~ N(0, 1/fan_in) (fan_in = H for
router, gate/up and shared/dense gate/up; fan_in = I for down projections).
bf16 tensors are the float32 draws rounded to nearest even; FP8 weights are
q = RNE(w / s) in OCP E4M3 with s[e, n] = max_k |w[e, n, k]| / 448 per expert
and output channel.  Skewed routing supplies logits N(0, 1) + b_e with a Zipf
bias b_e = -alpha * 1.2 * ln(rank_e) over a seeded rank permutation.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import math
from typing import Optional

import numpy as np
import torch

# Zipf bias amplitude: the value for which the 13 most-loaded of 128 experts
# (about 10%) take about 60% of the top-8 assignments at T = 4096, seed 0.
# Found by bisection with oracle/calibrate_zipf.py; checked by a CPU test.
ZIPF_S = 1.2
ZIPF_ALPHA = 0.6107177734375

_TID = dict(x=1, w_router=2, w13=3, w2=4, per_expert_scale=5, shared_w13=6, shared_w2=7,
            dense_w13=8, dense_w2=9, router_scale=10, zipf_rank=11, logit_noise=12,
            gammas=13)


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    name: str
    T: int
    H: int
    E: int
    K: int
    I: int
    act: str                     # "silu" | "gelu_tanh"
    wdtype: str                  # "fp32" | "bf16" | "fp8" | "mxfp4" (decode path only)
    renorm: bool = True
    router_mode: str = "plain"   # "plain" | "gemma"
    per_expert_scale: str = "ones"   # "ones" | "uniform"
    n_shared: int = 0
    I_shared: int = 0
    I_dense: int = 0             # > 0: Gemma-style parallel dense MLP with post-norms
    supplied_logits: bool = False    # True: logits N(0,1) + Zipf bias, no router weights
    random_gammas: bool = False      # test-only: non-unit norm / router scales
    scoring: str = "softmax"     # "softmax" over all experts | "sigmoid" per expert
    n_groups: int = 0            # > 1: group-limited routing over this many expert groups
    topk_groups: int = 0         # groups picked per token when n_groups > 1
    act_quant: Optional[str] = None  # "fp8_dynamic": FP8 activations (needs FP8 weights)
    block_tail: bool = False     # the FFN block's post_feedforward_layernorm and residual add

    def with_T(self, T):
        return dataclasses.replace(self, T=T)

    @property
    def act_dtype(self):
        return "fp32" if self.wdtype == "fp32" else "bf16"


SPECS = {
    "tiny": LayerSpec("tiny", 64, 256, 8, 2, 512, "silu", "fp32"),
    "mixtral": LayerSpec("mixtral", 4096, 4096, 8, 2, 14336, "silu", "bf16"),
    "gemma": LayerSpec("gemma", 8192, 2816, 128, 8, 704, "gelu_tanh", "bf16",
                       router_mode="gemma", per_expert_scale="uniform", I_dense=2112),
    "deepseek": LayerSpec("deepseek", 16384, 2048, 64, 6, 1408, "silu", "bf16",
                          renorm=False, n_shared=2, I_shared=1408),
    "skewed_fp8": LayerSpec("skewed_fp8", 4096, 2816, 128, 8, 704, "gelu_tanh", "fp8",
                            supplied_logits=True),
    # DeepSeek-V3 routing shape (256 routed experts + 1 shared, 8 per token) with sigmoid
    # scoring and expert groups, on the DeepSeek-MoE layer's hidden and expert widths
    "deepseek_v3": LayerSpec("deepseek_v3", 8192, 2048, 256, 8, 1408, "silu", "bf16",
                             n_shared=1, I_shared=1408, scoring="sigmoid", n_groups=8,
                             topk_groups=4),
    # 4-bit (MXFP4) expert weights for decode bandwidth: the Gemma and Mixtral layers
    "gemma_mxfp4": LayerSpec("gemma_mxfp4", 1, 2816, 128, 8, 704, "gelu_tanh", "mxfp4",
                             router_mode="gemma", per_expert_scale="uniform", I_dense=2112),
    "mixtral_mxfp4": LayerSpec("mixtral_mxfp4", 1, 4096, 8, 2, 14336, "silu", "mxfp4"),
    # the whole Gemma FFN block: the layer plus post_feedforward_layernorm and the residual add
    "gemma_block": LayerSpec("gemma_block", 8192, 2816, 128, 8, 704, "gelu_tanh", "bf16",
                             router_mode="gemma", per_expert_scale="uniform", I_dense=2112,
                             block_tail=True),
    # FP8 weights and dynamically quantised FP8 activations (W8A8)
    "mixtral_w8a8": LayerSpec("mixtral_w8a8", 4096, 4096, 8, 2, 14336, "silu", "fp8",
                              act_quant="fp8_dynamic"),
    "skewed_w8a8": LayerSpec("skewed_w8a8", 4096, 2816, 128, 8, 704, "gelu_tanh", "fp8",
                             supplied_logits=True, act_quant="fp8_dynamic"),
    # the Gemma layer as an FP8-Dynamic checkpoint runs it: FP8 experts with FP8
    # activations, the dense MLP in bf16
    "gemma_w8a8": LayerSpec("gemma_w8a8", 8192, 2816, 128, 8, 704, "gelu_tanh", "fp8",
                            router_mode="gemma", per_expert_scale="uniform", I_dense=2112,
                            act_quant="fp8_dynamic"),
}

# token counts the pages' configurations name for each layer shape
T_VALUES = {"tiny": [64], "mixtral": [4096], "gemma": [1, 16, 128, 8192],
            "deepseek": [16384], "skewed_fp8": [1, 4096], "deepseek_v3": [1, 16, 8192],
            "mixtral_w8a8": [4096], "skewed_w8a8": [1, 4096], "gemma_block": [1, 8192],
            "gemma_w8a8": [1, 8192], "gemma_mxfp4": [1, 16], "mixtral_mxfp4": [1]}


def _rng(seed, *key):
    return np.random.default_rng(np.random.SeedSequence(entropy=seed, spawn_key=key))


def _normal(seed, tid, shape, std, sub=()):
    a = _rng(seed, tid, *sub).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _per_expert(seed, tid, E, shape, std, threads=8):
    out = np.empty((E,) + tuple(shape), dtype=np.float32)

    def fill(e):
        out[e] = _normal(seed, tid, shape, std, (e,))

    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(fill, range(E)))
    return out


def _store(a, wdtype):
    t = torch.from_numpy(a)
    if wdtype == "fp32":
        return t.contiguous()
    return t.to(torch.bfloat16)


def _fp8(w):
    """Per-output-channel E4M3 quantisation of w [E, N, K] -> (codes uint8, scales fp32 [E, N])."""
    t = torch.from_numpy(w)
    s = t.abs().amax(dim=-1) / 448.0
    s = torch.where(s > 0, s, torch.ones_like(s))
    q = (t / s[..., None]).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), s.to(torch.float32)


_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _mxfp4(w):
    """MXFP4 quantisation of w [E, N, K] along K in blocks of 32: the block scale is
    2^(floor(log2(max|block|)) - 2) (2 = the exponent of E2M1's largest power of two),
    stored as E8M0 (exponent + 127); each element is the nearest E2M1 value of
    w / scale, ties to the even code, saturating at 6.  Returns (packed codes uint8
    [E, N, K/2], element 2i in the low nibble; scales uint8 [E, N, K/32])."""
    E, N, K = w.shape
    b = w.reshape(E, N, K // 32, 32).astype(np.float64)
    amax = np.abs(b).max(axis=-1)
    ex = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
    ex = np.clip(ex, -127, 127).astype(np.int64)
    v = np.abs(b) / np.ldexp(1.0, ex)[..., None]
    v = np.minimum(v, 6.0)
    hi = np.clip(np.searchsorted(_E2M1_GRID, v, side="left"), 0, 7)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = v - _E2M1_GRID[lo], _E2M1_GRID[hi] - v
    idx = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)), hi, lo)
    codes = (idx | np.where(np.signbit(b), 8, 0)).astype(np.uint8).reshape(E, N, K)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return torch.from_numpy(packed), torch.from_numpy((ex + 127).astype(np.uint8))


def zipf_bias(E, seed=0, alpha=ZIPF_ALPHA, s=ZIPF_S):
    ranks = _rng(seed, _TID["zipf_rank"]).permutation(E) + 1
    return (-alpha * s * np.log(ranks)).astype(np.float32)


def make_layer(spec: LayerSpec, seed: int = 0, T: Optional[int] = None, x_only=False):
    """Draw one layer.  Returns a dict of CPU torch tensors in storage dtypes:

    x [T,H] (fp32 or bf16); w_router [E,H] or None; logits [T,E] fp32 or None;
    router_scale [H] fp32 or None; per_expert_scale [E] fp32 or None;
    w13 [E,2I,H], w2 [E,H,I] (bf16 / fp32, or uint8 E4M3 codes with
    w13_scale [E,2I], w2_scale [E,H] fp32); shared_w13 [S,2Is,H],
    shared_w2 [S,H,Is] or None; dense_w13 [2Id,H], dense_w2 [H,Id] or None;
    gammas dict (pre, pre2, post1, post2) of [H] fp32 or None (= ones).
    """
    T = spec.T if T is None else T
    H, E, I = spec.H, spec.E, spec.I
    wd = "fp32" if spec.wdtype == "fp32" else "bf16"
    L = dict(spec=spec, T=T)
    L["x"] = _store(_normal(seed, _TID["x"], (T, H), 1.0), wd)
    if x_only:
        return L
    if spec.supplied_logits:
        L["w_router"] = None
    else:
        L["w_router"] = _store(_normal(seed, _TID["w_router"], (E, H), H ** -0.5), wd)
    w13 = _per_expert(seed, _TID["w13"], E, (2 * I, H), H ** -0.5)
    w2 = _per_expert(seed, _TID["w2"], E, (H, I), I ** -0.5)
    if spec.wdtype == "fp8":
        L["w13"], L["w13_scale"] = _fp8(w13)
        L["w2"], L["w2_scale"] = _fp8(w2)
    elif spec.wdtype == "mxfp4":
        L["w13"], L["w13_scale"] = _mxfp4(w13)
        L["w2"], L["w2_scale"] = _mxfp4(w2)
    else:
        L["w13"], L["w2"] = _store(w13, wd), _store(w2, wd)
        L["w13_scale"] = L["w2_scale"] = None
    del w13, w2
    if spec.per_expert_scale == "uniform":
        L["per_expert_scale"] = torch.from_numpy(
            _rng(seed, _TID["per_expert_scale"]).uniform(0.5, 1.5, E).astype(np.float32))
    else:
        L["per_expert_scale"] = None
    if spec.n_shared:
        Is = spec.I_shared
        L["shared_w13"] = _store(_per_expert(seed, _TID["shared_w13"], spec.n_shared,
                                             (2 * Is, H), H ** -0.5), wd)
        L["shared_w2"] = _store(_per_expert(seed, _TID["shared_w2"], spec.n_shared,
                                            (H, Is), Is ** -0.5), wd)
    else:
        L["shared_w13"] = L["shared_w2"] = None
    if spec.I_dense:
        Id = spec.I_dense
        L["dense_w13"] = _store(_normal(seed, _TID["dense_w13"], (2 * Id, H), H ** -0.5), wd)
        L["dense_w2"] = _store(_normal(seed, _TID["dense_w2"], (H, Id), Id ** -0.5), wd)
    else:
        L["dense_w13"] = L["dense_w2"] = None
    if spec.random_gammas:
        # test-only learned weights: router scale and input norms around 1; the
        # post-norm weights below 1 keep the output near unit scale
        g = _rng(seed, _TID["gammas"]).uniform(0.5, 1.5, (6, H)).astype(np.float32)
        g[3:] = (g[3:] - 0.5) * 0.4 + 0.3
        L["router_scale"] = torch.from_numpy(g[0].copy()) if spec.router_mode == "gemma" else None
        L["gammas"] = {k: torch.from_numpy(g[i + 1].copy())
                       for i, k in enumerate(["pre", "pre2", "post1", "post2", "post_ff"])}
    else:
        L["router_scale"] = None
        L["gammas"] = None
    if spec.supplied_logits:
        noise = _normal(seed, _TID["logit_noise"], (T, E), 1.0)
        L["logits"] = torch.from_numpy(noise + zipf_bias(E, seed)[None, :])
    else:
        L["logits"] = None
    return L


def oracle_layer(L):
    """The same layer as plain float64 numpy arrays in the oracle's dict form.
    Weights are widened lazily per expert by the oracle; here bf16 tensors are
    exposed as float32 views of their exact values."""
    spec = L["spec"]

    def f(t):
        if t is None:
            return None
        if t.dtype == torch.uint8:
            return t.numpy()
        return t.float().numpy()

    d = dict(E=spec.E, K=spec.K, act=spec.act, renorm=spec.renorm,
             scoring=spec.scoring, n_groups=max(spec.n_groups, 1),
             topk_groups=max(spec.topk_groups, 1), act_quant=spec.act_quant,
             router_mode=spec.router_mode, w_router=f(L["w_router"]),
             router_scale=f(L["router_scale"]), per_expert_scale=f(L["per_expert_scale"]),
             w13=f(L["w13"]), w2=f(L["w2"]), w13_scale=f(L["w13_scale"]),
             w2_scale=f(L["w2_scale"]))
    d["shared"] = None if L["shared_w13"] is None else (f(L["shared_w13"]), f(L["shared_w2"]))
    d["block_tail"] = spec.block_tail
    d["gamma_post_ff"] = f((L["gammas"] or {}).get("post_ff"))
    if L["dense_w13"] is not None:
        g = L["gammas"] or {}
        d["dense"] = dict(w13=f(L["dense_w13"]), w2=f(L["dense_w2"]),
                          gamma_pre=f(g.get("pre")), gamma_pre2=f(g.get("pre2")),
                          gamma_post1=f(g.get("post1")), gamma_post2=f(g.get("post2")))
    else:
        d["dense"] = None
    return d


def param_counts(spec: LayerSpec):
    """Parameter counts of one layer (3*H*I per gated FFN)."""
    per_expert = 3 * spec.H * spec.I
    dense = 3 * spec.H * spec.I_dense
    shared = spec.n_shared * 3 * spec.H * spec.I_shared
    return dict(per_expert=per_expert, experts=spec.E * per_expert, dense=dense,
                shared=shared, router=spec.E * spec.H)
