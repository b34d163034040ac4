"""Pins the CPU oracle to facts fixed by the pages and by mathematics.

None of these re-types the oracle's own formula: each compares it with a value
the pages print, a closed form the pages derive, an invariant they state, a
brute-force evaluation through torch.nn.functional in float64, or a library
routine (scipy softmax, numpy stable argsort, torch's float8_e4m3fn).
"""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

from oracle import moe_oracle as O
from mixture_experts_ffn_router_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    d = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, *v = line.split()
            d[k] = [float(t) for t in v]
    return d


# --------------------------------------------------------------------------- routing

def test_worked_example_from_page():
    g = _golden("routing_worked_example.txt")
    z = np.array([g["logits"]])
    k = int(g["k"][0])
    p = O.softmax_all(z)[0]
    np.testing.assert_allclose(p, g["softmax_all"], atol=5e-5)
    w, ids = O.route(z, k, renormalize=True)
    assert ids[0].tolist() == [int(v) for v in g["ids"]]
    np.testing.assert_allclose(p[ids[0]].sum(), g["renorm_divisor"][0], atol=5e-5)
    np.testing.assert_allclose(w[0], g["weights"], atol=5e-4)


def _rand_logits(rng, T, E, ties=False):
    z = rng.standard_normal((T, E))
    if ties:
        z = np.round(z * 2) / 2  # many exact ties
        z[z == 0] = -0.0
        z[::3] = 0.0
    return z


@pytest.mark.parametrize("E,k", [(8, 2), (128, 8), (64, 6), (5, 5)])
def test_closed_form_softmax_over_selected(E, k):
    """Renormalised weights equal the softmax over the selected logits alone."""
    rng = np.random.default_rng(1)
    z = _rand_logits(rng, 200, E) * 3
    w, ids = O.route(z, k, renormalize=True)
    zs = np.take_along_axis(z, ids, axis=-1)
    np.testing.assert_allclose(w, scipy.special.softmax(zs, axis=-1), rtol=1e-13, atol=0)


@pytest.mark.parametrize("E,k", [(8, 2), (64, 6)])
def test_no_renorm_is_full_softmax_gathered(E, k):
    rng = np.random.default_rng(2)
    z = _rand_logits(rng, 100, E) * 2
    w, ids = O.route(z, k, renormalize=False)
    p = scipy.special.softmax(z, axis=-1)
    np.testing.assert_allclose(w, np.take_along_axis(p, ids, axis=-1), rtol=1e-13, atol=0)


@pytest.mark.parametrize("E,k", [(8, 2), (128, 8), (3, 3)])
def test_weights_sum_to_one_and_ids_distinct(E, k):
    rng = np.random.default_rng(3)
    z = _rand_logits(rng, 300, E, ties=True)
    w, ids = O.route(z, k, renormalize=True)
    np.testing.assert_allclose(w.sum(axis=-1), 1.0, rtol=1e-14)
    for row in ids:
        assert len(set(row.tolist())) == k
    # the indicator has exactly k ones per row
    ind = np.zeros_like(z)
    np.put_along_axis(ind, ids, 1.0, axis=-1)
    assert (ind.sum(axis=-1) == k).all()


def test_topk_brute_force_with_ties_and_signed_zero():
    """Brute force: Python sorted with key (-value, index) on tiny rows."""
    rng = np.random.default_rng(4)
    z = _rand_logits(rng, 500, 9, ties=True)
    z[0] = [0.0, -0.0, 0.0, -0.0, 1.0, 1.0, -1.0, 0.0, -0.0]
    for k in (1, 3, 9):
        ids = O.select_topk(z, k)
        for r in range(z.shape[0]):
            ref = sorted(range(9), key=lambda e: (-float(z[r, e]) + 0.0, e))[:k]
            assert ids[r].tolist() == ref
    assert O.select_topk(z[:1], 4)[0].tolist() == [4, 5, 0, 1]


# ------------------------------------------------------------ routing variants (llama.cpp lesson 35)

def test_sigmoid_scores_match_library_and_closed_forms():
    rng = np.random.default_rng(20)
    z = rng.standard_normal((50, 16)) * 6
    np.testing.assert_allclose(O.sigmoid_scores(z), scipy.special.expit(z), rtol=1e-15, atol=0)
    assert O.sigmoid_scores(np.zeros((1, 1)))[0, 0] == 0.5
    np.testing.assert_allclose(O.sigmoid_scores(-z), 1.0 - O.sigmoid_scores(z), atol=1e-15)


@pytest.mark.parametrize("renorm", [True, False])
def test_sigmoid_route_sorts_probabilities(renorm):
    """The page's order of operations, through torch: probabilities first
    (torch.sigmoid), a stable descending sort of them, gather, L1-normalise."""
    rng = np.random.default_rng(21)
    z = rng.standard_normal((300, 64)) * 2
    K = 6
    w, ids = O.route(z, K, renormalize=renorm, scoring="sigmoid")
    p = torch.sigmoid(torch.from_numpy(z))
    order = torch.sort(p, dim=-1, descending=True, stable=True).indices[:, :K]
    assert np.array_equal(ids, order.numpy())
    g = torch.gather(p, 1, order)
    if renorm:
        g = F.normalize(g, p=1, dim=-1)
    np.testing.assert_allclose(w, g.numpy(), rtol=1e-13, atol=0)


def _brute_groups(zrow, G, KG):
    """The KG groups whose best logits have the largest sum, over every
    combination (distinct logits make the set unique)."""
    gsz = len(zrow) // G
    best = [max(zrow[g * gsz:(g + 1) * gsz]) for g in range(G)]
    return set(max(itertools.combinations(range(G), KG), key=lambda c: sum(best[i] for i in c)))


@pytest.mark.parametrize("E,G,KG,K", [(16, 4, 2, 3), (32, 8, 3, 5), (12, 6, 1, 2)])
def test_group_limited_topk_brute_force(E, G, KG, K):
    rng = np.random.default_rng(22)
    z = rng.standard_normal((200, E))
    w, ids = O.route(z, K, True, None, "softmax", G, KG)
    gsz = E // G
    for r in range(z.shape[0]):
        picked = _brute_groups(z[r].tolist(), G, KG)
        cand = [e for e in range(E) if e // gsz in picked]
        assert ids[r].tolist() == sorted(cand, key=lambda e: -z[r, e])[:K]
    # renormalised: the softmax over the selected logits (the full denominator cancels)
    zs = np.take_along_axis(z, ids, axis=-1)
    np.testing.assert_allclose(w, scipy.special.softmax(zs, axis=-1), rtol=1e-13, atol=0)


def test_group_limited_worked_case():
    """Hand-checked.  Groups {0,1} {2,3} {4,5} {6,7} have best logits 5, 4, 4.5, 0;
    groups 0 and 2 are picked, so expert 2 (the third largest logit) is out of
    reach and the third slot goes to expert 1 (tied with expert 5 at -9)."""
    z = np.array([[5.0, -9.0, 4.0, 0.0, 4.5, -9.0, 0.0, 0.0]])
    assert O.route(z, 3, True, None, "softmax", 4, 2)[1][0].tolist() == [0, 4, 1]
    assert O.route(z, 3)[1][0].tolist() == [0, 4, 2]
    # tied group scores (groups 0 and 1 both 1.0): the lower group index is picked
    z = np.array([[1.0, 0.0, 0.0, 1.0, 2.0, 2.0, -1.0, -1.0]])
    assert O.route(z, 4, True, None, "sigmoid", 4, 2)[1][0].tolist() == [4, 5, 0, 1]
    assert O.route(z, 4, True, None, "sigmoid")[1][0].tolist() == [4, 5, 0, 3]


def test_group_limited_reduces_to_plain_topk():
    """One expert per group with k groups picked, or every group picked, is the
    plain top-k (ties included)."""
    rng = np.random.default_rng(23)
    z = _rand_logits(rng, 300, 16, ties=True)
    for G, KG, K in [(16, 4, 4), (4, 4, 3), (8, 8, 8)]:
        for scoring in ("softmax", "sigmoid"):
            a = O.route(z, K, True, None, scoring, G, KG)
            b = O.route(z, K, True, None, scoring)
            assert np.array_equal(a[1], b[1])
            np.testing.assert_array_equal(a[0], b[0])


def test_group_limited_rejects_too_few_candidates():
    z = np.zeros((1, 8))
    with pytest.raises(ValueError):
        O.route(z, 5, True, None, "softmax", 4, 2)  # 2 groups of 2 experts < 5
    with pytest.raises(ValueError):
        O.route(z, 2, True, None, "softmax", 3, 1)  # 3 does not divide 8


def test_nonfinite_logits_rejected():
    z = np.array([[0.0, np.nan, 1.0]])
    with pytest.raises(ValueError):
        O.route(z, 1)


def test_scale_fold_identity():
    """(w s_e) y_e == w (s_e y_e): a per-expert scale on the routing weights
    equals scaling that expert's down projection."""
    rng = np.random.default_rng(5)
    T, H, E, K, I = 16, 32, 6, 3, 24
    x = rng.standard_normal((T, H))
    w13 = rng.standard_normal((E, 2 * I, H)) / math.sqrt(H)
    w2 = rng.standard_normal((E, H, I)) / math.sqrt(I)
    wr = rng.standard_normal((E, H))
    s = rng.uniform(0.5, 1.5, E)
    base = dict(E=E, K=K, act="silu", renorm=True, w_router=wr, w13=w13, w2=w2)
    a = O.moe_layer(x, dict(base, per_expert_scale=s))["out"]
    b = O.moe_layer(x, dict(base, w2=w2 * s[:, None, None]))["out"]
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------- experts

def _torch_ffn(x, w13, w2, act):
    I = w13.shape[0] // 2
    g = F.linear(x, w13[:I])
    u = F.linear(x, w13[I:])
    h = (F.silu(g) if act == "silu" else F.gelu(g, approximate="tanh")) * u
    return F.linear(h, w2)


def _tiny_layer(rng, T, H, E, K, I, act="silu", scale=True):
    return dict(E=E, K=K, act=act, renorm=True,
                w_router=rng.standard_normal((E, H)) / math.sqrt(H),
                w13=rng.standard_normal((E, 2 * I, H)) / math.sqrt(H),
                w2=rng.standard_normal((E, H, I)) / math.sqrt(I),
                per_expert_scale=rng.uniform(0.5, 1.5, E) if scale else None)


def _brute_dispatch(z, K, renorm, scale):
    """Dense [T, E] dispatch matrix by brute force (Python sort, scipy softmax)."""
    T, E = z.shape
    p = scipy.special.softmax(z, axis=-1)
    D = np.zeros((T, E))
    for t in range(T):
        sel = sorted(range(E), key=lambda e: (-z[t, e], e))[:K]
        for e in sel:
            D[t, e] = p[t, e]
        if renorm:
            D[t] /= D[t].sum()
    if scale is not None:
        D = D * scale[None, :]
    return D


@pytest.mark.parametrize("act", ["silu", "gelu_tanh"])
@pytest.mark.parametrize("T,H,E,K,I", [(64, 48, 8, 2, 40), (17, 32, 5, 3, 16)])
def test_brute_force_all_experts_then_mask(T, H, E, K, I, act):
    """Every expert computed densely through torch in float64, then masked by the
    brute-force dispatch matrix (the 'compute all then discard' form of
    llama.cpp lesson 35)."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((T, H))
    L = _tiny_layer(rng, T, H, E, K, I, act)
    got = O.moe_layer(x, L)
    z = x @ L["w_router"].T
    D = _brute_dispatch(z, K, True, L["per_expert_scale"])
    xt = torch.from_numpy(x)
    ref = sum(torch.from_numpy(D[:, e:e + 1]) *
              _torch_ffn(xt, torch.from_numpy(L["w13"][e]), torch.from_numpy(L["w2"][e]), act)
              for e in range(E)).numpy()
    np.testing.assert_allclose(got["out"], ref, rtol=1e-11, atol=1e-12)


def test_k_equals_e_is_probability_weighted_sum():
    """k = E with unit scales: the layer equals sum_e p_e FFN_e(x) (closed form)."""
    rng = np.random.default_rng(7)
    T, H, E, I = 20, 24, 6, 12
    x = rng.standard_normal((T, H))
    L = _tiny_layer(rng, T, H, E, E, I, scale=False)
    got = O.moe_layer(x, L)["out"]
    p = scipy.special.softmax(x @ L["w_router"].T, axis=-1)
    xt = torch.from_numpy(x)
    ref = sum(torch.from_numpy(p[:, e:e + 1]) *
              _torch_ffn(xt, torch.from_numpy(L["w13"][e]), torch.from_numpy(L["w2"][e]), "silu")
              for e in range(E)).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_single_expert_is_plain_gated_mlp():
    rng = np.random.default_rng(8)
    T, H, I = 9, 16, 20
    x = rng.standard_normal((T, H))
    L = _tiny_layer(rng, T, H, 1, 1, I, act="gelu_tanh", scale=False)
    got = O.moe_layer(x, L)["out"]
    ref = _torch_ffn(torch.from_numpy(x), torch.from_numpy(L["w13"][0]),
                     torch.from_numpy(L["w2"][0]), "gelu_tanh").numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_top1_picks_argmax_expert_with_weight_one():
    rng = np.random.default_rng(9)
    T, H, E, I = 12, 16, 4, 8
    x = rng.standard_normal((T, H))
    L = _tiny_layer(rng, T, H, E, 1, I, scale=False)
    got = O.moe_layer(x, L)["out"]
    e_star = np.argmax(x @ L["w_router"].T, axis=-1)
    for t in range(T):
        ref = _torch_ffn(torch.from_numpy(x[t:t + 1]), torch.from_numpy(L["w13"][e_star[t]]),
                         torch.from_numpy(L["w2"][e_star[t]]), "silu").numpy()[0]
        np.testing.assert_allclose(got[t], ref, rtol=1e-12, atol=1e-13)


def test_activations_match_torch():
    a = np.linspace(-12, 12, 4001)
    at = torch.from_numpy(a)
    np.testing.assert_allclose(O.silu(a), F.silu(at).numpy(), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(O.gelu_tanh(a), F.gelu(at, approximate="tanh").numpy(),
                               rtol=1e-14, atol=1e-15)
    with pytest.raises(ValueError):
        O.activation("gelu")


def test_fp8_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.decode_e4m3fn(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_e2m1_and_e8m0_decode_closed_forms():
    """E2M1 (the MXFP4 element) takes exactly the grid 0, 0.5, 1, 1.5, 2, 3, 4, 6 on
    codes 0-7, in order, and its negatives on 8-15; E8M0 is 2^(c-127), 255 is NaN."""
    assert O.decode_e2m1(np.arange(8)).tolist() == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert np.array_equal(O.decode_e2m1(np.arange(8, 16)), -O.decode_e2m1(np.arange(8)))
    assert np.signbit(O.decode_e2m1(8))
    sc = O.decode_e8m0(np.array([0, 1, 126, 127, 128, 254, 255]))
    assert sc[:6].tolist() == [2.0 ** -127, 2.0 ** -126, 0.5, 1.0, 2.0, 2.0 ** 127] and np.isnan(sc[6])


def _torch_mxfp4(packed, scales):
    """MXFP4 decode through torch: the published E2M1 grid as a lookup table, low
    nibble first, one ldexp per block of 32."""
    grid = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=torch.float64)
    p = torch.as_tensor(np.asarray(packed)).long()
    codes = torch.stack([p & 15, p >> 4], dim=-1).flatten(-2)
    v = grid[codes & 7] * torch.where(codes >= 8, -1.0, 1.0).double()
    e = torch.as_tensor(np.asarray(scales)).long() - 127
    return torch.ldexp(v, e.repeat_interleave(32, dim=-1))


def test_mxfp4_layer_equals_layer_on_torch_decoded_weights():
    rng = np.random.default_rng(34)
    T, H, E, K, I = 24, 64, 4, 2, 96
    x = rng.standard_normal((T, H))
    w13 = (rng.standard_normal((E, 2 * I, H)) / 8).astype(np.float32)
    w2 = (rng.standard_normal((E, H, I)) / 10).astype(np.float32)
    q13, s13 = W._mxfp4(w13)
    q2, s2 = W._mxfp4(w2)
    wr = rng.standard_normal((E, H))
    L4 = dict(E=E, K=K, act="silu", renorm=True, w_router=wr, w13=q13.numpy(), w2=q2.numpy(),
              w13_scale=s13.numpy(), w2_scale=s2.numpy())
    got = O.moe_layer(x, L4)["out"]
    d13, d2 = _torch_mxfp4(q13, s13).numpy(), _torch_mxfp4(q2, s2).numpy()
    ref = O.moe_layer(x, dict(L4, w13=d13, w2=d2, w13_scale=None, w2_scale=None))["out"]
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # the decoded weights approximate the drawn ones within the format's steps
    err = np.abs(d13 - w13)
    scale = np.repeat(O.decode_e8m0(s13.numpy()), 32, axis=-1)
    assert np.all(err <= np.maximum(0.25 * scale, np.abs(w13) * 0.25) + 1e-12)


def test_mxfp4_quantiser_block_scales():
    """Each block's largest magnitude lands on 4 or 6 (or saturates at 6) after the
    power-of-two scale; all-zero blocks have zero codes."""
    rng = np.random.default_rng(35)
    w = (rng.standard_normal((2, 8, 128)) * rng.uniform(1e-3, 10, (2, 8, 1))).astype(np.float32)
    w[0, 0, :32] = 0.0
    q, sc = W._mxfp4(w)
    d = _torch_mxfp4(q, sc).numpy().reshape(2, 8, 4, 32)
    sb = O.decode_e8m0(sc.numpy())
    top = np.abs(d).max(axis=-1) / sb
    nz = np.abs(w.reshape(2, 8, 4, 32)).max(axis=-1) > 0
    assert np.all(np.isin(top[nz], [4.0, 6.0]))
    assert not d[0, 0, 0].any()


def test_e4m3_encode_matches_torch_including_ties():
    """Nearest-even E4M3 encoding against torch's float8_e4m3fn conversion: every
    representable value, every midpoint between neighbours (ties), a dense sweep,
    values near zero of both signs, and saturation above 448."""
    vals = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([vals, -vals, mids, -mids, np.linspace(-460, 460, 40001),
                        np.linspace(-0.003, 0.003, 601)]).astype(np.float32)
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.encode_e4m3fn(x), ref)
    assert O.encode_e4m3fn(np.array([1e6, -1e6], dtype=np.float32)).tolist() == [0x7E, 0xFE]


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(30)
    a = np.concatenate([rng.standard_normal(20000) * 10, rng.standard_normal(2000) * 1e-30])
    ref = torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(O.round_bf16(a), ref.astype(np.float64))


def test_dynamic_fp8_rows_properties():
    """Per row: the largest magnitude maps to +-448 exactly; every value comes back
    within half an E4M3 step (relative 2^-4 above the subnormal range, absolute
    2^-10 scale below it); scaling a row by a power of two keeps its codes; an
    all-zero row has scale 1 and zero codes."""
    rng = np.random.default_rng(31)
    a = (rng.standard_normal((64, 300)) * rng.uniform(0.01, 100, (64, 1))).astype(np.float32)
    a[5] = 0.0
    codes, scale = O.quantize_rows_fp8(a)
    nz = np.arange(64) != 5
    arg = np.abs(a).argmax(axis=1)
    assert np.all((codes[nz, arg[nz]] & 0x7F) == 0x7E)
    assert scale[5] == 1.0 and not codes[5].any()
    back = O.decode_e4m3fn(codes) * scale[:, None].astype(np.float64)
    err = np.abs(back - a)
    bound = np.maximum(np.abs(a) * 2.0 ** -4, scale[:, None] * 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-6))
    c2, s2 = O.quantize_rows_fp8(a * np.float32(8.0))
    assert np.array_equal(c2, codes) and np.array_equal(s2[nz], scale[nz] * 8)


def _torch_fp8_rows(a):
    """Per-row dynamic FP8 through torch: scale max|row|/448 (1 for zeros), float8_e4m3fn
    conversion of a / scale, back to float64."""
    a = torch.as_tensor(a, dtype=torch.float32)
    s = a.abs().amax(dim=1) / 448.0
    s = torch.where(s > 0, s, torch.ones_like(s))
    return (a / s[:, None]).to(torch.float8_e4m3fn).double() * s.double()[:, None]


def test_fp8_dynamic_ffn_matches_torch_composition():
    """The W8A8 expert FFN through torch, one library step at a time: per-row scale,
    float8_e4m3fn conversion of x / scale, float64 matmuls, bfloat16 rounding of h,
    the same quantisation of h, the down projection."""
    rng = np.random.default_rng(32)
    H, I, R = 64, 48, 40
    x = rng.standard_normal((R, H)).astype(np.float32)
    w13 = rng.standard_normal((2 * I, H)) / 8
    w2 = rng.standard_normal((H, I)) / 7

    tq = _torch_fp8_rows
    xq = tq(x)
    W13 = torch.from_numpy(w13)
    g, u = xq @ W13[:I].T, xq @ W13[I:].T
    h = F.silu(g) * u
    hq = tq(h.to(torch.bfloat16).float())
    ref = (hq @ torch.from_numpy(w2).T).numpy()
    got = O.gated_ffn(x, w13, w2, "silu", act_quant="fp8_dynamic")
    np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-12)
    # and it is an approximation of the unquantised FFN, not a different function
    plain = O.gated_ffn(x, w13, w2, "silu")
    assert np.sqrt(np.mean((got - plain) ** 2) / np.mean(plain ** 2)) < 0.1


def test_fp8_layer_equals_decoded_bf16_layer():
    """The FP8 path is the plain layer on decode(q) * s."""
    rng = np.random.default_rng(10)
    T, H, E, K, I = 8, 32, 4, 2, 16
    x = rng.standard_normal((T, H))
    q13 = rng.integers(0, 256, (E, 2 * I, H), dtype=np.uint8)
    q13[(q13 & 0x7F) == 0x7F] = 0x10
    q2 = rng.integers(0, 256, (E, H, I), dtype=np.uint8)
    q2[(q2 & 0x7F) == 0x7F] = 0x22
    s13 = rng.uniform(1e-3, 1e-2, (E, 2 * I))
    s2 = rng.uniform(1e-3, 1e-2, (E, H))
    z = rng.standard_normal((T, E))
    base = dict(E=E, K=K, act="gelu_tanh", renorm=True, w_router=None)
    got = O.moe_layer(x, dict(base, w13=q13, w2=q2, w13_scale=s13, w2_scale=s2), logits=z)["out"]
    dec13 = torch.from_numpy(q13).view(torch.float8_e4m3fn).double().numpy() * s13[..., None]
    dec2 = torch.from_numpy(q2).view(torch.float8_e4m3fn).double().numpy() * s2[..., None]
    D = _brute_dispatch(z, K, True, None)
    ref = sum(D[:, e:e + 1] * _torch_ffn(torch.from_numpy(x), torch.from_numpy(dec13[e]),
                                         torch.from_numpy(dec2[e]), "gelu_tanh").numpy()
              for e in range(E))
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------- dispatch

@pytest.mark.parametrize("T,E,K", [(128, 128, 8), (33, 8, 2), (1, 16, 4), (0, 4, 2)])
def test_permutation_matches_stable_argsort(T, E, K):
    rng = np.random.default_rng(11)
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]) if T else np.zeros((0, K), int)
    counts, offsets, order = O.permutation(ids, E)
    flat = ids.reshape(-1)
    assert counts.sum() == T * K
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert np.array_equal(order, np.argsort(flat, kind="stable"))
    assert sorted(order.tolist()) == list(range(T * K))
    for e in range(E):
        assert (flat[order[offsets[e]:offsets[e + 1]]] == e).all()


# --------------------------------------------------------------------------- branches

def test_two_shared_experts_equal_one_of_double_width():
    rng = np.random.default_rng(12)
    T, H, E, K, I, Is = 10, 16, 4, 2, 8, 12
    x = rng.standard_normal((T, H))
    L = _tiny_layer(rng, T, H, E, K, I, scale=False)
    L["renorm"] = False
    sw13 = rng.standard_normal((2, 2 * Is, H))
    sw2 = rng.standard_normal((2, H, Is))
    a = O.moe_layer(x, dict(L, shared=(sw13, sw2)))["out"]
    cat13 = np.concatenate([sw13[0][:Is], sw13[1][:Is], sw13[0][Is:], sw13[1][Is:]])[None]
    cat2 = np.concatenate([sw2[0], sw2[1]], axis=1)[None]
    b = O.moe_layer(x, dict(L, shared=(cat13, cat2)))["out"]
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    no_shared = O.moe_layer(x, L)["out"]
    ref = no_shared + _torch_ffn(torch.from_numpy(x), torch.from_numpy(cat13[0]),
                                 torch.from_numpy(cat2[0]), "silu").numpy()
    np.testing.assert_allclose(a, ref, rtol=1e-11, atol=1e-12)


def test_router_input_has_unit_norm():
    """RMSNorm without gamma, times H**-0.5, with unit scale: every router input
    vector has norm ~1 (Gemma 4 walkthrough section 3)."""
    rng = np.random.default_rng(13)
    x = rng.standard_normal((50, 2816)) * rng.uniform(0.1, 100, (50, 1))
    r = O.router_input(x, "gemma")
    np.testing.assert_allclose(np.linalg.norm(r, axis=-1), 1.0, rtol=1e-5)


def test_gemma_branch_matches_torch_composition():
    """Gemma block: router on the raw residual with its own preprocessing; experts
    on pre_norm_2(x); dense MLP on pre_norm(x); each branch post-normed; summed
    without weights.  Rebuilt from torch.nn.functional (rms_norm, linear, gelu)."""
    rng = np.random.default_rng(14)
    T, H, E, K, I, Id = 12, 32, 8, 3, 16, 24
    eps = 1e-6
    x = rng.standard_normal((T, H)) * 3
    L = _tiny_layer(rng, T, H, E, K, I, act="gelu_tanh")
    L["router_mode"] = "gemma"
    L["router_scale"] = rng.uniform(0.5, 1.5, H)
    g = {k: rng.uniform(0.5, 1.5, H) for k in ("gamma_pre", "gamma_pre2", "gamma_post1", "gamma_post2")}
    dw13 = rng.standard_normal((2 * Id, H)) / math.sqrt(H)
    dw2 = rng.standard_normal((H, Id)) / math.sqrt(Id)
    L["dense"] = dict(w13=dw13, w2=dw2, **g)
    got = O.moe_layer(x, L)

    xt = torch.from_numpy(x)
    T_ = lambda a: torch.from_numpy(np.asarray(a))
    r = F.rms_norm(xt, (H,), eps=eps) * H ** -0.5 * T_(L["router_scale"])
    z = F.linear(r, T_(L["w_router"])).numpy()
    np.testing.assert_allclose(got["logits"], z, rtol=1e-12, atol=1e-13)
    D = _brute_dispatch(z, K, True, L["per_expert_scale"])
    xe = F.rms_norm(xt, (H,), weight=T_(g["gamma_pre2"]), eps=eps)
    moe = sum(T_(D[:, e:e + 1]) * _torch_ffn(xe, T_(L["w13"][e]), T_(L["w2"][e]), "gelu_tanh")
              for e in range(E))
    d = _torch_ffn(F.rms_norm(xt, (H,), weight=T_(g["gamma_pre"]), eps=eps), T_(dw13), T_(dw2),
                   "gelu_tanh")
    ref = (F.rms_norm(d, (H,), weight=T_(g["gamma_post1"]), eps=eps) +
           F.rms_norm(moe, (H,), weight=T_(g["gamma_post2"]), eps=eps))
    np.testing.assert_allclose(got["out"], ref.numpy(), rtol=1e-10, atol=1e-11)
    # the whole FFN block: post_feedforward_layernorm of the sum, then + residual
    gff = rng.uniform(0.5, 1.5, H)
    blk = O.moe_layer(x, dict(L, block_tail=True, gamma_post_ff=gff))["out"]
    ref_blk = xt + F.rms_norm(ref, (H,), weight=T_(gff), eps=eps)
    np.testing.assert_allclose(blk, ref_blk.numpy(), rtol=1e-10, atol=1e-11)


def test_gemma_w8a8_layer_matches_torch_composition():
    """FP8 activations with the Gemma branch: the experts' input is pre_norm_2(x) as
    stored in bf16, quantised per row; h quantised per row after its bf16 rounding; the
    dense MLP unquantised; post-norms and the sum as in the bf16 layer."""
    rng = np.random.default_rng(33)
    T, H, E, K, I, Id = 10, 32, 6, 2, 16, 24
    eps = 1e-6
    x = rng.standard_normal((T, H)).astype(np.float32).astype(np.float64)
    L = _tiny_layer(rng, T, H, E, K, I, act="gelu_tanh")
    g = {k: rng.uniform(0.5, 1.5, H) for k in ("gamma_pre", "gamma_pre2", "gamma_post1", "gamma_post2")}
    dw13 = rng.standard_normal((2 * Id, H)) / math.sqrt(H)
    dw2 = rng.standard_normal((H, Id)) / math.sqrt(Id)
    L["dense"] = dict(w13=dw13, w2=dw2, **g)
    L["act_quant"] = "fp8_dynamic"
    got = O.moe_layer(x, L)

    xt = torch.from_numpy(x)
    T_ = lambda a: torch.from_numpy(np.asarray(a))
    D = _brute_dispatch(got["logits"], K, True, L["per_expert_scale"])
    xe = F.rms_norm(xt, (H,), weight=T_(g["gamma_pre2"]), eps=eps).to(torch.bfloat16).double()
    xq = _torch_fp8_rows(xe)

    def ffn_q(e):
        W13 = T_(L["w13"][e])
        h = F.gelu(xq @ W13[:I].T, approximate="tanh") * (xq @ W13[I:].T)
        return _torch_fp8_rows(h.to(torch.bfloat16).float()) @ T_(L["w2"][e]).T

    moe = sum(T_(D[:, e:e + 1]) * ffn_q(e) for e in range(E))
    d = _torch_ffn(F.rms_norm(xt, (H,), weight=T_(g["gamma_pre"]), eps=eps), T_(dw13), T_(dw2), "gelu_tanh")
    ref = (F.rms_norm(d, (H,), weight=T_(g["gamma_post1"]), eps=eps) +
           F.rms_norm(moe, (H,), weight=T_(g["gamma_post2"]), eps=eps)).numpy()
    np.testing.assert_allclose(got["out"], ref, rtol=1e-9, atol=1e-10)


def test_fp8_h_codes_taken_as_given():
    """h_fp8: the down projection of given E4M3 codes and row scales (decoded by
    torch's float8_e4m3fn), per (token, slot); with the codes the oracle itself
    would pick, the layer is unchanged."""
    rng = np.random.default_rng(34)
    T, H, E, K, I, Id = 9, 32, 6, 2, 16, 24
    x = rng.standard_normal((T, H)).astype(np.float32).astype(np.float64)
    L = _tiny_layer(rng, T, H, E, K, I, act="gelu_tanh")
    L["dense"] = dict(w13=rng.standard_normal((2 * Id, H)) / math.sqrt(H),
                      w2=rng.standard_normal((H, Id)) / math.sqrt(Id))
    L["act_quant"] = "fp8_dynamic"
    own = O.moe_layer(x, L)
    ids = own["ids"]
    # the codes the oracle picks, rebuilt through torch: x quantised as stored, then h
    xe = torch.from_numpy(O.rmsnorm(x)).to(torch.bfloat16).double()
    xq = _torch_fp8_rows(xe)
    codes = np.zeros((T, K, I), np.uint8)
    scales = np.zeros((T, K), np.float32)
    for t in range(T):
        for j in range(K):
            W13 = torch.from_numpy(L["w13"][ids[t, j]])
            h = F.gelu(xq[t:t + 1] @ W13[:I].T, approximate="tanh") * (xq[t:t + 1] @ W13[I:].T)
            hb = h.to(torch.bfloat16).float()
            sc = torch.clamp(hb.abs().amax(), min=0) / 448.0
            sc = sc if sc > 0 else torch.ones(())
            q = (hb / sc).to(torch.float8_e4m3fn)
            codes[t, j] = q.view(torch.uint8).numpy()[0]
            scales[t, j] = sc.item()
    same = O.moe_layer(x, L, h_fp8=(codes, scales))
    np.testing.assert_allclose(same["out"], own["out"], rtol=1e-12, atol=1e-13)
    # other codes change the output by exactly their own down projection
    c2 = codes.copy()
    c2[4, 1, 7] ^= 0x01  # one mantissa step
    other = O.moe_layer(x, L, h_fp8=(c2, scales))
    dq = (torch.tensor([c2[4, 1, 7]], dtype=torch.uint8).view(torch.float8_e4m3fn).double() -
          torch.tensor([codes[4, 1, 7]], dtype=torch.uint8).view(torch.float8_e4m3fn).double()).item()
    dmoe = own["weights"][4, 1] * dq * float(scales[4, 1]) * L["w2"][ids[4, 1]][:, 7]
    moe_own = O.moe_combine(O.round_bf16(O.rmsnorm(x)), own["weights"], ids, L["w13"], L["w2"], "gelu_tanh",
                            act_quant="fp8_dynamic")
    d = O.gated_ffn(O.rmsnorm(x), L["dense"]["w13"], L["dense"]["w2"], "gelu_tanh")
    want = O.rmsnorm(d) + O.rmsnorm(moe_own + np.eye(T)[4][:, None] * dmoe[None, :])
    np.testing.assert_allclose(other["out"], want, rtol=1e-11, atol=1e-12)
    with pytest.raises(ValueError):
        O.gated_ffn(x, L["w13"][0], L["w2"][0], "silu", h_fp8=(codes[:, 0], scales[:, 0]))


def test_row_subset_matches_full():
    rng = np.random.default_rng(15)
    T, H, E, K, I = 40, 16, 8, 2, 8
    x = rng.standard_normal((T, H))
    L = _tiny_layer(rng, T, H, E, K, I)
    full = O.moe_layer(x, L)["out"]
    rows = np.array([3, 0, 39, 17])
    sub = O.moe_layer(x, L, rows=rows)["out"]
    np.testing.assert_allclose(sub, full[rows], rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------- workloads

def test_param_counts_match_page():
    g = _golden("param_counts.txt")
    c = W.param_counts(W.SPECS["gemma"])
    assert c["per_expert"] == 3 * 2816 * 704 == 5_947_392
    assert c["dense"] == 3 * 2816 * 2112 == 17_842_176
    assert abs(c["dense"] - g["dense_mlp"][0]) / g["dense_mlp"][0] < 0.01
    assert abs(c["per_expert"] - g["per_expert"][0]) / g["per_expert"][0] < 0.01
    assert abs(c["experts"] - g["all_experts"][0]) / g["all_experts"][0] < 0.01
    active = (8 * c["per_expert"] + c["dense"]) / (c["experts"] + c["dense"])
    assert abs(active - g["active_fraction"][0]) < 0.001


def test_zipf_skew_share():
    """About 10% of the experts (13 of 128) take about 60% of the assignments."""
    from oracle.calibrate_zipf import top_share
    L = W.make_layer(W.SPECS["skewed_fp8"].with_T(4096), x_only=True)
    noise = W._normal(0, W._TID["logit_noise"], (4096, 128), 1.0)
    z = noise + W.zipf_bias(128, 0)[None, :]
    share = top_share(z.astype(np.float64), 8, 13)
    assert 0.58 <= share <= 0.62


def test_generator_is_seeded_and_T_independent():
    s = W.SPECS["tiny"]
    a = W.make_layer(s, T=64)
    b = W.make_layer(s, T=5)
    assert torch.equal(a["w13"], b["w13"]) and torch.equal(a["x"][:5], b["x"])
    c = W.make_layer(s, seed=1, T=5)
    assert not torch.equal(a["w13"], c["w13"])
