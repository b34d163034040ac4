"""GPU parity of moe_route and moe_permute against the oracle: ids, counts,
offsets and the permutation bit-exact; routing weights within 1e-6 relative."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from tests.parity import assert_weights_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_ffn_router_amd import binding
    binding.load()
    return binding


def _logits(T, E, seed, kind="normal"):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((T, E)).astype(np.float32) * 2
    if kind == "ties":
        z = (np.round(z * 2) / 2).astype(np.float32)
        z[z == 0] = -0.0
        z[::5] = 0.0
        z[1::7, : E // 2] = 1.5
    elif kind == "skewed":
        z += np.linspace(3, -3, E, dtype=np.float32)[None, :]
    return z


def _check_route(B, z, K, renorm=True, scale=None, scoring="softmax", G=0, KG=0):
    zt = torch.from_numpy(z).cuda()
    st = None if scale is None else torch.from_numpy(scale).cuda()
    w, ids = B.route(zt, K, renorm, st, scoring=scoring, n_groups=G, topk_groups=KG)
    torch.cuda.synchronize()
    wr, idr = O.route(z.astype(np.float64), K, renorm, scale, scoring, max(G, 1), max(KG, 1))
    assert np.array_equal(ids.cpu().numpy(), idr), "topk_ids differ"
    assert_weights_close(w.cpu().numpy(), wr)


@pytest.mark.parametrize("E,K", [(1, 1), (2, 1), (8, 2), (8, 8), (63, 5), (64, 6), (65, 8), (128, 8),
                                 (200, 3), (256, 8), (512, 16), (64, 64)])
@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_route_matches_oracle(B, E, K, kind):
    z = _logits(1003, E, seed=E * 7 + K, kind=kind)
    _check_route(B, z, K, True)


@pytest.mark.parametrize("renorm", [True, False])
def test_route_scale_and_renorm(B, renorm):
    E, K = 128, 8
    z = _logits(517, E, seed=3, kind="skewed")
    scale = np.random.default_rng(4).uniform(0.5, 1.5, E).astype(np.float32)
    _check_route(B, z, K, renorm, scale)


# sigmoid scoring and expert groups (llama.cpp MoE lesson): group ranges that
# straddle lanes (25, 32 experts), one expert per group, the 64-group limit
@pytest.mark.parametrize("E,K,G,KG", [(256, 8, 8, 4), (64, 6, 8, 3), (96, 8, 3, 1), (200, 10, 8, 2),
                                      (16, 4, 16, 4), (512, 16, 64, 8), (8, 2, 0, 0)])
@pytest.mark.parametrize("scoring,renorm", [("sigmoid", True), ("sigmoid", False), ("softmax", False)])
@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_route_sigmoid_and_groups(B, E, K, G, KG, scoring, renorm, kind):
    z = _logits(1003, E, seed=E * 11 + K + G, kind=kind)
    scale = np.random.default_rng(E).uniform(0.5, 1.5, E).astype(np.float32)
    _check_route(B, z, K, renorm, scale, scoring, G, KG)


def test_route_groups_tied_group_scores(B):
    """Groups whose best logits tie: the lower group is picked (hand-checked row
    from the oracle's pins), on every token of a 4-token batch."""
    z = np.tile(np.array([[1.0, 0.0, 0.0, 1.0, 2.0, 2.0, -1.0, -1.0]], dtype=np.float32), (4, 1))
    zt = torch.from_numpy(z).cuda()
    w, ids = B.route(zt, 4, True, scoring="sigmoid", n_groups=4, topk_groups=2)
    assert ids.cpu().tolist() == [[4, 5, 0, 1]] * 4
    _check_route(B, z, 4, True, None, "sigmoid", 4, 2)


@pytest.mark.parametrize("T", [0, 1, 2, 3, 4, 5, 4097])
def test_route_token_counts(B, T):
    z = _logits(T, 64, seed=T)
    if T == 0:
        w, ids = B.route(torch.zeros(0, 64, device="cuda"), 6)
        assert w.shape == (0, 6)
        return
    _check_route(B, z, 6, False)


def test_route_signed_zero_and_all_equal(B):
    z = np.zeros((4, 16), dtype=np.float32)
    z[1, ::2] = -0.0
    z[2] = 1.0
    z[3, 5] = -0.0
    z[3, 9] = 0.0
    _check_route(B, z, 4)


def test_route_extreme_logits(B):
    z = _logits(64, 128, seed=9) * 40  # softmax far from uniform, exp underflows for most
    _check_route(B, z, 8)


def _check_permute(B, ids, E, bm):
    T, K = ids.shape
    res = B.permute(torch.from_numpy(ids.astype(np.int32)).cuda(), E, bm)
    torch.cuda.synchronize()
    counts, offsets, order = O.permutation(ids, E)
    c = res["counts"].cpu().numpy()
    off = res["offsets"].cpu().numpy()
    ss = res["sorted_slots"].cpu().numpy()
    be = res["block_expert"].cpu().numpy()
    assert np.array_equal(c, counts)
    padded = (counts + bm - 1) // bm * bm
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(padded)]))
    compact = np.concatenate([ss[off[e]:off[e] + c[e]] for e in range(E)]) if E else ss[:0]
    assert np.array_equal(compact, order)
    for e in range(E):
        assert (ss[off[e] + c[e]:off[e + 1]] == -1).all()
        assert (be[off[e] // bm:off[e + 1] // bm] == e).all()
    assert off[E] <= res["capacity"]
    assert int(res["num_padded"].item()) == off[E]
    # inverse map: the oracle's compact position of each slot, moved to its padded segment
    inv = np.empty(T * K, dtype=np.int64)
    inv[order] = np.arange(T * K)
    flat = ids.reshape(-1)
    want = inv - offsets[flat] + off[flat]
    assert np.array_equal(res["slot_row"].cpu().numpy(), want)
    assert np.array_equal(ss[want], np.arange(T * K))


@pytest.mark.parametrize("T,K,E", [(1, 1, 1), (1, 8, 128), (16, 8, 128), (128, 8, 128), (4096, 2, 8),
                                   (1000, 6, 66), (333, 3, 1024), (8192, 8, 128), (5, 2, 700),
                                   # the one-block path at its limits (8192 slots; its table full
                                   # at 2048 x 4 over 256 experts), then just past them
                                   (1024, 8, 128), (2048, 4, 256), (2048, 8, 128), (4096, 4, 1024),
                                   # the chunked path: whole 4096-slot chunks only, and a few
                                   # slots past them
                                   (4096, 8, 128), (4097, 4, 256),
                                   # many chunks with many experts: 16384 x 64 slots over 512 experts
                                   (16384, 64, 512), (16384, 6, 1024)])
@pytest.mark.parametrize("bm", [16, 64, 256])
def test_permute_matches_oracle(B, T, K, E, bm):
    rng = np.random.default_rng(T + K + E)
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)])
    _check_permute(B, ids, E, bm)


def test_permute_skewed_and_empty_experts(B):
    rng = np.random.default_rng(1)
    T, K, E = 3000, 4, 64
    p = np.exp(-np.arange(E) / 3.0)
    p /= p.sum()
    ids = np.stack([rng.choice(E, K, replace=False, p=p) for _ in range(T)])
    _check_permute(B, ids, E, 64)
    ids = np.zeros((257, 1), dtype=np.int64) + 5  # every token on one expert
    _check_permute(B, ids, 16, 32)


def test_permute_is_deterministic(B):
    rng = np.random.default_rng(2)
    ids = torch.from_numpy(np.stack([rng.permutation(128)[:8] for _ in range(2048)]).astype(np.int32)).cuda()
    ref = B.permute(ids, 128, 64)["sorted_slots"].clone()
    for _ in range(20):
        assert torch.equal(B.permute(ids, 128, 64)["sorted_slots"], ref)
