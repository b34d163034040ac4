"""CPU checks of the C ABI: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host before any launch.
No call here reaches a GPU: every path exercised returns during validation."""
import ctypes as C
import os
import re

import pytest

from mixture_experts_ffn_router_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libmoe_mi355x.so is not built (python -m mixture_experts_ffn_router_amd.build)")
    return B.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert set(_declared()) == set(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in _declared():
        assert hasattr(lib, name), name


def test_only_the_c_abi_is_exported():
    out = os.popen(f"nm -D --defined-only {B.LIB_PATH}").read()
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(_declared()) <= exported
    assert not [s for s in exported if s.startswith("_ZN3moe")], "internal symbols leak"


def test_status_strings():
    lib = _lib()
    assert lib.moe_status_string(0) == b"MOE_OK"
    assert lib.moe_status_string(3) == b"MOE_WORKSPACE_TOO_SMALL"
    assert lib.moe_status_string(99) == b"MOE_UNKNOWN_STATUS"


def _desc(**kw):
    d = dict(hidden=256, num_experts=8, top_k=2, inter=512, act=0, act_dtype=B.DT_BF16,
             weight_dtype=B.DT_BF16, renormalize=1, router_mode=0, n_shared=0, inter_dense=0,
             dense_act=0, eps=1e-6)
    d.update(kw)
    return B.LayerDesc(**d)


def _ws(desc, T):
    n = C.c_size_t(0)
    st = _lib().moe_forward_workspace_size(C.byref(desc), T, C.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,status", [
    (dict(top_k=9), B.MOE_INVALID_ARG),
    (dict(top_k=0), B.MOE_INVALID_ARG),
    (dict(num_experts=513, top_k=2), B.MOE_UNSUPPORTED),
    (dict(hidden=200), B.MOE_UNSUPPORTED),
    (dict(inter=100), B.MOE_UNSUPPORTED),
    (dict(act=7), B.MOE_INVALID_ARG),
    (dict(act_dtype=B.DT_F32), B.MOE_UNSUPPORTED),
    (dict(weight_dtype=B.DT_F32), B.MOE_UNSUPPORTED),
    (dict(weight_dtype=B.DT_FP8, n_shared=1), B.MOE_UNSUPPORTED),
    (dict(n_shared=9), B.MOE_INVALID_ARG),
    (dict(inter_dense=100), B.MOE_UNSUPPORTED),
    (dict(router_mode=5), B.MOE_INVALID_ARG),
    (dict(eps=-1.0), B.MOE_INVALID_ARG),
    (dict(top_k=60, num_experts=128, n_shared=8), B.MOE_UNSUPPORTED),
    (dict(scoring=2), B.MOE_INVALID_ARG),
    (dict(n_groups=-1), B.MOE_INVALID_ARG),
    (dict(n_groups=3), B.MOE_INVALID_ARG),                 # does not divide E = 8
    (dict(n_groups=4, topk_groups=0), B.MOE_INVALID_ARG),
    (dict(n_groups=4, topk_groups=5), B.MOE_INVALID_ARG),
    (dict(n_groups=4, topk_groups=1, top_k=3), B.MOE_INVALID_ARG),  # 2 candidates < 3
    (dict(num_experts=128, top_k=2, n_groups=128, topk_groups=2), B.MOE_UNSUPPORTED),
    (dict(act_quant=2), B.MOE_INVALID_ARG),
    (dict(block_tail=2), B.MOE_INVALID_ARG),
    (dict(weight_dtype=B.DT_MXFP4, n_shared=1), B.MOE_UNSUPPORTED),
    (dict(weight_dtype=B.DT_MXFP4, act_dtype=B.DT_F32), B.MOE_UNSUPPORTED),
    (dict(weight_dtype=B.DT_MXFP4, act_quant=1), B.MOE_UNSUPPORTED),
    (dict(act_quant=1), B.MOE_UNSUPPORTED),                              # bf16 weights
    (dict(act_quant=1, weight_dtype=B.DT_FP8, inter=16448), B.MOE_UNSUPPORTED),
])
def test_bad_descriptors_rejected(kw, status):
    st, _ = _ws(_desc(**kw), 16)
    assert st == status, _lib().moe_last_error()
    assert _lib().moe_last_error() != b""


def test_workspace_size_grows_with_T_and_covers_buffers():
    d = _desc()
    st0, n0 = _ws(d, 0)
    st1, n1 = _ws(d, 64)
    st2, n2 = _ws(d, 4096)
    assert st0 == st1 == st2 == B.MOE_OK
    assert n0 <= n1 < n2
    # per-slot outputs alone need T*K*H*2 bytes
    assert n2 >= 4096 * 2 * 256 * 2


@pytest.mark.parametrize("shape", [
    dict(hidden=4096, num_experts=8, top_k=2, inter=14336),                      # Mixtral-style
    dict(hidden=2048, num_experts=64, top_k=6, inter=1408, n_shared=2),          # DeepSeek-style
    dict(hidden=2816, num_experts=128, top_k=8, inter=704, inter_dense=2112),    # Gemma-style
    dict(hidden=256, num_experts=2, top_k=1, inter=4096),                        # long down reduction
    # DeepSeek-V3 routing shape: below 4 tokens its decode down kernel splits the
    # reduction into parts (128 feature groups, long per-block streams)
    dict(hidden=2048, num_experts=256, top_k=8, inter=1408, n_shared=1, scoring=1, n_groups=8,
         topk_groups=4),
    # FP8 weights and activations: the decode layout (codes and scales) up to 16 tokens
    dict(hidden=2816, num_experts=128, top_k=8, inter=704, weight_dtype=B.DT_FP8, act_quant=1),
])
def test_workspace_size_never_decreases_with_T(shape):
    """A workspace sized for the largest T serves every smaller T: the reported
    size is non-decreasing over every T up to 20000 or the largest supported T
    (row-block changes and the down GEMM's reduction parts included)."""
    d = _desc(**shape)
    prev = 0
    for T in range(0, 20001):
        st, n = _ws(d, T)
        if st == B.MOE_UNSUPPORTED and T > 4096:  # an activation buffer would pass 2 GiB
            break
        assert st == B.MOE_OK
        assert n >= prev, f"workspace size falls from {prev} to {n} at T = {T}"
        prev = n


def test_forward_rejects_missing_tensors_and_small_workspace():
    lib = _lib()
    d = _desc()
    fake = 0x1000  # never dereferenced: validation fails first
    ts = B.Tensors(x=fake, w13=fake, w2=fake, out=fake)  # no logits, no router
    st = lib.moe_forward(C.byref(d), C.byref(ts), 16, fake, 1 << 30, None)
    assert st == B.MOE_INVALID_ARG and b"logits" in lib.moe_last_error()
    ts.w_router = fake
    st = lib.moe_forward(C.byref(d), C.byref(ts), 16, fake, 16, None)
    assert st == B.MOE_WORKSPACE_TOO_SMALL
    st = lib.moe_forward(C.byref(d), C.byref(ts), 16, fake + 8, 1 << 40, None)
    assert st == B.MOE_INVALID_ARG and b"aligned" in lib.moe_last_error()
    st = lib.moe_forward(C.byref(d), None, 16, fake, 1 << 40, None)
    assert st == B.MOE_INVALID_ARG
    for name in ("x", "w13", "w2", "out", "w_router"):  # matrix operands move in 16-byte pieces
        bad = B.Tensors(x=fake, w13=fake, w2=fake, out=fake, w_router=fake)
        setattr(bad, name, fake + 8)
        st = lib.moe_forward(C.byref(d), C.byref(bad), 16, fake, 1 << 40, None)
        assert st == B.MOE_INVALID_ARG and name.encode() in lib.moe_last_error() and b"aligned" in lib.moe_last_error()
    d8 = _desc(weight_dtype=B.DT_FP8)
    st = lib.moe_forward(C.byref(d8), C.byref(ts), 16, fake, 1 << 40, None)
    assert st == B.MOE_INVALID_ARG and b"scale" in lib.moe_last_error()
    # T = 0 is a no-op
    assert lib.moe_forward(C.byref(d), C.byref(ts), 0, None, 0, None) == B.MOE_OK


def test_noalloc_refuses_large_layouts_before_any_launch():
    """The no-allocation entry point checks its static scratch's size on the host:
    a layout beyond it is refused with MOE_WORKSPACE_TOO_SMALL, nothing touched."""
    lib = _lib()
    d = _desc(hidden=4096, num_experts=8, top_k=2, inter=14336)
    st, need = _ws(d, 4096)
    assert st == B.MOE_OK and need > B.NOALLOC_SCRATCH_BYTES
    fake = 0x1000
    ts = B.Tensors(x=fake, w_router=fake, w13=fake, w2=fake, out=fake)
    assert lib.moe_forward_noalloc(C.byref(d), C.byref(ts), 4096, None) == B.MOE_WORKSPACE_TOO_SMALL
    assert b"static scratch" in lib.moe_last_error()
    assert lib.moe_forward_noalloc(C.byref(d), C.byref(ts), 0, None) == B.MOE_OK  # T = 0: a no-op
    assert lib.moe_forward_noalloc(C.byref(d), None, 16, None) == B.MOE_INVALID_ARG


def test_route_and_permute_validation():
    lib = _lib()
    fake = 0x1000
    assert lib.moe_route(fake, 4, 8, 9, 1, 0, 0, 0, None, fake, fake, None) == B.MOE_INVALID_ARG
    assert lib.moe_route(fake, 4, 600, 2, 1, 0, 0, 0, None, fake, fake, None) == B.MOE_UNSUPPORTED
    assert lib.moe_route(fake, -1, 8, 2, 1, 0, 0, 0, None, fake, fake, None) == B.MOE_INVALID_ARG
    assert lib.moe_route(None, 0, 8, 2, 1, 0, 0, 0, None, None, None, None) == B.MOE_OK
    assert lib.moe_route(None, 4, 8, 2, 1, 0, 0, 0, None, fake, fake, None) == B.MOE_INVALID_ARG
    # routing options are checked before anything else, T = 0 included
    assert lib.moe_route(None, 0, 8, 2, 1, 2, 0, 0, None, None, None, None) == B.MOE_INVALID_ARG
    assert lib.moe_route(None, 0, 8, 2, 1, 1, 3, 1, None, None, None, None) == B.MOE_INVALID_ARG
    assert lib.moe_route(None, 0, 8, 5, 1, 1, 4, 2, None, None, None, None) == B.MOE_INVALID_ARG
    assert lib.moe_route(None, 0, 8, 4, 1, 1, 4, 2, None, None, None, None) == B.MOE_OK
    assert lib.moe_route(None, 0, 8, 2, 1, 0, 1, 0, None, None, None, None) == B.MOE_OK  # 1 group = none
    assert lib.moe_permute(fake, 4, 2, 8, 48, fake, fake, fake, fake, None, fake, None) == B.MOE_INVALID_ARG
    assert lib.moe_permute(fake, 4, 2, 8, 512, fake, fake, fake, fake, None, fake, None) == B.MOE_INVALID_ARG
    assert lib.moe_permute(fake, 4, 0, 8, 64, fake, fake, fake, fake, None, fake, None) == B.MOE_INVALID_ARG
    assert lib.moe_permute(fake, 4, 2, 8, 64, None, fake, fake, fake, None, fake, None) == B.MOE_INVALID_ARG
    # slot_row (the inverse map) is required for T > 0; num_padded is optional
    assert lib.moe_permute(fake, 4, 2, 8, 64, fake, fake, fake, fake, fake, None, None) == B.MOE_INVALID_ARG


def test_permute_capacity():
    lib = _lib()
    assert lib.moe_permute_capacity(128, 8, 128, 64) == (1024 + 128 * 63) // 64 * 64
    assert lib.moe_permute_capacity(1, 1, 1, 16) == 16
    assert lib.moe_permute_capacity(4, 2, 8, 48) == -1
    assert lib.moe_permute_capacity(-1, 2, 8, 64) == -1


def test_fp8_activation_layers_take_the_decode_path_up_to_16_tokens():
    lib = _lib()
    d = _desc(act_quant=1, weight_dtype=B.DT_FP8)
    assert [lib.moe_forward_path(C.byref(d), t) for t in (1, 4, 16, 17, 4096)] == [1, 1, 1, 0, 0]
    d0 = _desc(weight_dtype=B.DT_FP8)
    assert lib.moe_forward_path(C.byref(d0), 4) == 1
    # the workspace holds the codes and scales of x and h as well
    st0, n0 = _ws(d0, 4096)
    st1, n1 = _ws(d, 4096)
    assert st0 == st1 == B.MOE_OK and n1 > n0 + 4096 * 256


def test_decode_layout_exposes_h_and_the_fp8_activation_codes():
    """On the decode path the layout query gives h per slot row and, with FP8
    activations, the codes and scales of x and h, all inside the workspace the
    size query reports; the grouped path's buffers are -1."""
    lib = _lib()
    fake = 0x1000  # never dereferenced: the query launches nothing
    ts = B.Tensors(x=fake, w13=fake, w2=fake, out=fake, w_router=fake, w13_scale=fake, w2_scale=fake)
    for aq in (0, 1):
        d = _desc(act_quant=aq, weight_dtype=B.DT_FP8, top_k=2, num_experts=8, hidden=256, inter=512)
        T = 5
        lay = B.WorkspaceLayout()
        assert lib.moe_forward_workspace_layout(C.byref(d), C.byref(ts), T, C.byref(lay)) == B.MOE_OK
        _, total = _ws(d, T)
        assert lay.path == 1 and lay.slots_per_token == 2 and lay.capacity == T * 2 and lay.y_parts == 0
        assert lay.topk_w == lay.sorted_slots == lay.slot_row == lay.y == lay.x_expert == -1
        assert 0 <= lay.h and lay.h + T * 2 * 512 * 2 <= total
        bufs = [(lay.x_codes, T * 256), (lay.x_scales, T * 4), (lay.h_codes, T * 2 * 512), (lay.h_scales, T * 2 * 4)]
        if aq:
            for off, n in bufs:
                assert off >= 0 and off % 256 == 0 and off + n <= total
            ends = sorted((off, off + n) for off, n in bufs + [(lay.h, T * 2 * 512 * 2)])
            assert all(a[1] <= b[0] for a, b in zip(ends, ends[1:])), "buffers overlap"
        else:
            assert all(off == -1 for off, _ in bufs)


def test_mxfp4_layers_run_on_the_decode_path_only():
    lib = _lib()
    d = _desc(weight_dtype=B.DT_MXFP4)
    assert lib.moe_forward_path(C.byref(d), 4) == 1
    fake = 0x1000  # never dereferenced: the call is refused before any launch
    ts = B.Tensors(x=fake, w13=fake, w2=fake, out=fake, w_router=fake, w13_scale=fake, w2_scale=fake)
    st = lib.moe_forward(C.byref(d), C.byref(ts), 64, fake, 1 << 40, None)
    assert st == B.MOE_UNSUPPORTED and b"decode path" in lib.moe_last_error()
    ts.w13_scale = None
    assert lib.moe_forward(C.byref(d), C.byref(ts), 4, fake, 1 << 40, None) == B.MOE_INVALID_ARG


def test_every_entry_point_raises_without_the_library(monkeypatch, tmp_path):
    """No fallback: with the library missing, the loader and the calls that go
    through it raise instead of computing anything another way."""
    missing = str(tmp_path / "libmoe_mi355x.so")
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", missing)
    with pytest.raises(ImportError, match="is missing"):
        B.load()
    with pytest.raises(ImportError, match="is missing"):
        B.permute_capacity(16, 2, 8, 64)
    d = B.LayerDesc(hidden=256, num_experts=8, top_k=2, inter=512, act=0, act_dtype=B.DT_BF16,
                    weight_dtype=B.DT_BF16, renormalize=1, eps=1e-6)
    layer = B.DeviceLayer.__new__(B.DeviceLayer)
    layer.desc = d
    with pytest.raises(ImportError, match="is missing"):
        layer.path(16)
    with pytest.raises(ImportError, match="is missing"):
        layer.workspace_size(16)



def _valid_desc(draw):
    """A random descriptor inside the header's limits (every rule of moe.h)."""
    from hypothesis import strategies as st
    wd = draw(st.sampled_from([B.DT_BF16, B.DT_FP8, B.DT_MXFP4, B.DT_F32]))
    f32 = wd == B.DT_F32
    n_shared = 0 if wd in (B.DT_FP8, B.DT_MXFP4) else draw(st.integers(0, 8))
    E = draw(st.integers(1, 512))
    K = draw(st.integers(1, min(E, 64 - n_shared)))
    kw = dict(hidden=64 * draw(st.integers(1, 128)), num_experts=E, top_k=K, inter=64 * draw(st.integers(1, 256)),
              act=draw(st.integers(0, 1)), act_dtype=B.DT_F32 if f32 else B.DT_BF16, weight_dtype=wd,
              renormalize=draw(st.integers(0, 1)), router_mode=draw(st.integers(0, 1)), n_shared=n_shared,
              inter_dense=64 * draw(st.integers(0, 64)), dense_act=draw(st.integers(0, 1)),
              scoring=draw(st.integers(0, 1)), block_tail=draw(st.integers(0, 1)),
              combine=0 if f32 else draw(st.integers(0, 1)),
              act_quant=1 if wd == B.DT_FP8 and draw(st.booleans()) else 0)
    groups = [g for g in range(2, 65) if E % g == 0]
    if groups and draw(st.booleans()):
        G = draw(st.sampled_from(groups))
        kg_min = -(-K // (E // G))  # the picked groups must hold at least K experts
        kw.update(n_groups=G, topk_groups=draw(st.integers(kg_min, G)))
    return _desc(**kw)


def test_workspace_size_never_decreases_for_random_layers():
    """The size contract (non-decreasing in T, so a workspace sized for the
    largest T serves every smaller one) over random layers inside every limit the
    header states: each T up to 300 (the decode range and the row-block changes
    of small batches), then T growing by an eighth up to 2^17.  A layer whose
    buffers would pass 2 GiB is refused from some T on (from T = 0 when the row
    padding of very many wide experts alone passes it), and then for every larger
    T.  Every size also holds the gated intermediate of all T * (top_k +
    n_shared) rows."""
    hyp = pytest.importorskip("hypothesis")
    from hypothesis import strategies as st
    Ts = list(range(0, 301))
    while Ts[-1] < 1 << 17:
        Ts.append(Ts[-1] + max(1, Ts[-1] // 8))

    seen = []

    @hyp.settings(max_examples=400, deadline=None, derandomize=True, database=None)
    @hyp.given(st.composite(_valid_desc)())
    def run(d):
        seen.append((d.num_experts, d.hidden, d.inter, d.weight_dtype))
        # the T that take the decode path form a prefix of 1..16 (its LDS needs grow with T)
        paths = [_lib().moe_forward_path(C.byref(d), T) for T in range(1, 18)]
        assert paths == sorted(paths, reverse=True) and paths[-1] == 0, paths
        prev, refused = 0, None
        ae = 4 if d.act_dtype == B.DT_F32 else 2
        for T in Ts:
            st_, n = _ws(d, T)
            if refused is not None:
                assert st_ == B.MOE_UNSUPPORTED, f"T = {T} accepted after T = {refused} was refused"
                continue
            if st_ == B.MOE_UNSUPPORTED:  # from T = 0 on when the padding alone passes the limit
                assert b"would exceed 2 GiB" in _lib().moe_last_error(), _lib().moe_last_error()
                refused = T
                continue
            assert st_ == B.MOE_OK, _lib().moe_last_error()
            assert n >= prev, f"workspace size falls from {prev} to {n} at T = {T}"
            assert n >= T * (d.top_k + d.n_shared) * d.inter * ae
            prev = n

    run()
    print(f"{len(seen)} layers, {len(set(seen))} distinct (experts, hidden, inter, weight type)")
    assert len(set(seen)) >= 100, len(set(seen))


def _layout_extents(d, lay, T):
    """(name, offset, bytes) of every buffer the layout query reports, with the
    shapes moe.h gives for them."""
    Kp, Ep = d.top_k + d.n_shared, d.num_experts + d.n_shared
    H, I, cap = d.hidden, d.inter, lay.capacity
    ae = 4 if d.act_dtype == B.DT_F32 else 2
    if lay.path == 1:  # decode: h per slot row, FP8 activation codes and scales
        bufs = [("h", lay.h, T * Kp * I * 2), ("x_codes", lay.x_codes, T * H), ("x_scales", lay.x_scales, T * 4),
                ("h_codes", lay.h_codes, T * Kp * I), ("h_scales", lay.h_scales, T * Kp * 4)]
    else:
        y_bytes = T * H * 4 if lay.y_parts == 0 else T * Kp * lay.y_parts * H * (4 if lay.y_f32 else ae)
        bufs = [("topk_w", lay.topk_w, T * Kp * 4), ("topk_ids", lay.topk_ids, T * Kp * 4),
                ("counts", lay.counts, Ep * 4), ("offsets", lay.offsets, (Ep + 1) * 4),
                ("sorted_slots", lay.sorted_slots, cap * 4), ("block_expert", lay.block_expert, cap // lay.block_m * 4),
                ("slot_row", lay.slot_row, T * Kp * 4), ("inv_rms", lay.inv_rms, T * 4),
                ("x_expert", lay.x_expert, T * H * ae), ("h", lay.h, cap * I * ae), ("y", lay.y, y_bytes),
                ("x_codes", lay.x_codes, T * H), ("x_scales", lay.x_scales, T * 4),
                ("h_codes", lay.h_codes, cap * I), ("h_scales", lay.h_scales, cap * 4)]
    return [b for b in bufs if b[1] != -1]


def test_workspace_layout_fits_the_reported_size_for_random_layers():
    """For random layers and token counts, every buffer the layout query reports
    (at the shape the header gives it) is 256-byte aligned, lies inside the
    workspace the size query asks for, and overlaps no other; the grouped path's
    capacity is the padded total moe_permute_capacity gives, and the decode path
    keeps one h row per slot."""
    hyp = pytest.importorskip("hypothesis")
    from hypothesis import strategies as st
    lib = _lib()
    fake = 0x1000  # never dereferenced: the queries launch nothing
    seen = []

    @hyp.settings(max_examples=300, deadline=None, derandomize=True, database=None)
    @hyp.given(st.composite(_valid_desc)(), st.sampled_from([1, 2, 5, 16, 17, 64, 129, 300, 1000, 4099]))
    def run(d, T):
        ts = B.Tensors(x=fake, w13=fake, w2=fake, out=fake, w_router=fake, w13_scale=fake, w2_scale=fake,
                       shared_w13=fake if d.n_shared else None, shared_w2=fake if d.n_shared else None,
                       dense_w13=fake if d.inter_dense else None, dense_w2=fake if d.inter_dense else None)
        st_, total = _ws(d, T)
        if st_ == B.MOE_UNSUPPORTED:
            return
        assert st_ == B.MOE_OK
        lay = B.WorkspaceLayout()
        assert lib.moe_forward_workspace_layout(C.byref(d), C.byref(ts), T, C.byref(lay)) == B.MOE_OK
        assert lay.path == lib.moe_forward_path(C.byref(d), T)
        Kp = d.top_k + d.n_shared
        if lay.path == 1:
            assert lay.capacity == T * Kp
        else:
            assert lay.capacity == lib.moe_permute_capacity(T, Kp, d.num_experts + d.n_shared, lay.block_m)
        bufs = _layout_extents(d, lay, T)
        for name, off, n in bufs:
            assert off % 256 == 0 and 0 <= off and off + n <= total, (name, off, n, total)
        ends = sorted((off, off + n, name) for name, off, n in bufs if n)
        for a, b in zip(ends, ends[1:]):
            assert a[1] <= b[0], f"{a[2]} and {b[2]} overlap"
        seen.append((lay.path, T))

    run()
    print(f"{len(seen)} layouts checked")
    assert {p for p, _ in seen} == {0, 1} and len(seen) >= 200, len(seen)


def _header_accepts(d):
    """The descriptor rules as include/moe.h states them (field comments, the
    routing limits of moe_route, and the 2 GiB rule for one expert's weights)."""
    H, E, K, I = d.hidden, d.num_experts, d.top_k, d.inter
    wd, f32 = d.weight_dtype, d.act_dtype == B.DT_F32
    rules = [
        0 < H <= 8192 and H % 64 == 0, 1 <= E <= 512, 1 <= K <= min(E, 64), I > 0 and I % 64 == 0,
        d.act in (0, 1), d.act_dtype in (B.DT_F32, B.DT_BF16),
        wd == B.DT_F32 if f32 else wd in (B.DT_BF16, B.DT_FP8, B.DT_MXFP4),
        d.router_mode in (0, 1), 0 <= d.n_shared <= 8,
        not (wd in (B.DT_FP8, B.DT_MXFP4) and d.n_shared), K + d.n_shared <= 64,
        d.inter_dense >= 0 and d.inter_dense % 64 == 0, not d.inter_dense or d.dense_act in (0, 1),
        d.eps >= 0, d.scoring in (0, 1), 0 <= d.n_groups <= 64, d.act_quant in (0, 1),
        not d.act_quant or (wd == B.DT_FP8 and not f32 and I <= 16384),
        d.block_tail in (0, 1), d.combine in (0, 1), not (d.combine == 1 and f32),
    ]
    if d.n_groups > 1:
        G, KG = d.n_groups, d.topk_groups
        rules += [E % G == 0, 1 <= KG <= G, KG * (E // G) >= K if E % G == 0 else False]
    wb = {B.DT_FP8: 1, B.DT_F32: 4}.get(wd, 2)
    if all(rules):  # the 32-bit offset rule, only meaningful for otherwise valid sizes
        rules += [2 * I * H * wb < 2 ** 31, 2 * d.inter_dense * H * 4 < 2 ** 31, E * H * 4 < 2 ** 31]
    return all(rules)


def test_descriptor_validation_follows_the_header():
    """20000 random descriptors, each field drawn mostly from valid values and
    sometimes from invalid ones: the library accepts exactly those the header's
    rules accept (besides a layer whose row padding alone passes 2 GiB, which the
    size query refuses by name), and every refusal carries a message."""
    import numpy as np
    lib = _lib()
    rng = np.random.default_rng(3)

    def pick(valid, invalid, p=0.08):
        return int(rng.choice(invalid)) if rng.random() < p else int(rng.choice(valid))

    accepted = 0
    for _ in range(20000):
        E = pick([1, 2, 8, 64, 128, 256, 512, int(rng.integers(1, 513))], [0, -1, 513, 1024])
        d = _desc(hidden=pick([64, 128, 2816, 4096, 8192], [0, -64, 32, 100, 8256, 16384]),
                  num_experts=E, top_k=pick([1, 2, 8, max(1, min(E, 64)), int(rng.integers(1, 65))], [0, -1, 65, 600]),
                  inter=pick([64, 512, 704, 14336, 16384, 16448, 65536], [0, -64, 100, 32]),
                  act=pick([0, 1], [2, -1]), act_dtype=pick([0, 1], [2, 3, -1]), weight_dtype=pick([0, 1, 2, 3], [4, -1]),
                  renormalize=pick([0, 1, 5], [0]), router_mode=pick([0, 1], [2, -1]),
                  n_shared=pick([0, 0, 1, 2, 8], [9, -1]), inter_dense=pick([0, 0, 64, 2112], [-64, 100]),
                  dense_act=pick([0, 1], [2, -1]),
                  eps=float(rng.choice([1e-6, 0.0])) if rng.random() > 0.05 else float(rng.choice([-1.0, np.nan])),
                  scoring=pick([0, 1], [2, -1]), n_groups=pick([0, 1, 2, 4, 8, 16, 64], [-1, 3, 65, 128]),
                  topk_groups=pick([0, 1, 2, 3, 4, 8], [-1, 65]), act_quant=pick([0, 1], [2, -1]),
                  block_tail=pick([0, 1], [2, -1]), combine=pick([0, 1], [2, -1]))
        st, _ = _ws(d, 16)
        msg = lib.moe_last_error()
        expect = _header_accepts(d)
        if expect and st == B.MOE_UNSUPPORTED and b"padded rows" in msg:
            Kp, Ep = d.top_k + d.n_shared, d.num_experts + d.n_shared
            assert (16 * Kp + Ep * 255) * d.inter * 4 >= 2 ** 31, msg  # padding at the largest row block
            continue
        assert (st == B.MOE_OK) == expect, (st, msg, {f: getattr(d, f) for f, _ in B.LayerDesc._fields_})
        assert st == B.MOE_OK or msg
        accepted += st == B.MOE_OK
    assert accepted >= 200, accepted


def test_route_validation_follows_the_header():
    """moe_route at T = 0 (nothing launches) over random options: accepted exactly
    when the header's limits hold (1 <= K <= E <= 512, K <= 64, a known scoring,
    no groups or 2..64 groups dividing E with 1..n_groups picked that hold at
    least K experts), and every refusal carries a message."""
    import numpy as np
    lib = _lib()
    rng = np.random.default_rng(4)
    accepted = 0
    for _ in range(20000):
        E = int(rng.choice([-1, 0, 1, 2, 7, 8, 64, 128, 256, 512, 513, int(rng.integers(1, 600))]))
        K = int(rng.choice([-1, 0, 1, 2, 5, 8, 64, 65, int(rng.integers(1, 80))]))
        scoring = int(rng.choice([0, 1, 1, 2, -1]))
        G = int(rng.choice([-1, 0, 1, 2, 3, 4, 8, 16, 64, 65, 128]))
        KG = int(rng.choice([-1, 0, 1, 2, 3, 4, 8, 64, 65]))
        ok = 1 <= K <= E <= 512 and K <= 64 and scoring in (0, 1) and 0 <= G <= 64
        if ok and G > 1:
            ok = E % G == 0 and 1 <= KG <= G and KG * (E // G) >= K
        st = lib.moe_route(None, 0, E, K, 1, scoring, G, KG, None, None, None, None)
        assert (st == B.MOE_OK) == ok, (E, K, scoring, G, KG, st, lib.moe_last_error())
        assert st == B.MOE_OK or lib.moe_last_error()
        accepted += ok
    assert accepted >= 1000, accepted


def test_permute_capacity_follows_the_header_formula():
    """floor((T*K + E*(block_m-1)) / block_m) * block_m for valid arguments, -1 for
    T < 0, K < 1, E < 1 or a block_m that is not a power of two in [16, 256]; the
    capacity always holds every slot plus each expert's padding."""
    import numpy as np
    lib = _lib()
    rng = np.random.default_rng(6)
    for _ in range(20000):
        T = int(rng.choice([-1, 0, 1, 16, 17, int(rng.integers(0, 1 << 20))]))
        K = int(rng.choice([-1, 0, 1, 2, 8, 64, int(rng.integers(1, 65))]))
        E = int(rng.choice([-1, 0, 1, 8, 128, 1024, int(rng.integers(1, 1025))]))
        bm = int(rng.choice([-16, 0, 8, 16, 32, 48, 64, 128, 256, 512, int(rng.integers(1, 300))]))
        got = lib.moe_permute_capacity(T, K, E, bm)
        valid = T >= 0 and K >= 1 and E >= 1 and bm in (16, 32, 64, 128, 256)
        if not valid:
            assert got == -1, (T, K, E, bm, got)
            continue
        assert got == (T * K + E * (bm - 1)) // bm * bm, (T, K, E, bm, got)
        assert got % bm == 0 and got >= T * K
