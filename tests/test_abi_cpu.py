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
    assert lib.moe_permute(fake, 4, 2, 8, 48, fake, fake, fake, fake, None) == B.MOE_INVALID_ARG
    assert lib.moe_permute(fake, 4, 2, 8, 512, fake, fake, fake, fake, None) == B.MOE_INVALID_ARG
    assert lib.moe_permute(fake, 4, 0, 8, 64, fake, fake, fake, fake, None) == B.MOE_INVALID_ARG
    assert lib.moe_permute(fake, 4, 2, 8, 64, None, fake, fake, fake, None) == B.MOE_INVALID_ARG


def test_permute_capacity():
    lib = _lib()
    assert lib.moe_permute_capacity(128, 8, 128, 64) == (1024 + 128 * 63) // 64 * 64
    assert lib.moe_permute_capacity(1, 1, 1, 16) == 16
    assert lib.moe_permute_capacity(4, 2, 8, 48) == -1
    assert lib.moe_permute_capacity(-1, 2, 8, 64) == -1


def test_fp8_activation_layers_take_the_grouped_path():
    lib = _lib()
    d = _desc(act_quant=1, weight_dtype=B.DT_FP8)
    assert [lib.moe_forward_path(C.byref(d), t) for t in (1, 4, 16, 4096)] == [0, 0, 0, 0]
    d0 = _desc(weight_dtype=B.DT_FP8)
    assert lib.moe_forward_path(C.byref(d0), 4) == 1
    # the workspace holds the codes and scales of x and h as well
    st0, n0 = _ws(d0, 4096)
    st1, n1 = _ws(d, 4096)
    assert st0 == st1 == B.MOE_OK and n1 > n0 + 4096 * 256


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
