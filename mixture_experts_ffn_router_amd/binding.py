"""ctypes binding of libmoe_mi355x.so: argument marshalling only.

Every step of the layer runs in the HIP library; this module checks tensor
dtypes, shapes and devices, passes raw device pointers and the current HIP
stream, and turns status codes into exceptions.  There is no fallback: when
the library is missing or was built for nothing, using any function raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_mi355x.so")

MOE_OK, MOE_INVALID_ARG, MOE_UNSUPPORTED, MOE_WORKSPACE_TOO_SMALL, MOE_HIP_ERROR = range(5)
ACT = {"silu": 0, "gelu_tanh": 1}
DT_F32, DT_BF16, DT_FP8, DT_MXFP4 = 0, 1, 2, 3
ROUTER_PLAIN, ROUTER_GEMMA = 0, 1
SCORING = {"softmax": 0, "sigmoid": 1}
ACT_QUANT = {None: 0, "fp8_dynamic": 1}


class MoEError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


_STATUS = {0: "MOE_OK", 1: "MOE_INVALID_ARG", 2: "MOE_UNSUPPORTED", 3: "MOE_WORKSPACE_TOO_SMALL",
           4: "MOE_HIP_ERROR"}


class LayerDesc(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("num_experts", C.c_int32), ("top_k", C.c_int32),
                ("inter", C.c_int32), ("act", C.c_int32), ("act_dtype", C.c_int32),
                ("weight_dtype", C.c_int32), ("renormalize", C.c_int32), ("router_mode", C.c_int32),
                ("n_shared", C.c_int32), ("inter_dense", C.c_int32), ("dense_act", C.c_int32),
                ("eps", C.c_float), ("scoring", C.c_int32), ("n_groups", C.c_int32),
                ("topk_groups", C.c_int32), ("act_quant", C.c_int32), ("block_tail", C.c_int32),
                ("combine", C.c_int32)]
COMBINE = {"slot_order": 0, "atomic": 1}


class Tensors(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "x", "logits", "w_router", "router_scale", "per_expert_scale", "w13", "w2", "w13_scale",
        "w2_scale", "shared_w13", "shared_w2", "dense_w13", "dense_w2", "gamma_pre", "gamma_pre2",
        "gamma_post1", "gamma_post2", "out", "logits_out", "topk_w_out", "topk_ids_out", "out_f32",
        "gamma_post_ff")]


class WorkspaceLayout(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("path", "block_m", "slots_per_token", "y_parts", "y_f32")] + \
               [(n, C.c_int64) for n in ("capacity", "topk_w", "topk_ids", "counts", "offsets", "sorted_slots",
                                         "block_expert", "slot_row", "inv_rms", "x_expert", "h", "y", "x_codes",
                                         "x_scales", "h_codes", "h_scales")]


EXPORTS = ["moe_status_string", "moe_last_error", "moe_route", "moe_permute_capacity", "moe_permute",
           "moe_forward_workspace_size", "moe_forward", "moe_forward_profiled", "moe_forward_path",
           "moe_decode_dense_gate_up_stage", "moe_forward_workspace_layout", "moe_forward_noalloc"]
NOALLOC_SCRATCH_BYTES = 64 << 20
PATHS = {0: "grouped", 1: "decode"}
STAGES = ["prenorm", "router", "route", "permute", "quant_x", "gate_up", "quant_h", "down", "dense_gate_up",
          "dense_down", "finalize"]

_lib = None


def load(path: Optional[str] = None):
    """Load the library (once; `path` defaults to LIB_PATH, read at call time).
    Raises if it is missing: there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    path = LIB_PATH if path is None else path
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          f"`python -m mixture_experts_ffn_router_amd.build`")
    lib = C.CDLL(path)
    lib.moe_status_string.restype = C.c_char_p
    lib.moe_status_string.argtypes = [C.c_int]
    lib.moe_last_error.restype = C.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_route.restype = C.c_int
    lib.moe_route.argtypes = [C.c_void_p, C.c_int64, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                              C.c_int32, C.c_int32, C.c_void_p,
                              C.c_void_p, C.c_void_p, C.c_void_p]
    lib.moe_permute_capacity.restype = C.c_int64
    lib.moe_permute_capacity.argtypes = [C.c_int64, C.c_int32, C.c_int32, C.c_int32]
    lib.moe_permute.restype = C.c_int
    lib.moe_permute.argtypes = [C.c_void_p, C.c_int64, C.c_int32, C.c_int32, C.c_int32, C.c_void_p,
                                C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
    lib.moe_forward_workspace_size.restype = C.c_int
    lib.moe_forward_workspace_size.argtypes = [C.POINTER(LayerDesc), C.c_int64, C.POINTER(C.c_size_t)]
    lib.moe_forward.restype = C.c_int
    lib.moe_forward.argtypes = [C.POINTER(LayerDesc), C.POINTER(Tensors), C.c_int64, C.c_void_p,
                                C.c_size_t, C.c_void_p]
    lib.moe_forward_profiled.restype = C.c_int
    lib.moe_forward_profiled.argtypes = [C.POINTER(LayerDesc), C.POINTER(Tensors), C.c_int64, C.c_void_p,
                                         C.c_size_t, C.c_void_p, C.POINTER(C.c_void_p)]
    lib.moe_forward_path.restype = C.c_int32
    lib.moe_forward_path.argtypes = [C.POINTER(LayerDesc), C.c_int64]
    lib.moe_forward_noalloc.restype = C.c_int
    lib.moe_forward_noalloc.argtypes = [C.POINTER(LayerDesc), C.POINTER(Tensors), C.c_int64, C.c_void_p]
    lib.moe_forward_workspace_layout.restype = C.c_int
    lib.moe_forward_workspace_layout.argtypes = [C.POINTER(LayerDesc), C.POINTER(Tensors), C.c_int64,
                                                 C.POINTER(WorkspaceLayout)]
    lib.moe_decode_dense_gate_up_stage.restype = C.c_int32
    lib.moe_decode_dense_gate_up_stage.argtypes = [C.POINTER(LayerDesc), C.c_int64]
    _lib = lib
    return lib


def _check(status):
    if status != MOE_OK:
        raise MoEError(status, load().moe_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dev(t, name, dtype=None, shape=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


# ----------------------------------------------------------------------------- moe_route

def route(logits: torch.Tensor, k: int, renormalize: bool = True,
          per_expert_scale: Optional[torch.Tensor] = None, out=None, scoring: str = "softmax",
          n_groups: int = 0, topk_groups: int = 0):
    """moe_route: (topk_w fp32 [T,k], topk_ids int32 [T,k]) from fp32 logits [T,E]."""
    lib = load()
    T, E = logits.shape
    _dev(logits, "logits", torch.float32)
    _dev(per_expert_scale, "per_expert_scale", torch.float32, (E,))
    if out is None:
        w = torch.empty(T, k, dtype=torch.float32, device=logits.device)
        ids = torch.empty(T, k, dtype=torch.int32, device=logits.device)
    else:
        w, ids = out
    _check(lib.moe_route(_ptr(logits), T, E, k, int(bool(renormalize)), SCORING[scoring], n_groups,
                         topk_groups, _ptr(per_expert_scale),
                         _ptr(w), _ptr(ids), _stream()))
    return w, ids


# ----------------------------------------------------------------------------- moe_permute

def permute_capacity(T, k, E, block_m):
    return int(load().moe_permute_capacity(T, k, E, block_m))


def permute(topk_ids: torch.Tensor, num_experts: int, block_m: int = 64):
    """moe_permute: dict(counts [E], offsets [E+1], sorted_slots [cap], block_expert [cap/block_m],
    num_padded [1], slot_row [T*k])."""
    lib = load()
    T, k = topk_ids.shape
    _dev(topk_ids, "topk_ids", torch.int32)
    cap = permute_capacity(T, k, num_experts, block_m)
    if cap < 0:
        raise MoEError(MOE_INVALID_ARG, "bad permute arguments")
    dev = topk_ids.device
    counts = torch.empty(num_experts, dtype=torch.int32, device=dev)
    offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
    sorted_slots = torch.full((max(cap, 1),), -7, dtype=torch.int32, device=dev)
    block_expert = torch.full((max(cap // block_m, 1),), -7, dtype=torch.int32, device=dev)
    num_padded = torch.full((1,), -7, dtype=torch.int32, device=dev)
    slot_row = torch.full((max(T * k, 1),), -7, dtype=torch.int32, device=dev)
    _check(lib.moe_permute(_ptr(topk_ids), T, k, num_experts, block_m, _ptr(counts), _ptr(offsets),
                           _ptr(sorted_slots), _ptr(block_expert), _ptr(num_padded), _ptr(slot_row),
                           _stream()))
    return dict(counts=counts, offsets=offsets, sorted_slots=sorted_slots[:cap],
                block_expert=block_expert[:cap // block_m], num_padded=num_padded,
                slot_row=slot_row[:T * k], capacity=cap)


# ----------------------------------------------------------------------------- moe_forward

class DeviceLayer:
    """Device tensors plus the C descriptor of one MoE layer."""

    def __init__(self, desc: LayerDesc, tensors: dict):
        self.desc = desc
        self.t = tensors  # name -> device tensor or None

    @property
    def act_dtype(self):
        return torch.float32 if self.desc.act_dtype == DT_F32 else torch.bfloat16

    @classmethod
    def from_generated(cls, L: dict, device="cuda", eps: float = 1e-6, combine: str = "slot_order"):
        """Build from a workloads.make_layer() dict (CPU tensors in storage dtypes).
        combine: "slot_order" (deterministic) or "atomic" (moe_combine)."""
        spec = L["spec"]
        f32 = spec.wdtype == "fp32"
        desc = LayerDesc(hidden=spec.H, num_experts=spec.E, top_k=spec.K, inter=spec.I,
                         act=ACT[spec.act], act_dtype=DT_F32 if f32 else DT_BF16,
                         weight_dtype={"fp32": DT_F32, "bf16": DT_BF16, "fp8": DT_FP8, "mxfp4": DT_MXFP4}[spec.wdtype],
                         renormalize=int(spec.renorm),
                         router_mode=ROUTER_GEMMA if spec.router_mode == "gemma" else ROUTER_PLAIN,
                         n_shared=spec.n_shared, inter_dense=spec.I_dense, dense_act=ACT[spec.act],
                         eps=eps, scoring=SCORING[spec.scoring], n_groups=spec.n_groups,
                         topk_groups=spec.topk_groups, act_quant=ACT_QUANT[spec.act_quant],
                         block_tail=int(spec.block_tail), combine=COMBINE[combine])

        def d(t):
            return None if t is None else t.to(device, non_blocking=False).contiguous()

        g = L.get("gammas") or {}
        t = dict(x=d(L["x"]), logits=d(L.get("logits")), w_router=d(L["w_router"]),
                 router_scale=d(L.get("router_scale")), per_expert_scale=d(L["per_expert_scale"]),
                 w13=d(L["w13"]), w2=d(L["w2"]), w13_scale=d(L["w13_scale"]), w2_scale=d(L["w2_scale"]),
                 shared_w13=d(L["shared_w13"]), shared_w2=d(L["shared_w2"]),
                 dense_w13=d(L["dense_w13"]), dense_w2=d(L["dense_w2"]),
                 gamma_pre=d(g.get("pre")), gamma_pre2=d(g.get("pre2")),
                 gamma_post1=d(g.get("post1")), gamma_post2=d(g.get("post2")),
                 gamma_post_ff=d(g.get("post_ff")) if spec.block_tail else None)
        return cls(desc, t)

    def path(self, T):
        """Which execution path moe_forward takes for T tokens: "grouped" or "decode"."""
        r = load().moe_forward_path(C.byref(self.desc), T)
        if r < 0:
            raise ValueError("invalid layer descriptor or T")
        return PATHS[r]

    def dense_gate_up_stage(self, T):
        """Stage name whose launch runs the dense gate/up on the decode path, or None."""
        r = load().moe_decode_dense_gate_up_stage(C.byref(self.desc), T)
        return None if r < 0 else STAGES[r]

    def workspace_size(self, T):
        n = C.c_size_t(0)
        _check(load().moe_forward_workspace_size(C.byref(self.desc), T, C.byref(n)))
        return n.value

    def forward(self, x: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = "layer",
                out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                want_routing: bool = False, events=None, want_intermediates: bool = False,
                noalloc: bool = False):
        """moe_forward.  Returns out [T,H]; with want_routing also a dict of the
        logits, topk_w, topk_ids and out_f32 (the output before its final rounding).
        events: optional list of len(STAGES)+1 recorded torch.cuda.Event objects; the
        library records them between its stages (moe_forward_profiled).
        want_intermediates (with want_routing): the dict also holds "ws", views of
        the call's intermediates in its workspace (moe_forward_workspace_layout).
        noalloc: call moe_forward_noalloc (the library's static scratch, no workspace)."""
        lib = load()
        t = self.t
        x = t["x"] if x is None else x
        if isinstance(logits, str):
            logits = t["logits"]
        T, H = x.shape
        E, K = self.desc.num_experts, self.desc.top_k
        _dev(x, "x", self.act_dtype, (T, self.desc.hidden))
        _dev(logits, "logits", torch.float32, (T, E))
        if out is None:
            out = torch.empty(T, H, dtype=self.act_dtype, device=x.device)
        _dev(out, "out", self.act_dtype, (T, H))
        if noalloc:
            if events is not None or want_intermediates:
                raise ValueError("the no-allocation entry point takes no events and keeps no workspace")
        else:
            ws_bytes = self.workspace_size(T)
            if workspace is None or workspace.numel() < ws_bytes:
                workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
        extra = {}
        if want_routing:
            extra = dict(logits=torch.empty(T, E, dtype=torch.float32, device=x.device),
                         topk_w=torch.empty(T, K, dtype=torch.float32, device=x.device),
                         topk_ids=torch.empty(T, K, dtype=torch.int32, device=x.device),
                         out_f32=torch.empty(T, H, dtype=torch.float32, device=x.device))
        ts = Tensors(x=_ptr(x), logits=_ptr(logits), out=_ptr(out),
                     logits_out=_ptr(extra.get("logits")), topk_w_out=_ptr(extra.get("topk_w")),
                     topk_ids_out=_ptr(extra.get("topk_ids")), out_f32=_ptr(extra.get("out_f32")),
                     **{k: _ptr(t.get(k)) for k in (
                         "w_router", "router_scale", "per_expert_scale", "w13", "w2", "w13_scale",
                         "w2_scale", "shared_w13", "shared_w2", "dense_w13", "dense_w2", "gamma_pre",
                         "gamma_pre2", "gamma_post1", "gamma_post2", "gamma_post_ff")})
        if noalloc:
            _check(lib.moe_forward_noalloc(C.byref(self.desc), C.byref(ts), T, _stream()))
        elif events is None:
            _check(lib.moe_forward(C.byref(self.desc), C.byref(ts), T, _ptr(workspace), workspace.numel(),
                                   _stream()))
        else:
            if len(events) != len(STAGES) + 1:
                raise ValueError(f"need {len(STAGES) + 1} events")
            arr = (C.c_void_p * len(events))(*[e._as_parameter_.value for e in events])
            _check(lib.moe_forward_profiled(C.byref(self.desc), C.byref(ts), T, _ptr(workspace),
                                            workspace.numel(), _stream(), arr))
        if want_intermediates:
            extra["ws"] = self._intermediates(ts, T, workspace)
        if want_routing:
            return out, extra
        return out

    def _intermediates(self, ts, T, workspace):
        lay = WorkspaceLayout()
        _check(load().moe_forward_workspace_layout(C.byref(self.desc), C.byref(ts), T, C.byref(lay)))
        d = self.desc
        kp, cap, H, I = lay.slots_per_token, lay.capacity, d.hidden, d.inter
        act = self.act_dtype
        ydt = torch.float32 if lay.y_f32 else act

        def view(off, dtype, shape):
            if off < 0:
                return None
            n = 1
            for v in shape:
                n *= v
            nb = n * torch.empty((), dtype=dtype).element_size()
            return workspace[off:off + nb].view(dtype).view(*shape)

        return dict(
            path=PATHS[lay.path], block_m=lay.block_m, slots_per_token=kp, y_parts=lay.y_parts,
            y_f32=bool(lay.y_f32), capacity=cap,
            topk_w=view(lay.topk_w, torch.float32, (T, kp)), topk_ids=view(lay.topk_ids, torch.int32, (T, kp)),
            counts=view(lay.counts, torch.int32, (d.num_experts + d.n_shared,)),
            offsets=view(lay.offsets, torch.int32, (d.num_experts + d.n_shared + 1,)),
            sorted_slots=view(lay.sorted_slots, torch.int32, (cap,)),
            block_expert=view(lay.block_expert, torch.int32, (cap // max(lay.block_m, 1),)),
            slot_row=view(lay.slot_row, torch.int32, (T * kp,)),
            inv_rms=view(lay.inv_rms, torch.float32, (T,)),
            x_expert=view(lay.x_expert, act, (T, H)),
            h=view(lay.h, act, (cap, I)),
            y=view(lay.y, ydt, (T, H) if lay.y_parts == 0 else (T * kp * lay.y_parts, H)),
            x_codes=view(lay.x_codes, torch.uint8, (T, H)), x_scales=view(lay.x_scales, torch.float32, (T,)),
            h_codes=view(lay.h_codes, torch.uint8, (cap, I)), h_scales=view(lay.h_scales, torch.float32, (cap,)))
