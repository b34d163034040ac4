"""Comparison helpers shared by the GPU parity tests."""
import numpy as np
import torch

# Output tolerances: (max-abs, rel-RMS) for bf16 and fp8-weight layers; fp32 layers
# are held to 1e-5 relative: max-abs <= 1e-5 * max|ref| and rel-RMS <= 1e-5.
TOL = {"bf16": (2e-2, 1e-2), "fp8": (5e-2, 3e-2)}
TOL_F32_REL = 1e-5
TOPK_W_REL = 1e-6


def to64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().float().cpu().numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)


def errors(got, ref):
    got, ref = to64(got), to64(ref)
    d = got - ref
    max_abs = float(np.abs(d).max()) if d.size else 0.0
    rms_ref = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    rel_rms = float(np.sqrt(np.mean(d * d)) / rms_ref) if rms_ref > 0 else 0.0
    return max_abs, rel_rms, float(np.abs(ref).max()) if ref.size else 0.0


def assert_close(got, ref, kind, what=""):
    max_abs, rel_rms, ref_max = errors(got, ref)
    if kind == "fp32":
        ok = max_abs <= TOL_F32_REL * ref_max and rel_rms <= TOL_F32_REL
        bound = (TOL_F32_REL * ref_max, TOL_F32_REL)
    else:
        bound = TOL[kind]
        ok = max_abs <= bound[0] and rel_rms <= bound[1]
    assert ok, (f"{what}: max-abs {max_abs:.3e} rel-RMS {rel_rms:.3e} exceed {bound} "
                f"(max|ref| {ref_max:.3f})")
    return max_abs, rel_rms


def assert_weights_close(got, ref, what="topk_w"):
    got, ref = to64(got), to64(ref)
    rel = np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30)
    assert rel.max() <= TOPK_W_REL, f"{what}: max rel err {rel.max():.3e} > {TOPK_W_REL}"
