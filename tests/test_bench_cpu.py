"""bench.py's host logic on the CPU: the one-GPU contract and the algorithmic
work it divides by the measured times (closed forms of the layer shapes)."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from mixture_experts_ffn_router_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_prefill_flop_closed_forms():
    """Mixtral-style layer, T=4096, top-2 of 8, H=4096, I=14336: the gate/up GEMM
    does 2*T*K*H*2I FLOP and the down GEMM 2*T*K*I*H; the router 2*T*E*H."""
    s = W.SPECS["mixtral"]
    T = 4096
    fl, by = bench.stage_work(s, T, np.full(s.E, T * s.K // s.E), "grouped")
    assert fl["gate_up"] == 2 * T * 2 * 4096 * 2 * 14336 == 1_924_145_348_608
    assert fl["down"] == fl["gate_up"] // 2
    assert fl["router"] == 2 * T * 8 * 4096
    # the whole layer: 2*T*H*E + 6*T*K*H*I = 2.886e12 FLOP
    assert abs(sum(fl.values()) - 2.886e12) / 2.886e12 < 1e-3
    # weights are counted once: every expert's w13 (2I x H bf16) in the gate/up bytes
    assert by["gate_up"] >= 8 * 2 * 14336 * 4096 * 2


def test_decode_bytes_gemma_t1():
    """Gemma-style layer at T=1 with 8 experts picked: 8 x 3 x H x I bf16 expert
    weights (95.2 MB), the dense MLP 3 x H x 2112 (35.7 MB) and the router E x H
    (0.72 MB): about 131.6 MB a step, activations aside."""
    s = W.SPECS["gemma"]
    counts = np.zeros(s.E, dtype=np.int64)
    counts[:8] = 1
    fl, by = bench.stage_work(s, 1, counts, "decode", dense_stage="gate_up")
    experts = 8 * 3 * 2816 * 704 * 2
    dense = 3 * 2816 * 2112 * 2
    router = 128 * 2816 * 2
    assert experts == 95_158_272 and dense == 35_684_352 and router == 720_896
    total = sum(by.values())
    assert experts + dense + router <= total <= (experts + dense + router) * 1.01


def test_decode_bytes_mxfp4_half_a_byte_and_a_scale_per_32():
    s = W.SPECS["gemma_mxfp4"]
    counts = np.zeros(s.E, dtype=np.int64)
    counts[:8] = 1
    _, by4 = bench.stage_work(s, 1, counts, "decode", dense_stage="gate_up")
    _, by16 = bench.stage_work(W.SPECS["gemma"], 1, counts, "decode", dense_stage="gate_up")
    H, I = 2816, 704
    w4 = 8 * (2 * I * (H // 2 + H // 32) + H * (I // 2 + I // 32))
    w16 = 8 * 3 * H * I * 2
    # only the expert weights differ between the two layers
    assert sum(by16.values()) - sum(by4.values()) == pytest.approx(w16 - w4, abs=1)


def test_rooflines_follow_the_configurations_split():
    """Prefill-sized token counts are rated by FLOP against the MFMA peak of the
    contraction's dtype, decode-sized ones (T <= 128) by bytes against HBM."""
    S = W.SPECS
    assert bench.roofline_class(S["mixtral"], 4096, "gate_up") == ("mfma", 2500.0)
    assert bench.roofline_class(S["gemma"], 8192, "gate_up") == ("mfma", 2500.0)
    assert bench.roofline_class(S["deepseek_v3"], 8192, "gate_up") == ("mfma", 2500.0)
    assert bench.roofline_class(S["gemma_w8a8"], 8192, "down") == ("mfma", 5000.0)
    assert bench.roofline_class(S["mixtral_w8a8"], 4096, "gate_up") == ("mfma", 5000.0)
    # the dense MLP of an FP8-activation layer stays bf16
    assert bench.roofline_class(S["gemma_w8a8"], 8192, "dense_gate_up") == ("mfma", 2500.0)
    for T in (1, 16, 128):
        assert bench.roofline_class(S["gemma"], T, "gate_up") == ("hbm", 8000.0)
    assert bench.roofline_class(S["skewed_w8a8"], 1, "gate_up") == ("hbm", 8000.0)
    assert bench.roofline_class(S["tiny"], 64, "gate_up")[0] == "alu"


def test_combine_bytes_are_the_combined_rows():
    """The down GEMM with its weighted combine reads h and writes one combined row
    per token; the per-slot rows a design keeps in between are not algorithmic."""
    s = W.SPECS["gemma"]
    T = 8192
    counts = np.full(s.E, T * s.K // s.E)
    _, by = bench.stage_work(s, T, counts, "grouped")
    H, I, E, K = 2816, 704, 128, 8
    assert by["down"] == E * H * I * 2 + T * K * I * 2 + T * H * 4
    assert by["finalize"] == T * H * 4 + T * H * 4 + T * H * 2
