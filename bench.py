#!/usr/bin/env python3
"""Benchmark of the MoE FFN layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config mixtral] [--T N]

One step is one moe_forward call (router logits -> routing -> permutation ->
grouped gate/up GEMM + gated activation -> grouped down GEMM + weighted
combine -> finalize) over one batch of T synthetic tokens whose inputs and
weights are already resident in HBM.  The default workload is the Mixtral-style
layer (T=4096, H=4096, E=8, top-2, I=14336, SwiGLU, bf16).

Prints one JSON line:
  value        tokens/s of the whole step (HIP events around K back-to-back steps)
  roofline     the dominant kernel's algorithmic FLOP (or bytes) per launch over its
               average duration, timed with HIP events that the library records on
               its launch stream between stages, against MI355X's published peak
  cpu_baseline the float64 CPU oracle on a bounded row sample of the same workload
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "MoE layer tokens/s; prefill TFLOP/s % MFMA peak; decode GB/s % HBM peak"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="mixtral")
    ap.add_argument("--T", type=int, default=None)
    ap.add_argument("--cpu-rows", type=int, default=None, help="oracle row sample (default per config)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def stage_work(spec, T, counts=None):
    """Algorithmic FLOP and HBM bytes per stage (padding and skipped experts not counted)."""
    H, E, K, I = spec.H, spec.E, spec.K, spec.I
    S, Is, Id = spec.n_shared, spec.I_shared, spec.I_dense
    wb = 1 if spec.wdtype == "fp8" else (4 if spec.wdtype == "fp32" else 2)
    ab = 4 if spec.wdtype == "fp32" else 2
    rows = T * K
    fl = {}
    fl["router"] = 0 if spec.supplied_logits else 2 * T * E * H
    fl["gate_up"] = 2 * rows * H * 2 * I + 2 * T * S * H * 2 * Is
    fl["down"] = 2 * rows * I * H + 2 * T * S * Is * H
    fl["dense_gate_up"] = 2 * T * H * 2 * Id
    fl["dense_down"] = 2 * T * Id * H
    # weights actually touched: experts with at least one row
    used = E if counts is None else int((counts > 0).sum())
    by = {}
    by["gate_up"] = used * 2 * I * H * wb + S * 2 * Is * H * ab + T * H * ab + rows * I * ab
    by["down"] = used * H * I * wb + S * H * Is * ab + rows * I * ab + (rows + T * S) * H * ab
    by["router"] = 0 if spec.supplied_logits else E * H * ab + T * H * ab + T * E * 4
    by["dense_gate_up"] = 2 * Id * H * ab + T * H * ab + T * Id * ab
    by["dense_down"] = H * Id * ab + T * Id * ab + T * H * 4
    return fl, by


def cpu_baseline(L, rows_n):
    import numpy as np
    from mixture_experts_ffn_router_amd import workloads as W
    from oracle import moe_oracle as O
    try:
        import threadpoolctl
        threads = max((d.get("num_threads", 1) for d in threadpoolctl.threadpool_info()), default=1)
    except Exception:
        threads = None
    T = L["T"]
    rows = np.sort(np.random.default_rng(0).choice(T, min(rows_n, T), replace=False))
    layer = W.oracle_layer(L)
    x = L["x"].float().numpy().astype(np.float64)
    logits = None if L["logits"] is None else L["logits"].numpy().astype(np.float64)
    t0 = time.perf_counter()
    O.moe_layer(x, layer, rows=rows, logits=logits)
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    return {"value": len(rows) / dt, "unit": "tokens/s", "cores": threads or cores, "kind": "oracle",
            "sample": f"{len(rows)} of {T} token rows through the experts (routing and permutation "
                      f"over all {T}); {dt:.1f} s on {cores} host cores, numpy BLAS threads {threads}"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from mixture_experts_ffn_router_amd import binding as B
    from mixture_experts_ffn_router_amd import workloads as W

    B.load()
    spec = W.SPECS[args.config]
    T = args.T or spec.T
    spec = spec.with_T(T)
    L = W.make_layer(spec, seed=0)
    dl = B.DeviceLayer.from_generated(L)
    act_dtype = dl.act_dtype
    out = torch.empty(T, spec.H, dtype=act_dtype, device="cuda")
    ws = torch.empty(dl.workspace_size(T), dtype=torch.uint8, device="cuda")
    print(f"[bench] {spec.name} T={T}: warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        dl.forward(out=out, workspace=ws)
    torch.cuda.synchronize()

    # timed region: K back-to-back steps
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for _ in range(args.steps):
        dl.forward(out=out, workspace=ws)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    print(f"[bench] {ms_per_step:.4f} ms/step (wall {1e3 * wall / args.steps:.4f})", file=sys.stderr, flush=True)

    # per-stage durations: the same K steps with events recorded by the library between stages
    nev = len(B.STAGES) + 1
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    for row in evs:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    _, routing = dl.forward(out=out, workspace=ws, want_routing=True)
    counts = torch.bincount(routing["topk_ids"].flatten().long(), minlength=spec.E).cpu().numpy()
    torch.cuda.synchronize()
    p0 = torch.cuda.Event(enable_timing=True)
    p1 = torch.cuda.Event(enable_timing=True)
    p0.record()
    for row in evs:
        dl.forward(out=out, workspace=ws, events=row)
    p1.record()
    torch.cuda.synchronize()
    prof_ms = p0.elapsed_time(p1) / args.steps
    stage_ms = {name: sum(row[i].elapsed_time(row[i + 1]) for row in evs) / args.steps
                for i, name in enumerate(B.STAGES)}

    fl, by = stage_work(spec, T, counts)
    total_flop = sum(fl.values())
    gemm_stages = [s for s in ("gate_up", "down", "dense_gate_up", "dense_down", "router") if fl[s] > 0]
    dom = max(gemm_stages, key=lambda s: stage_ms[s])
    dom_s = stage_ms[dom] / 1e3
    intensity = fl[dom] / max(by[dom], 1)
    # ridge point of MI355X: 2500e12 / 8e12 = 312 FLOP/byte
    if intensity >= PEAK_BF16_TFLOPS / PEAK_HBM_GBS * 1e3:
        achieved = fl[dom] / dom_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None}
    else:
        achieved = by[dom] / dom_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None}
    roof.update({"kernel": dom, "kernel_ms": round(stage_ms[dom], 5),
                 "algorithmic_per_launch": fl[dom] if roof["bound"] == "mfma" else by[dom]})

    line = {
        "metric": METRIC,
        "value": round(T / (ms_per_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp32": "f32", "bf16": "bf16", "fp8": "fp8-e4m3 weights, bf16 activations"}[spec.wdtype],
        "data": "synthetic",
        "config": {"workload": f"{spec.name} MoE FFN layer forward", "T": T, "hidden": spec.H,
                   "experts": spec.E, "top_k": spec.K, "inter": spec.I, "act": spec.act,
                   "shared": spec.n_shared, "dense_inter": spec.I_dense},
        "step_tflops": round(total_flop / (ms_per_step / 1e3) / 1e12, 2),
        "stages_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "profiled_ms_per_step": round(prof_ms, 5),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        rows_n = args.cpu_rows or (256 if T > 256 else T)
        print(f"[bench] cpu oracle on {rows_n} rows", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(L, rows_n)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
