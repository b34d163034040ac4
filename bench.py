#!/usr/bin/env python3
"""Benchmark of the MoE FFN layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config mixtral] [--T N]

One step is one moe_forward call over one batch of T synthetic tokens whose
inputs and weights are already resident in HBM: router logits -> routing ->
(grouped path: permutation -> grouped gate/up GEMM + gated activation -> grouped
down GEMM + weighted combine -> finalize; decode path, T <= 16: fused weight-
streaming kernels).  The default workload is the Mixtral-style layer (T=4096,
H=4096, E=8, top-2, I=14336, SwiGLU, bf16).

Decode-path workloads rotate over several copies of the layer whose experts are
permuted differently (at least 4 copies and 512 MB of weights), so a step never
finds the experts it reads in the 256 MB last-level cache from the step before.

Prints one JSON line:
  value        tokens/s of the whole step (HIP events around K back-to-back steps)
  roofline     the dominant kernel's algorithmic FLOP (or bytes) per launch over its
               average duration, timed with HIP events that the library records on
               its launch stream between stages (less the cost of one event record,
               measured in the same run), against MI355X's published peak
  cpu_baseline the float64 CPU oracle on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))

METRIC = "MoE layer tokens/s; prefill TFLOP/s % MFMA peak; decode GB/s % HBM peak"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA (the FP8-activation layers' contraction)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
PEAK_F32_TFLOPS = 157.3    # MI355X fp32 vector FMA
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="mixtral")
    ap.add_argument("--T", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for the HBM byte counters)")
    return ap.parse_args()


# Kernel sources whose change invalidates stored HBM byte counts, per path.
KERNEL_SOURCES = {"grouped": ["gemm.hip"], "decode": ["decode.hip"]}


def source_digest(path):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[path]:
        with open(os.path.join(ROOT, "mixture_experts_ffn_router_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload, kernel, path):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by the copy calibration), or None when
    there is none or the kernel source changed since it was taken."""
    f = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(f):
        return None
    with open(f) as fh:
        rec = json.load(fh).get(f"{workload}/{kernel}")
    if not rec or rec.get("source_digest") != source_digest(path):
        return None
    return rec["bytes_per_launch"]


def copy_calibration():
    """A plain device-to-device copy of 1 GiB, five times: its FETCH_SIZE and
    WRITE_SIZE per dispatch against the 1 GiB it moves give the counters' scale."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "dispatches": 5}), flush=True)


def stage_work(spec, T, counts, path, dense_stage=None):
    """Algorithmic FLOP and HBM bytes per stage of the library's stage events.
    Padding and experts nobody picked are not counted; weights count once.
    dense_stage: decode path only, the stage whose launch runs the dense gate/up."""
    H, E, K, I = spec.H, spec.E, spec.K, spec.I
    S, Id = spec.n_shared, spec.I_dense
    wb = {"fp8": 1, "fp32": 4, "bf16": 2, "mxfp4": 0.5}[spec.wdtype]
    ab = 4 if spec.wdtype == "fp32" else 2
    sb = 4 if spec.wdtype == "fp8" else 0  # fp32 scale per output channel
    mx = spec.wdtype == "mxfp4"            # MXFP4: one scale byte per 32 along the reduction
    Kp = K + S
    rows = T * K
    used = int((counts > 0).sum())
    z = 0 if spec.supplied_logits else 1
    fl = {s: 0 for s in ("router", "gate_up", "down", "dense_gate_up", "dense_down")}
    fl["router"] = z * 2 * T * E * H
    fl["gate_up"] = 2 * rows * H * 2 * I + 2 * T * S * H * 2 * I
    fl["down"] = 2 * rows * I * H + 2 * T * S * I * H
    fl["dense_gate_up"] = 2 * T * H * 2 * Id
    fl["dense_down"] = 2 * T * Id * H
    w_up = int(used * 2 * I * (H * wb + sb + (H // 32 if mx else 0))) + S * 2 * I * H * ab
    w_down = int(used * H * (I * wb + sb + (I // 32 if mx else 0))) + S * H * I * ab
    by = {}
    if path == "decode":
        # router launch: router logits; gate/up launch: routing + expert gate/up; down
        # launch: dense down + expert down + combine; finalize: post-norms.  The dense
        # gate/up rides with the router or the gate/up launch (dense_stage).
        dgu_fl, dgu_by = fl["dense_gate_up"], 2 * Id * H * ab + T * H * ab + T * Id * ab
        fl = {"router": fl["router"], "gate_up": fl["gate_up"], "down": fl["down"] + fl["dense_down"],
              "dense_gate_up": 0, "dense_down": 0}
        by["router"] = z * (E * H * ab + T * E * 4 + T * H * ab)
        by["gate_up"] = w_up + T * H * ab + T * Kp * I * ab
        by["down"] = w_down + T * Kp * I * ab + T * H * (4 if Id else ab) + (H * Id * ab + T * Id * ab + T * H * 4 if Id else 0)
        if spec.act_quant:
            # the gate/up launch also writes x's codes and scales; the h rows are
            # quantised between the launches; the down launch reads 1-byte codes
            by["gate_up"] += T * H + T * 4
            by["quant_h"] = T * Kp * I * ab + T * Kp * I + T * Kp * 4
            by["down"] -= T * Kp * I * (ab - 1)
        if Id:
            fl[dense_stage] += dgu_fl
            by[dense_stage] += dgu_by
        by["dense_gate_up"] = by["dense_down"] = 0
        by["finalize"] = 2 * T * H * 4 + T * H * ab if Id else 0
    else:
        by["router"] = z * (E * H * ab + T * H * ab + T * E * 4)
        by["gate_up"] = w_up + T * H * ab + rows * I * ab
        # down + weighted combine: reads h, writes each token's combined row once (the
        # per-slot rows the library keeps in between are its own design, not counted)
        ob = 4 if Id else ab  # the MoE sum is fp32 when a post-norm follows
        by["down"] = w_down + rows * I * ab + T * H * ob
        if spec.act_quant:
            # the GEMMs read 1-byte codes; the quantisations read bf16 rows and write
            # codes and one fp32 scale per row
            by["gate_up"] -= T * H * (ab - 1)
            by["down"] -= rows * I * (ab - 1)
            by["quant_x"] = T * H * ab + T * H + T * 4
            by["quant_h"] = rows * I * ab + rows * I + rows * 4
        by["dense_gate_up"] = 2 * Id * H * ab + T * H * ab + T * Id * ab
        by["dense_down"] = H * Id * ab + T * Id * ab + T * H * 4
        # combined MoE rows (+ the dense branch's rows) in, the layer output out
        by["finalize"] = T * H * ob + (T * H * 4 if Id else 0) + T * H * ab
    return fl, by


# Which roofline a workload is rated against (the configurations' own split): the
# decode-sized token counts (T <= 128) by the bytes the dominant kernel must move,
# against HBM; the prefill-sized ones by its FLOP, against the MFMA peak of the
# contraction's dtype (FP8 x FP8 for layers with FP8 activations, else bf16); the
# fp32 layer runs on the vector ALUs (fp32 FMA, 157.3 TFLOP/s).
DECODE_MAX_T = 128


def roofline_class(spec, T, dom):
    if spec.wdtype == "fp32":
        return "alu", PEAK_F32_TFLOPS
    if T <= DECODE_MAX_T:
        return "hbm", PEAK_HBM_GBS
    if spec.act_quant and dom in ("gate_up", "down"):
        return "mfma", PEAK_FP8_TFLOPS
    return "mfma", PEAK_BF16_TFLOPS


def launched_stages(spec, path, dense_stage, raw_ms, marker_ms):
    """The library stages that launch work for this layer (the others hold only
    their event record)."""
    supplied, dense = spec.supplied_logits, spec.I_dense > 0
    if path == "decode":
        st = {"gate_up", "down"} | ({"quant_h"} if spec.act_quant else set())
        if not supplied or (dense and dense_stage == "router"):
            st.add("router")
        # finalize: with the dense branch, or when the down kernel splits its
        # reduction (chosen inside the library from the device's CU count)
        if dense or raw_ms["finalize"] > marker_ms + 1e-3:
            st.add("finalize")
        return st
    st = {"route", "permute", "gate_up", "down", "finalize"}
    if spec.act_quant:
        st |= {"quant_x", "quant_h"}
    if (spec.router_mode == "gemma" and not supplied) or dense:
        st.add("prenorm")
    if not supplied:
        st.add("router")
    if dense:
        st |= {"dense_gate_up", "dense_down"}
    return st


def rotated_sets(B, dl, path):
    """Copies of the layer with the experts rolled along the expert axis, enough
    that the weights a decode step reads were not read by the previous step."""
    import torch
    if path != "decode" or dl.desc.num_experts < 2:
        return [dl]
    t = dl.t
    nbytes = sum(v.numel() * v.element_size() for v in t.values() if v is not None)
    n = max(4, math.ceil(2 * MALL_BYTES / max(nbytes, 1)))
    E = dl.desc.num_experts
    sets = [dl]
    for i in range(1, n):
        shift = max(1, (i * E) // n)
        c = {}
        for k, v in t.items():
            if v is None or k in ("x", "logits"):
                c[k] = v
            elif k in ("w13", "w2", "w13_scale", "w2_scale", "per_expert_scale"):
                c[k] = torch.roll(v, shifts=shift, dims=0).contiguous()
            else:
                c[k] = v.clone()
        sets.append(B.DeviceLayer(dl.desc, c))
    return sets


def cpu_baseline(L, seconds):
    """The oracle on a row sample of the workload sized for about `seconds` of CPU
    time: routing over all T rows, the expert FFNs over the sample (repeated when
    even all T rows take less)."""
    import numpy as np
    from mixture_experts_ffn_router_amd import workloads as W
    from oracle import moe_oracle as O
    try:
        import threadpoolctl
        threads = max((d.get("num_threads", 1) for d in threadpoolctl.threadpool_info()), default=1)
    except Exception:
        threads = None
    T = L["T"]
    layer = W.oracle_layer(L)
    x = L["x"].float().numpy().astype(np.float64)
    logits = None if L["logits"] is None else L["logits"].numpy().astype(np.float64)
    rng = np.random.default_rng(0)

    def run(n, reps=1):
        rows = np.sort(rng.choice(T, n, replace=False))
        t0 = time.perf_counter()
        for _ in range(reps):
            O.moe_layer(x, layer, rows=rows, logits=logits)
        return time.perf_counter() - t0

    # Grow the sample (then repeat all T rows) by at most 8x per try until one run
    # takes at least half the target; that run is the measurement.
    n, reps = min(T, 16), 1
    while True:
        dt = run(n, reps)
        if dt >= seconds / 2:
            break
        scale = min(8.0, seconds / max(dt, 1e-3))
        if n < T:
            n = min(T, max(n + 1, int(n * scale)))
        else:
            reps = max(reps + 1, int(reps * scale))
    cores = len(os.sched_getaffinity(0))
    return {"value": round(n * reps / dt, 2), "unit": "tokens/s", "cores": threads or cores, "kind": "oracle",
            "sample": f"{n} of {T} token rows through the experts (routing over all {T}), {reps} time(s): "
                      f"{dt:.1f} s on {cores} host cores, numpy BLAS threads {threads}"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the layer has no multi-GPU path here (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import torch
    from mixture_experts_ffn_router_amd import binding as B
    from mixture_experts_ffn_router_amd import workloads as W

    B.load()
    spec = W.SPECS[args.config]
    T = args.T or spec.T
    spec = spec.with_T(T)
    L = W.make_layer(spec, seed=0)
    dl = B.DeviceLayer.from_generated(L)
    path = dl.path(T)
    sets = rotated_sets(B, dl, path)
    act_dtype = dl.act_dtype
    out = torch.empty(T, spec.H, dtype=act_dtype, device="cuda")
    ws = torch.empty(dl.workspace_size(T), dtype=torch.uint8, device="cuda")
    print(f"[bench] {spec.name} T={T} path={path} weight sets={len(sets)}: warmup {args.warmup}",
          file=sys.stderr, flush=True)
    for i in range(args.warmup):
        sets[i % len(sets)].forward(out=out, workspace=ws)
    torch.cuda.synchronize()

    # timed region: K back-to-back steps
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        sets[i % len(sets)].forward(out=out, workspace=ws)
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
    for i, row in enumerate(evs):
        sets[i % len(sets)].forward(out=out, workspace=ws, events=row)
    p1.record()
    torch.cuda.synchronize()
    prof_ms = p0.elapsed_time(p1) / args.steps
    raw_ms = {name: sum(row[i].elapsed_time(row[i + 1]) for row in evs) / args.steps
              for i, name in enumerate(B.STAGES)}
    # Each event record costs stream time of its own (two back-to-back records on
    # the stream, reported as event_marker_ms).  Stage intervals are kept as
    # measured in stages_ms; the dominant kernel's duration is its interval less
    # one record.
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a_, b_ in pairs:
        a_.record()
        b_.record()
    torch.cuda.synchronize()
    marker_ms = sorted(a_.elapsed_time(b_) for a_, b_ in pairs)[len(pairs) // 2]
    launched = launched_stages(spec, path, dl.dense_gate_up_stage(T), raw_ms, marker_ms)
    stage_ms = {k: (v if k in launched else 0.0) for k, v in raw_ms.items()}  # empty stages: 0

    fl, by = stage_work(spec, T, counts, path, dl.dense_gate_up_stage(T))
    total_flop = sum(fl.values())
    total_bytes = sum(by.values())
    cand = [s for s in ("gate_up", "down", "dense_gate_up", "dense_down", "router") if fl[s] > 0]
    dom = max(cand, key=lambda s: stage_ms[s])
    # the stage interval holds the kernel and one event record (marker_ms, measured
    # in this run): the kernel's duration is the interval less that record
    kernel_ms = max(stage_ms[dom] - marker_ms, 1e-6)
    dom_s = kernel_ms / 1e3
    bound, peak = roofline_class(spec, T, dom)
    if bound != "hbm":
        achieved = fl[dom] / dom_s / 1e12
        roof = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": None}
    else:
        achieved = by[dom] / dom_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": peak, "unit": "GB/s",
                "frac": round(achieved / peak, 4), "traffic": None}
    wl = f"{spec.name}_T{T}"
    traffic = stored_traffic(wl, dom, path)
    roof["traffic"] = traffic
    roof.update({"kernel": dom, "kernel_ms": round(kernel_ms, 5), "stage_interval_ms": round(stage_ms[dom], 5),
                 "algorithmic_per_launch": fl[dom] if roof["bound"] != "hbm" else by[dom],
                 "algorithmic_bytes_per_launch": by[dom],
                 "traffic_over_algorithmic": round(traffic / by[dom], 3) if traffic else None,
                 "event_marker_ms": round(marker_ms, 5), "kernel_source_digest": source_digest(path)})

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
        "dtype": ("fp8-e4m3 weights and activations (per-row dynamic activation scales)" if spec.act_quant else
                  {"fp32": "f32", "bf16": "bf16", "fp8": "fp8-e4m3 weights, bf16 activations",
                   "mxfp4": "mxfp4 (e2m1 + e8m0 per 32) weights, bf16 activations"}[spec.wdtype]),
        "data": "synthetic",
        "config": {"workload": f"{spec.name} MoE FFN layer forward", "T": T, "hidden": spec.H,
                   "experts": spec.E, "top_k": spec.K, "inter": spec.I, "act": spec.act,
                   "shared": spec.n_shared, "dense_inter": spec.I_dense, "scoring": spec.scoring,
                   "groups": [spec.n_groups, spec.topk_groups] if spec.n_groups > 1 else None,
                   "act_quant": spec.act_quant, "path": path,
                   "weight_sets": len(sets)},
        "step_tflops": round(total_flop / (ms_per_step / 1e3) / 1e12, 2),
        "step_gbps": round(total_bytes / (ms_per_step / 1e3) / 1e9, 1),
        "experts_touched": int((counts > 0).sum()),
        "stages_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "profiled_ms_per_step": round(prof_ms, 5),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        print(f"[bench] cpu oracle, about {args.cpu_seconds:.0f} s", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(L, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
