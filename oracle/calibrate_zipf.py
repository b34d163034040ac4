"""Calibrate the Zipf bias amplitude of the skewed-routing workload.

The workload asks for logits N(0,1) + a Zipf(s=1.2) per-expert bias such that
about 10% of the experts receive about 60% of the top-8 assignments.  Taken
literally (b_e = -1.2 ln rank_e) the 13 busiest of 128 experts take about 81%,
so the bias is scaled by alpha, found here by bisection on the oracle's own
top-k selection (T = 4096, seed 0), targeting a 0.60 share.

Run:  python -m oracle.calibrate_zipf      (prints alpha and the share)
"""
import numpy as np

from oracle.moe_oracle import select_topk


def top_share(logits, k, n_top):
    ids = select_topk(logits, k)
    counts = np.bincount(ids.ravel(), minlength=logits.shape[1])
    return np.sort(counts)[::-1][:n_top].sum() / ids.size


def calibrate(T=4096, E=128, k=8, seed=0, target=0.60, iters=12):
    from mixture_experts_ffn_router_amd.workloads import _normal, _TID, zipf_bias
    noise = _normal(seed, _TID["logit_noise"], (T, E), 1.0).astype(np.float64)
    n_top = int(round(0.1 * E))
    lo, hi = 0.0, 1.0
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        share = top_share(noise + zipf_bias(E, seed, alpha=mid)[None, :].astype(np.float64), k, n_top)
        if share < target:
            lo = mid
        else:
            hi = mid
    alpha = 0.5 * (lo + hi)
    return alpha, top_share(noise + zipf_bias(E, seed, alpha=alpha)[None, :].astype(np.float64), k, n_top)


if __name__ == "__main__":
    a, s = calibrate()
    print(f"alpha={a!r} share={s:.4f}")
