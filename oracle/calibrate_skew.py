"""Fit the Zipf-bias scale beta of the skewed workload (test infrastructure).

Bisection on beta so that experts 0 and 1 receive half of all top-2
assignments of the skewed workload's CPU draw (T = 16384, seed 0), with the
routing computed by the fp64 oracle.  Prints the beta to store as
SKEW_BETA in sparse_mixture_experts_31_amd/inputs.py.

    python -m oracle.calibrate_skew
"""
from __future__ import annotations

import numpy as np

import oracle
from sparse_mixture_experts_31_amd.inputs import WORKLOADS, make_layer


def share01(beta: float, seed: int = 0) -> float:
    w = WORKLOADS["skewed"].with_(beta=beta)
    L = make_layer(w, "cpu", seed)
    idx = oracle.route(L["x"], L["Wg"], w.k)["idx"]
    c = np.bincount(idx.reshape(-1), minlength=w.E)
    return float(c[:2].sum() / c.sum())


def main(target: float = 0.5, iters: int = 14) -> float:
    lo, hi = 0.0, 1.5
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        s = share01(mid)
        print(f"beta={mid:.5f} share01={s:.4f}", flush=True)
        if s < target:
            lo = mid
        else:
            hi = mid
    beta = round(0.5 * (lo + hi), 3)
    print(f"SKEW_BETA = {beta}  (share {share01(beta):.4f})")
    return beta


if __name__ == "__main__":
    main()
