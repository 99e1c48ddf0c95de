"""Comparison helpers shared by the GPU parity tests (HIP path vs the oracle)."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import oracle

# Normwise relative error bounds on y: fp32 and bf16 layers.
TOL = {"f32": 1e-5, "bf16": 2e-2}
# A token whose 2nd/3rd score gap (k-th / (k+1)-th) is below this is exempt
# from the exact routing-set check; one whose kept scores are this close is
# exempt from the order check only.  Both are counted and reported.
NEAR_TIE = 1e-6


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def normwise(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    return float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))


# Near-tie report: one entry per routing comparison made in this session
# (the test, tokens compared, tokens whose oracle set / order gap is below
# NEAR_TIE, and how many of those the GPU routed differently).  conftest.py
# prints it at the end of the run, so it survives -q.
NEAR_TIE_LOG = []


def _current_test():
    return os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]


def check_routing(gpu_idx, gpu_w, orc, near_tie=NEAR_TIE, gate_tol=2e-6, label=None):
    """Exact per-token routing agreement, with the near-tie exemptions.

    Returns (identical_mask, n_set_exempt, n_order_exempt)."""
    gi = np.asarray(gpu_idx)
    oi = orc["idx"]
    same = np.all(gi == oi, axis=1)
    n_set = n_order = 0
    for t in np.nonzero(~same)[0]:
        if set(gi[t].tolist()) != set(oi[t].tolist()):
            assert orc["gap_set"][t] < near_tie, (
                f"token {t}: gpu {gi[t]} vs oracle {oi[t]}, set gap {orc['gap_set'][t]:.3e}")
            n_set += 1
        else:
            assert orc["gap_order"][t] < near_tie, (
                f"token {t}: order {gi[t]} vs {oi[t]}, gap {orc['gap_order'][t]:.3e}")
            n_order += 1
    gw = np.asarray(gpu_w, np.float64)
    if same.any():
        err = np.abs(gw[same] - orc["gates"][same]).max()
        assert err <= gate_tol, f"gate error {err:.3e}"
    near_set = int((orc["gap_set"] < near_tie).sum())
    near_order = int((orc["gap_order"] < near_tie).sum())
    NEAR_TIE_LOG.append(dict(test=_current_test() + (f" [{label}]" if label else ""),
                             tokens=int(gi.shape[0]), near_set=near_set,
                             near_order=near_order, exempt_set=n_set, exempt_order=n_order))
    if n_set or n_order or near_set or near_order:
        log(f"  near ties: {near_set} tokens with set gap < {near_tie:g} ({n_set} routed "
            f"differently), {near_order} with order gap < {near_tie:g} ({n_order} differently)")
    return same, n_set, n_order


def to_np(t: torch.Tensor):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy()


def bf16_rne(a):
    """Nearest bf16 values (ties to even) of float64 data, as float64."""
    a = np.asarray(a, np.float64)
    m, e = np.frexp(a)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def bf16_step(a):
    """Spacing of bf16 values at magnitude |a| (normal range)."""
    _, e = np.frexp(np.asarray(a, np.float64))
    return np.ldexp(1.0, e - 8)


def check_near_rounding_floor(got, want_exact, slack=1.25):
    """got (bf16 values) against the exact result: the normwise error may
    exceed that of rounding the exact result to bf16 once only by `slack`.
    Returns (error, floor)."""
    got = np.asarray(got, np.float64)
    floor = normwise(bf16_rne(want_exact), want_exact)
    err = normwise(got, want_exact)
    assert err <= slack * floor, (err, floor)
    return err, floor
