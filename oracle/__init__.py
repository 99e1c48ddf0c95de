"""fp64 CPU oracle for the Mixtral sparse-MoE feed-forward layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product library
never loads it and shares no code with it.

The arithmetic lives in ``moe_oracle.c`` (plain fp64 loops); this module only
marshals numpy arrays through ctypes.  Each function names the passage of the
pages about "Mixtral of Experts" that it follows; see ``moe_oracle.h``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1


def default_threads() -> int:
    """Threads the oracle uses: every core this process may run on."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build

            _build.build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, dbl = ctypes.c_int, ctypes.c_long, ctypes.c_double
        L.orc_bf16_round.restype = dbl
        L.orc_bf16_round.argtypes = [dbl]
        L.orc_router_logits.argtypes = [P, i32, P, i64, i32, i32, P, i32]
        L.orc_topk_gates.argtypes = [P, i64, i32, i32, P, P, P, P]
        L.orc_permute.argtypes = [P, i64, i32, i32, P, P, P, P]
        L.orc_balance.argtypes = [P, P, i64, i32, i32, P, P, P]
        L.orc_swiglu_expert.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, P]
        L.orc_moe_rows.argtypes = [P, i32, P, P, P, P, i32, i32, i32, i32, i32, i32, P, i64,
                                   P, P, P, P, P, i32]
        L.orc_rmsnorm.argtypes = [P, i32, dbl, P]
        L.orc_rmsnorm_rows.argtypes = [P, i64, i32, dbl, i32, P]
        L.orc_rmsnorm_rows.restype = ctypes.c_int
        L.orc_block_step.argtypes = [P, i64, P, P, P, P, i32, i32, i32, i32, dbl, i32, P, P, P,
                                     P, i32]
        for name in ("orc_router_logits", "orc_topk_gates", "orc_permute", "orc_swiglu_expert",
                     "orc_moe_rows", "orc_rmsnorm", "orc_block_step"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _raw(a):
    """(array, dtype code) for fp32 or bf16 data.

    bf16 arrives as uint16 bit patterns (numpy has no bf16 type) or as a torch
    bfloat16 tensor, which is viewed as int16 without conversion.
    """
    if hasattr(a, "dtype") and str(a.dtype) == "torch.bfloat16":
        import torch

        a = a.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    elif hasattr(a, "detach"):
        a = a.detach().cpu().contiguous().numpy()
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    raise TypeError(f"oracle takes fp32 or bf16 data, got {a.dtype}")


def _f32(a):
    if hasattr(a, "detach"):
        a = a.detach().cpu().float().numpy()
    return np.ascontiguousarray(a, dtype=np.float32)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments")


def bf16_round(v: float) -> float:
    """Nearest bf16 value (ties to even) of a double."""
    return float(lib().orc_bf16_round(float(v)))


def router_logits(x, Wg, nthreads=None):
    """fp64 scores l[t][e] = x_t . Wg_e  (x: [T][d] fp32/bf16, Wg: [E][d] fp32)."""
    xa, dt = _raw(x)
    wg = _f32(Wg)
    T, d = xa.shape
    E = wg.shape[0]
    assert wg.shape[1] == d
    out = np.empty((T, E), np.float64)
    _check(lib().orc_router_logits(_ptr(xa), dt, _ptr(wg), T, d, E, _ptr(out),
                                   nthreads or default_threads()), "router_logits")
    return out


def topk_gates(logits, k):
    """(idx int32[T][k], gates f64[T][k], gap_order f64[T], gap_set f64[T])."""
    lg = np.ascontiguousarray(logits, np.float64)
    T, E = lg.shape
    idx = np.empty((T, k), np.int32)
    gates = np.empty((T, k), np.float64)
    go = np.empty(T, np.float64)
    gs = np.empty(T, np.float64)
    _check(lib().orc_topk_gates(_ptr(lg), T, E, k, _ptr(idx), _ptr(gates), _ptr(go), _ptr(gs)),
           "topk_gates")
    return idx, gates, go, gs


def route(x, Wg, k, nthreads=None):
    """Router scores, top-k choice and gates for every row of x."""
    lg = router_logits(x, Wg, nthreads)
    idx, gates, go, gs = topk_gates(lg, k)
    return dict(logits=lg, idx=idx, gates=gates, gap_order=go, gap_set=gs)


def balance(logits, idx):
    """Router load statistics: f[e] (share of the T*k assignments), P[e]
    (mean full-softmax probability) and laux = E * sum f * P."""
    lg = np.ascontiguousarray(logits, np.float64)
    ia = np.ascontiguousarray(idx, np.int32)
    T, E = lg.shape
    k = ia.shape[1]
    f = np.empty(E, np.float64)
    P = np.empty(E, np.float64)
    laux = np.empty(1, np.float64)
    _check(lib().orc_balance(_ptr(lg), _ptr(ia), T, E, k, _ptr(f), _ptr(P), _ptr(laux)),
           "balance")
    return dict(f=f, P=P, laux=float(laux[0]))


def permute(idx, E):
    """Stable grouping of the T*k assignments by expert."""
    ia = np.ascontiguousarray(idx, np.int32)
    T, k = ia.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    row_of = np.empty((T, k), np.int32)
    token_of = np.empty(T * k, np.int32)
    _check(lib().orc_permute(_ptr(ia), T, E, k, _ptr(counts), _ptr(offsets), _ptr(row_of),
                             _ptr(token_of)), "permute")
    return dict(counts=counts, offsets=offsets, row_of=row_of, token_of=token_of)


def swiglu_expert(xrow, W1, W3, W2, e, round_mid=False):
    """One expert on one fp64 row: W2_e (silu(W1_e x) * W3_e x); round_mid
    rounds the intermediate to bf16 before W2."""
    w1, dt = _raw(W1)
    w3, dt3 = _raw(W3)
    w2, dt2 = _raw(W2)
    assert dt == dt3 == dt2
    E, d_ff, d = w1.shape
    xr = np.ascontiguousarray(xrow, np.float64)
    assert xr.shape == (d,)
    out = np.empty(d, np.float64)
    _check(lib().orc_swiglu_expert(_ptr(xr), _ptr(w1), _ptr(w3), _ptr(w2), dt, int(e), d, d_ff,
                                   int(bool(round_mid)), _ptr(out)), "swiglu_expert")
    return out


def moe_rows(x, Wg, W1, W3, W2, k, rows=None, nthreads=None, round_mid=False):
    """The whole layer for the listed rows of x (default: all rows).  round_mid
    rounds each expert's SwiGLU intermediate to bf16 before W2.

    Returns dict y f64[n][d], idx, gates, gap_order, gap_set.
    """
    xa, xdt = _raw(x)
    wg = _f32(Wg)
    w1, wdt = _raw(W1)
    w3, _ = _raw(W3)
    w2, _ = _raw(W2)
    T, d = xa.shape
    E, d_ff, d1 = w1.shape
    assert d1 == d and w2.shape == (E, d, d_ff) and wg.shape == (E, d)
    if rows is None:
        rows = np.arange(T, dtype=np.int64)
    rows = np.ascontiguousarray(rows, np.int64)
    n = rows.shape[0]
    y = np.empty((n, d), np.float64)
    idx = np.empty((n, k), np.int32)
    gates = np.empty((n, k), np.float64)
    go = np.empty(n, np.float64)
    gs = np.empty(n, np.float64)
    _check(lib().orc_moe_rows(_ptr(xa), xdt, _ptr(wg), _ptr(w1), _ptr(w3), _ptr(w2), wdt, d,
                              d_ff, E, k, int(bool(round_mid)), _ptr(rows), n, _ptr(y), _ptr(idx),
                              _ptr(gates),
                              _ptr(go), _ptr(gs), nthreads or default_threads()), "moe_rows")
    return dict(y=y, idx=idx, gates=gates, gap_order=go, gap_set=gs)


def rmsnorm(h, eps):
    ha = np.ascontiguousarray(h, np.float64)
    out = np.empty_like(ha)
    _check(lib().orc_rmsnorm(_ptr(ha), ha.shape[0], float(eps), _ptr(out)), "rmsnorm")
    return out


def rmsnorm_rows(h, eps, round_bf16=True):
    """rmsnorm of every row of h (f64[n][d]), optionally rounded to bf16."""
    ha = np.ascontiguousarray(h, np.float64)
    n, d = ha.shape
    out = np.empty_like(ha)
    _check(lib().orc_rmsnorm_rows(_ptr(ha), n, d, float(eps), int(bool(round_bf16)), _ptr(out)),
           "rmsnorm_rows")
    return out


def block_step(h, Wg, W1, W3, W2, k, eps, round_mid=False, nthreads=None):
    """One block h <- bf16(h + moe(bf16(rmsnorm(h)))) on n independent rows.

    round_mid rounds each expert's SwiGLU intermediate to bf16 (the one
    quantisation point a bf16 matrix-core data path adds inside the layer).

    h: f64[n][d] holding bf16 values; updated in place.  Weights bf16.
    Returns the step's routing dict (idx, gates, gap_order, gap_set).
    """
    assert h.dtype == np.float64 and h.flags.c_contiguous
    wg = _f32(Wg)
    w1, wdt = _raw(W1)
    w3, _ = _raw(W3)
    w2, _ = _raw(W2)
    assert wdt == BF16
    n, d = h.shape
    E, d_ff, _ = w1.shape
    idx = np.empty((n, k), np.int32)
    gates = np.empty((n, k), np.float64)
    go = np.empty(n, np.float64)
    gs = np.empty(n, np.float64)
    _check(lib().orc_block_step(_ptr(h), n, _ptr(wg), _ptr(w1), _ptr(w3), _ptr(w2), d, d_ff, E,
                                k, float(eps), int(bool(round_mid)), _ptr(idx), _ptr(gates),
                                _ptr(go), _ptr(gs),
                                nthreads or default_threads()), "block_step")
    return dict(idx=idx, gates=gates, gap_order=go, gap_set=gs)


def layer_flops(T, d, d_ff, E, k):
    """Algorithmic FLOPs of one layer: router 2*T*d*E plus 2*k*3*d*d_ff per token
    (two multiply-adds per weight of each of the k experts a token visits)."""
    return T * (2 * k * 3 * d * d_ff + 2 * d * E)


def expert_params(d, d_ff):
    """Weights of one SwiGLU expert: w1 and w3 are d_ff x d, w2 is d x d_ff."""
    return 3 * d * d_ff
