"""Thin Python binding over libmoe.so (C ABI declared in include/moe.h).

Every function has the name of the C entry point it wraps and does argument
marshalling only: it takes torch tensors on the GPU, allocates missing
outputs with torch, and passes raw device pointers plus the current HIP
stream to the library.  All arithmetic runs in the library's HIP kernels; if
libmoe.so is not built, every call raises instead of falling back to anything.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1

_lib = None


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}: {detail}")


def lib():
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m sparse_mixture_experts_31_amd.build` "
                "(or __graft_entry__.build()) first")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                                ctypes.c_size_t)
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [i32]
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_workspace_size.restype = sz
        L.moe_workspace_size.argtypes = [i64, i32, i32, i32, i32, i32]
        L.moe_forward_noalloc_max_scratch.restype = sz
        L.moe_forward_noalloc_max_scratch.argtypes = []
        L.moe_expert_ffn_kernels.restype = ctypes.c_char_p
        L.moe_expert_ffn_kernels.argtypes = [i64, i32, i32, i32, i32, i32]
        L.moe_forward_kernels.restype = ctypes.c_char_p
        L.moe_forward_kernels.argtypes = [i64, i32, i32, i32, i32, i32]
        L.moe_route_balance_workspace_size.restype = sz
        L.moe_route_balance_workspace_size.argtypes = [i64, i32]
        L.moe_permute_workspace_size.restype = sz
        L.moe_permute_workspace_size.argtypes = [i64, i32, i32]
        sigs = {
            "moe_route": [P, P, i32, i64, i32, i32, i32, P, P, P, P],
            "moe_route_balance": [P, P, i32, i64, i32, i32, i32, P, P, P, P, P, P, sz, P],
            "moe_permute": [P, P, i32, i64, i32, i32, i32, P, P, P, P, P, P, sz, P],
            "moe_expert_ffn": [P, P, P, P, P, i32, i64, i32, i32, i32, i32, P, P, sz, P],
            "moe_combine": [P, P, P, P, i32, i64, i32, i32, P, P],
            "moe_forward": [P, P, P, P, P, i32, i64, i32, i32, i32, i32, P, P, sz, P],
            "moe_forward_profiled": [P, P, P, P, P, i32, i64, i32, i32, i32, i32, P, P, sz, P, P],
            "moe_forward_noalloc": [P, P, P, P, P, i32, i64, i32, i32, i32, i32, P, P],
            "moe_rmsnorm": [P, i32, i64, i32, f32, P, P],
            "moe_block_forward": [P, P, P, P, P, i32, i64, i32, i32, i32, i32, f32, P, P, P, sz,
                                  P],
        }
        for name, args in sigs.items():
            fn = getattr(L, name)
            fn.restype = i32
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().moe_status_string(int(s)).decode()


def _call(name, *args):
    rc = getattr(lib(), name)(*args)
    if rc != MOE_OK:
        raise MoeError(rc, name, lib().moe_last_error().decode())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"activations and expert weights must be fp32 or bf16, got {t.dtype}")


def _check_router(x, Wg):
    """Raise before the call if Wg is not the fp32 [E][d] gate matrix of x [T][d]
    (the library reads E*d fp32 values from it)."""
    if x.dim() != 2:
        raise ValueError(f"x must be [T][d], got shape {tuple(x.shape)}")
    if Wg.dtype != torch.float32:
        raise TypeError(f"Wg must be fp32, got {Wg.dtype}")
    if Wg.dim() != 2 or Wg.shape[1] != x.shape[1]:
        raise ValueError(f"Wg must be [E][d] with d = {x.shape[1]}, got {tuple(Wg.shape)}")


def _check_experts(act, W1, W3, W2):
    """Raise before the call unless W1, W3 are [E][d_ff][d] and W2 is
    [E][d][d_ff] in the activations' dtype (d = act's row length)."""
    d = act.shape[-1]
    for name, W in (("W1", W1), ("W3", W3), ("W2", W2)):
        if W.dtype != act.dtype:
            raise TypeError(f"{name} must have the activations' dtype {act.dtype}, got {W.dtype}")
        if W.dim() != 3:
            raise ValueError(f"{name} must be 3-dimensional, got shape {tuple(W.shape)}")
    E, d_ff, d1 = W1.shape
    if d1 != d or tuple(W3.shape) != (E, d_ff, d) or tuple(W2.shape) != (E, d, d_ff):
        raise ValueError(f"expert shapes W1 {tuple(W1.shape)}, W3 {tuple(W3.shape)}, W2 "
                         f"{tuple(W2.shape)} do not fit d = {d}")


def _check_out(name, t, shape, dtype):
    if t is not None and (tuple(t.shape) != tuple(shape) or t.dtype != dtype):
        raise ValueError(f"{name} must be {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")


def _p(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to libmoe must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _s(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def moe_workspace_size(T, d, d_ff, E, k, dtype) -> int:
    dt = MOE_F32 if dtype in (torch.float32, MOE_F32) else MOE_BF16
    return int(lib().moe_workspace_size(T, d, d_ff, E, k, dt))


def moe_expert_ffn_kernels(T, d, d_ff, E, k, dtype) -> str:
    """Kernel family the library picks for the expert GEMMs of this shape."""
    dt = MOE_F32 if dtype in (torch.float32, MOE_F32) else MOE_BF16
    return lib().moe_expert_ffn_kernels(T, d, d_ff, E, k, dt).decode()


def moe_forward_kernels(T, d, d_ff, E, k, dtype) -> str:
    """Kernel family of the fused layer's expert GEMMs at T tokens."""
    dt = MOE_F32 if dtype in (torch.float32, MOE_F32) else MOE_BF16
    return lib().moe_forward_kernels(T, d, d_ff, E, k, dt).decode()


def workspace(T, d, d_ff, E, k, dtype, device="cuda") -> torch.Tensor:
    n = moe_workspace_size(T, d, d_ff, E, k, dtype)
    if n == 0:
        raise ValueError("shape rejected by libmoe")
    return torch.empty(n, dtype=torch.uint8, device=device)


def moe_route(x, Wg, k, topk_idx=None, topk_w=None, logits=None, stream=None):
    _check_router(x, Wg)
    T, d = x.shape
    E = Wg.shape[0]
    _check_out("topk_idx", topk_idx, (T, k), torch.int32)
    _check_out("topk_w", topk_w, (T, k), torch.float32)
    _check_out("logits", logits, (T, E), torch.float32)
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    _call("moe_route", _p(x), _p(Wg), _dt(x), T, d, E, k, _p(topk_idx), _p(topk_w), _p(logits),
          _s(stream))
    return topk_idx, topk_w


def moe_permute_workspace_size(T, E, k) -> int:
    return int(lib().moe_permute_workspace_size(T, E, k))


def moe_route_balance_workspace_size(T, E) -> int:
    return int(lib().moe_route_balance_workspace_size(T, E))


def moe_route_balance(x, Wg, k, topk_idx=None, topk_w=None, ws=None, stream=None):
    """moe_route plus the load statistics: returns (topk_idx, topk_w, f, P,
    laux) with f, P fp32 [E] and laux an fp32 tensor of one element."""
    _check_router(x, Wg)
    T, d = x.shape
    E = Wg.shape[0]
    _check_out("topk_idx", topk_idx, (T, k), torch.int32)
    _check_out("topk_w", topk_w, (T, k), torch.float32)
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    f = torch.empty(E, dtype=torch.float32, device=x.device)
    P = torch.empty(E, dtype=torch.float32, device=x.device)
    laux = torch.empty(1, dtype=torch.float32, device=x.device)
    if ws is None:
        n = moe_route_balance_workspace_size(T, E)
        if n == 0:
            raise ValueError("shape rejected by libmoe")
        ws = torch.empty(n, dtype=torch.uint8, device=x.device)
    _call("moe_route_balance", _p(x), _p(Wg), _dt(x), T, d, E, k, _p(topk_idx), _p(topk_w),
          _p(f), _p(P), _p(laux), _p(ws), ws.numel(), _s(stream))
    return topk_idx, topk_w, f, P, laux


def moe_permute(x, topk_idx, E, counts=None, offsets=None, row_of=None, token_of=None,
                x_perm=None, stream=None):
    T, d = x.shape
    k = topk_idx.shape[1]
    dev = x.device
    _check_out("topk_idx", topk_idx, (T, k), torch.int32)
    _check_out("counts", counts, (E,), torch.int32)
    _check_out("offsets", offsets, (E + 1,), torch.int32)
    _check_out("row_of", row_of, (T, k), torch.int32)
    _check_out("token_of", token_of, (T * k,), torch.int32)
    _check_out("x_perm", x_perm, (T * k, d), x.dtype)
    counts = torch.empty(E, dtype=torch.int32, device=dev) if counts is None else counts
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    row_of = torch.empty((T, k), dtype=torch.int32, device=dev) if row_of is None else row_of
    token_of = torch.empty(T * k, dtype=torch.int32, device=dev) if token_of is None else token_of
    x_perm = torch.empty((T * k, d), dtype=x.dtype, device=dev) if x_perm is None else x_perm
    n = moe_permute_workspace_size(T, E, k)
    ws = torch.empty(n, dtype=torch.uint8, device=dev) if n else None
    _call("moe_permute", _p(x), _p(topk_idx), _dt(x), T, d, E, k, _p(counts), _p(offsets),
          _p(row_of), _p(token_of), _p(x_perm), _p(ws), n, _s(stream))
    return dict(counts=counts, offsets=offsets, row_of=row_of, token_of=token_of, x_perm=x_perm)


def moe_expert_ffn(x_perm, offsets, W1, W3, W2, T, k, out_perm=None, ws=None, stream=None):
    _check_experts(x_perm, W1, W3, W2)
    E, d_ff, d = W1.shape
    _check_out("x_perm", x_perm, (T * k, d), x_perm.dtype)
    _check_out("offsets", offsets, (E + 1,), torch.int32)
    _check_out("out_perm", out_perm, (T * k, d), x_perm.dtype)
    if out_perm is None:
        out_perm = torch.empty((T * k, d), dtype=x_perm.dtype, device=x_perm.device)
    if ws is None:
        ws = workspace(T, d, d_ff, E, k, x_perm.dtype, x_perm.device)
    _call("moe_expert_ffn", _p(x_perm), _p(offsets), _p(W1), _p(W3), _p(W2), _dt(x_perm), T, d,
          d_ff, E, k, _p(out_perm), _p(ws), ws.numel(), _s(stream))
    return out_perm


def moe_combine(out_perm, row_of, topk_w, residual=None, y=None, stream=None):
    T, k = row_of.shape
    d = out_perm.shape[1]
    _check_out("row_of", row_of, (T, k), torch.int32)
    _check_out("topk_w", topk_w, (T, k), torch.float32)
    _check_out("residual", residual, (T, d), out_perm.dtype)
    _check_out("y", y, (T, d), out_perm.dtype)
    if y is None:
        y = torch.empty((T, d), dtype=out_perm.dtype, device=out_perm.device)
    _call("moe_combine", _p(out_perm), _p(row_of), _p(topk_w), _p(residual), _dt(out_perm), T,
          d, k, _p(y), _s(stream))
    return y


def moe_forward(x, Wg, W1, W3, W2, k, y=None, ws=None, stream=None):
    _check_router(x, Wg)
    _check_experts(x, W1, W3, W2)
    T, d = x.shape
    E, d_ff, _ = W1.shape
    if Wg.shape[0] != E:
        raise ValueError(f"Wg has {Wg.shape[0]} experts, W1 {E}")
    _check_out("y", y, (T, d), x.dtype)
    if y is None:
        y = torch.empty_like(x)
    if ws is None:
        ws = workspace(T, d, d_ff, E, k, x.dtype, x.device)
    _call("moe_forward", _p(x), _p(Wg), _p(W1), _p(W3), _p(W2), _dt(x), T, d, d_ff, E, k, _p(y),
          _p(ws), ws.numel(), _s(stream))
    return y


def moe_forward_noalloc(x, Wg, W1, W3, W2, k, y=None, stream=None):
    """The layer on the library's static scratch array: no workspace argument.
    (The C call allocates nothing; pass y to avoid torch allocating it.)"""
    _check_router(x, Wg)
    _check_experts(x, W1, W3, W2)
    T, d = x.shape
    E, d_ff, _ = W1.shape
    if Wg.shape[0] != E:
        raise ValueError(f"Wg has {Wg.shape[0]} experts, W1 {E}")
    _check_out("y", y, (T, d), x.dtype)
    if y is None:
        y = torch.empty_like(x)
    _call("moe_forward_noalloc", _p(x), _p(Wg), _p(W1), _p(W3), _p(W2), _dt(x), T, d, d_ff, E,
          k, _p(y), _s(stream))
    return y


def moe_forward_profiled(x, Wg, W1, W3, W2, k, events, y=None, ws=None, stream=None):
    """moe_forward that records 6 caller-owned hipEvent_t handles (ints or
    None) around its stages: router, dispatch, GEMM1, GEMM2, combine."""
    _check_router(x, Wg)
    _check_experts(x, W1, W3, W2)
    T, d = x.shape
    E, d_ff, _ = W1.shape
    if Wg.shape[0] != E:
        raise ValueError(f"Wg has {Wg.shape[0]} experts, W1 {E}")
    _check_out("y", y, (T, d), x.dtype)
    if y is None:
        y = torch.empty_like(x)
    if ws is None:
        ws = workspace(T, d, d_ff, E, k, x.dtype, x.device)
    arr = (ctypes.c_void_p * 6)(*[ctypes.c_void_p(e) if e else None for e in events])
    _call("moe_forward_profiled", _p(x), _p(Wg), _p(W1), _p(W3), _p(W2), _dt(x), T, d, d_ff, E,
          k, _p(y), _p(ws), ws.numel(), arr, _s(stream))
    return y


def moe_rmsnorm(h, eps, out=None, stream=None):
    T, d = h.shape
    _check_out("out", out, (T, d), h.dtype)
    if out is None:
        out = torch.empty_like(h)
    _call("moe_rmsnorm", _p(h), _dt(h), T, d, float(eps), _p(out), _s(stream))
    return out


def moe_block_forward(h, Wg, W1, W3, W2, k, eps, topk_idx=None, topk_w=None, ws=None,
                      stream=None):
    """In place: h <- h + moe(rms_norm(h)).  Returns h."""
    _check_router(h, Wg)
    _check_experts(h, W1, W3, W2)
    T, d = h.shape
    E, d_ff, _ = W1.shape
    if Wg.shape[0] != E:
        raise ValueError(f"Wg has {Wg.shape[0]} experts, W1 {E}")
    _check_out("topk_idx", topk_idx, (T, k), torch.int32)
    _check_out("topk_w", topk_w, (T, k), torch.float32)
    if ws is None:
        ws = workspace(T, d, d_ff, E, k, h.dtype, h.device)
    _call("moe_block_forward", _p(h), _p(Wg), _p(W1), _p(W3), _p(W2), _dt(h), T, d, d_ff, E, k,
          float(eps), _p(topk_idx), _p(topk_w), _p(ws), ws.numel(), _s(stream))
    return h
