"""C ABI checks that need no GPU: the library loads, exports every entry point
include/moe.h declares, and rejects bad arguments with status codes before
anything is launched."""
import ctypes
import os
import re

import pytest

from sparse_mixture_experts_31_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

FAKE = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: checks fail first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_forward",
                 "moe_workspace_size", "moe_rmsnorm", "moe_block_forward",
                 "moe_status_string", "moe_last_error"):
        assert want in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(moe.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings():
    assert moe.status_string(moe.MOE_OK) == "MOE_OK"
    assert moe.status_string(moe.MOE_ERR_WORKSPACE) == "MOE_ERR_WORKSPACE"
    assert moe.status_string(99) == "MOE_ERR_UNKNOWN"


def test_workspace_size_rules():
    ws = moe.moe_workspace_size
    base = ws(4096, 4096, 14336, 8, 2, moe.MOE_BF16)
    assert base > 0
    # the SwiGLU intermediate dominates: T*k rows of d_ff
    assert base >= 4096 * 2 * 14336 * 2
    assert ws(4097, 4096, 14336, 8, 2, moe.MOE_BF16) > base
    assert ws(4096, 4096, 14336, 8, 2, moe.MOE_F32) > base
    assert ws(0, 4096, 14336, 8, 2, moe.MOE_BF16) > 0       # T = 0 is legal
    for bad in [(-1, 64, 64, 8, 2), (8, 100, 64, 8, 2), (8, 64, 96, 8, 2), (8, 64, 64, 65, 2),
                (8, 64, 64, 8, 9), (8, 64, 64, 4, 5), (8, 64, 64, 8, 0), (1 << 30, 64, 64, 8, 2)]:
        assert ws(*bad, moe.MOE_BF16) == 0, bad


def test_permute_workspace_size_rules():
    """One workgroup groups up to 4096 assignments (no workspace); above that
    the chunk counts need E ints per chunk, at most 512 chunks; the layer's
    workspace always holds them."""
    pw = moe.moe_permute_workspace_size
    assert pw(2048, 8, 2) == 0 and pw(4096, 8, 1) == 0 and pw(0, 8, 2) == 0
    assert pw(2049, 8, 2) == 4 * 17 * 8               # 4098 assignments, 17 chunks of 256
    assert pw(16384, 8, 2) == 4 * 128 * 8
    assert pw(1 << 20, 8, 2) <= 4 * 512 * 8           # chunks grow instead of their count
    for bad in [(-1, 8, 2), (8, 65, 2), (8, 8, 9), (8, 4, 5), (8, 8, 0), (1 << 30, 8, 2)]:
        assert pw(*bad) == 0, bad
    for T in (1, 100, 2049, 4096, 16384):
        assert moe.moe_workspace_size(T, 4096, 14336, 8, 2, moe.MOE_BF16) >= pw(T, 8, 2)


def test_kernel_family_labels_follow_rows_per_expert():
    """The expert kernels are chosen by rows per expert (T k / E) on the host:
    the weight stream below 27, grouped GEMM1 with wide GEMM2 below 49, the
    wide kernels above (128-row token tiles up to 100, then 256), bf16 only
    for the stream and wide kernels; the grouped kernels take the rest
    (fp32, and d or d_ff too small for the wide tiles)."""
    f = lambda T, E=8, k=2, dt=moe.MOE_BF16, d=4096: moe.moe_expert_ffn_kernels(
        T, d, 14336, E, k, dt)
    assert f(1) == f(107) == "stream_gemm_kernel"
    assert f(108) == f(195) == ("grouped_gemm_kernel (128 x 64 tiles) + "
                                "wide_gemm_kernel (128-row token tiles) (W2)")
    assert f(196) == "wide_gemm_kernel (128-row token tiles)"
    assert f(160, d=64).startswith("grouped_gemm_kernel (128 x 64")  # too small for wide
    assert f(196) == "wide_gemm_kernel (128-row token tiles)"
    assert f(400) == "wide_gemm_kernel (128-row token tiles)"
    assert f(401) == f(4096) == "wide_gemm_kernel (256-row token tiles)"
    assert f(8, E=1, k=1) == "stream_gemm_kernel"          # one expert per GPU, decode share
    assert f(1024, E=1, k=1) == "wide_gemm_kernel (256-row token tiles)"
    assert not f(4096, dt=moe.MOE_F32).startswith("wide")
    assert f(8, E=65) == ""


def test_layer_kernel_labels_name_the_column_kernels_up_to_eight_tokens():
    """The fused layer takes the column kernels for one to eight tokens where
    the expert FFN alone would take the tile kernel, within their LDS limits
    (at most eight GEMM1 stages per workgroup, and eight GEMM2 stages up to
    four tokens, four from five to eight, on 256 CUs)."""
    f = lambda T, d=4096, d_ff=14336, E=8, k=2: moe.moe_forward_kernels(T, d, d_ff, E, k,
                                                                        moe.MOE_BF16)
    g = lambda T, d=4096, d_ff=14336, E=8, k=2: moe.moe_expert_ffn_kernels(T, d, d_ff, E, k,
                                                                           moe.MOE_BF16)
    for T in range(1, 9):
        assert f(T) == "stream_cols_kernel" and g(T) == "stream_gemm_kernel"
    hybrid = "stream_gemm_kernel + stream_cols_kernel (W2)"   # GEMM1 tiles, GEMM2 columns
    assert f(9) == f(32) == hybrid and g(9) == g(32) == "stream_gemm_kernel"
    assert f(33) == f(107) == "stream_gemm_kernel"
    assert f(9, d=8192) == "stream_gemm_kernel"          # GEMM2: one column stage at most
    assert f(16, E=64, k=4) == hybrid and f(17, E=64, k=4) == "stream_gemm_kernel"  # 64 assignments
    assert f(100) == g(100) and f(4096) == g(4096)
    assert f(4, E=64, k=8) == "stream_cols_kernel"       # 32 assignments, the most
    assert f(5, E=64, k=8) == "stream_gemm_kernel"       # 40
    assert f(4, d=32768) == "stream_cols_kernel"         # GEMM2: 8 stages per workgroup
    assert f(5, d=32768) == "stream_gemm_kernel"         # more than 4 at five tokens
    assert f(8, d_ff=16384) == "stream_cols_kernel"      # GEMM1: 8 stages
    assert f(1, d_ff=16896) == "stream_gemm_kernel"      # 9 would be needed
    assert moe.moe_forward_kernels(4, 4096, 14336, 8, 2, moe.MOE_F32) == \
        moe.moe_expert_ffn_kernels(4, 4096, 14336, 8, 2, moe.MOE_F32)
    assert f(8, E=65) == ""


def _rc(name, *args):
    return getattr(moe.lib(), name)(*args)


def test_forward_argument_checks_return_codes():
    f = "moe_forward"
    ok_args = dict(x=FAKE, Wg=FAKE, W1=FAKE, W3=FAKE, W2=FAKE, dt=moe.MOE_BF16, T=32, d=128,
                   d_ff=256, E=8, k=2, y=FAKE, ws=FAKE, ws_bytes=0, stream=None)

    def call(**over):
        a = dict(ok_args, **over)
        return _rc(f, a["x"], a["Wg"], a["W1"], a["W3"], a["W2"], a["dt"], a["T"], a["d"],
                   a["d_ff"], a["E"], a["k"], a["y"], a["ws"], a["ws_bytes"], a["stream"])

    assert call(ws_bytes=0) == moe.MOE_ERR_WORKSPACE
    assert "workspace" in moe.lib().moe_last_error().decode()
    assert call(x=None) == moe.MOE_ERR_INVALID_ARG
    assert call(W2=ctypes.c_void_p((1 << 20) + 8)) == moe.MOE_ERR_INVALID_ARG  # misaligned
    assert call(k=9) == moe.MOE_ERR_UNSUPPORTED
    assert call(E=65) == moe.MOE_ERR_UNSUPPORTED
    assert call(d=100) == moe.MOE_ERR_UNSUPPORTED
    assert call(d_ff=200) == moe.MOE_ERR_UNSUPPORTED
    assert call(T=-5) == moe.MOE_ERR_INVALID_ARG
    assert call(dt=7) == moe.MOE_ERR_INVALID_ARG
    # T = 0 enqueues nothing and succeeds even with NULL buffers
    assert call(T=0, x=None, y=None, ws=None) == moe.MOE_OK


def test_other_entry_points_reject_before_launch():
    L = moe.lib()
    assert L.moe_route(None, FAKE, moe.MOE_BF16, 4, 64, 8, 2, FAKE, FAKE, None, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert L.moe_route(FAKE, FAKE, moe.MOE_BF16, 4, 64, 8, 0, FAKE, FAKE, None, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert L.moe_expert_ffn(FAKE, FAKE, FAKE, FAKE, FAKE, moe.MOE_BF16, 4, 64, 64, 8, 2, FAKE,
                            FAKE, 16, None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_combine(FAKE, FAKE, FAKE, None, moe.MOE_BF16, 4, 64, 2, None, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert L.moe_rmsnorm(FAKE, moe.MOE_BF16, 4, 64, ctypes.c_float(-1.0), FAKE, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert L.moe_block_forward(FAKE, FAKE, FAKE, FAKE, FAKE, moe.MOE_BF16, 4, 64, 64, 8, 2,
                               ctypes.c_float(1e-5), None, None, FAKE, 0, None) == \
        moe.MOE_ERR_WORKSPACE
    assert L.moe_permute(FAKE, FAKE, moe.MOE_BF16, 4, 64, 8, 2, None, FAKE, FAKE, FAKE, FAKE,
                         None, 0, None) == moe.MOE_ERR_INVALID_ARG


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(moe, "_lib", None)
    monkeypatch.setattr(moe, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        moe.lib()


def test_route_balance_workspace_size_rules():
    ws = moe.moe_route_balance_workspace_size
    assert ws(0, 8) == 0 and ws(16, 65) == 0 and ws(16, 0) == 0
    # one fp64 and one int32 statistics row per router workgroup
    assert ws(32, 8) >= 32 * 8 * 12
    assert ws(16384, 8) >= 4096 * 8 * 12
    assert ws(16384, 8) > ws(4096, 8) > 0


def test_binding_rejects_mismatched_tensors_before_the_call():
    """The binding checks dtypes and shapes on the host: a bf16 gate matrix or
    experts of another width would otherwise be read past their ends."""
    import torch

    T, d, d_ff, E = 4, 64, 128, 8
    x = torch.zeros((T, d), dtype=torch.bfloat16)
    Wg = torch.zeros((E, d), dtype=torch.float32)
    W1 = torch.zeros((E, d_ff, d), dtype=torch.bfloat16)
    W2 = torch.zeros((E, d, d_ff), dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="fp32"):
        moe.moe_route(x, Wg.to(torch.bfloat16), 2)
    with pytest.raises(ValueError, match="Wg"):
        moe.moe_route(x, torch.zeros((E, d + 64)), 2)
    with pytest.raises(TypeError, match="W1"):
        moe.moe_forward(x, Wg, W1.float(), W1, W2, 2)
    with pytest.raises(ValueError, match="expert shapes"):
        moe.moe_forward(x, Wg, W1, W1, W1, 2)
    with pytest.raises(ValueError, match="experts"):
        moe.moe_forward(x, Wg[:4], W1, W1, W2, 2)
    with pytest.raises(ValueError, match="topk_idx"):
        moe.moe_route(x, Wg, 2, topk_idx=torch.zeros((T, 3), dtype=torch.int32))
    # well-formed host tensors pass the checks and stop at the device check
    with pytest.raises(ValueError, match="GPU"):
        moe.moe_forward(x, Wg, W1, W1, W2, 2)


def test_noalloc_entry_point_rejects_shapes_beyond_its_array():
    """moe_forward_noalloc works inside the library's fixed static array:
    shapes whose workspace exceeds it are refused before anything else
    happens (no device is touched), smaller ones pass this check."""
    L = moe.lib()
    cap = L.moe_forward_noalloc_max_scratch()
    assert cap == 96 << 20
    ws = moe.moe_workspace_size
    assert ws(292, 4096, 14336, 8, 2, moe.MOE_BF16) <= cap < ws(293, 4096, 14336, 8, 2,
                                                               moe.MOE_BF16)

    def call(T):
        return L.moe_forward_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, moe.MOE_BF16, T, 4096, 14336,
                                     8, 2, FAKE, None)

    assert call(293) == moe.MOE_ERR_WORKSPACE
    assert "static array" in L.moe_last_error().decode()
    assert call(-1) == moe.MOE_ERR_INVALID_ARG
    assert call(0) == moe.MOE_OK
