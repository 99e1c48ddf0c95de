"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Every input comes from the seeded generator; the oracle receives host copies
of exactly the tensors the GPU used.  Routing indices, counts and the
grouping must match bit for bit (near-tie tokens excepted, counted and
reported); y must match within the normwise bound of its dtype.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import (NEAR_TIE, TOL, check_near_rounding_floor, check_routing, log,
                    normwise, to_np)
from sparse_mixture_experts_31_amd import moe
from sparse_mixture_experts_31_amd.inputs import WORKLOADS, Workload, make_layer

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(w: Workload, seed=0):
    log(f"case {w.name}: T={w.T} d={w.d} d_ff={w.d_ff} E={w.E} k={w.k} {w.dtype} seed={seed}")
    return make_layer(w, DEV, seed)


def _forward_and_check(w: Workload, L, rows=None, tol=None):
    """moe_forward on the GPU vs the oracle on `rows` (default all tokens)."""
    y = moe.moe_forward(L["x"], L["Wg"], L["W1"], L["W3"], L["W2"], w.k)
    torch.cuda.synchronize()
    if rows is None:
        rows = np.arange(w.T)
    ref = oracle.moe_rows(L["x"], L["Wg"], L["W1"], L["W3"], L["W2"], w.k, rows=rows)
    idx, gw = moe.moe_route(L["x"], L["Wg"], w.k)
    torch.cuda.synchronize()
    same, _, _ = check_routing(to_np(idx)[rows], to_np(gw)[rows], ref)
    got = to_np(y)[rows]
    err = normwise(got[same], ref["y"][same])
    log(f"  normwise error {err:.3e} over {same.sum()} tokens")
    assert err <= (tol if tol is not None else TOL[w.dtype])
    assert np.isfinite(got).all()
    return y, ref


# ------------------------------------------------------------------ small shapes

SMALL = [
    WORKLOADS["tiny"],
    Workload("mid-bf16", 10, T=300, d=512, d_ff=1024),
    Workload("mid-f32-ragged-n", 11, T=300, d=256, d_ff=320, dtype="f32"),
    Workload("decode-like", 12, T=20, d=512, d_ff=960),
    Workload("e13-k3", 13, T=257, d=192, d_ff=448, E=13, k=3),
    Workload("e64-k8", 14, T=100, d=256, d_ff=256, E=64, k=8),
    Workload("k1", 15, T=128, d=256, d_ff=512, k=1),
    Workload("one-token", 16, T=1, d=512, d_ff=512),
    Workload("wide-few", 17, T=700, d=320, d_ff=704, E=4, k=2),
    # more wide tiles than workgroups (the load ring crosses tiles), the
    # shortest k-loop (d = 128) and a W2 tile half past N
    Workload("wide-many", 18, T=2048, d=128, d_ff=2304),
    # every token takes both of two experts: 300 rows each, a full 256-row
    # tile and a ragged one of 44 rows
    Workload("wide-narrow", 19, T=300, d=256, d_ff=512, E=2, k=2),
    # ~300 rows per expert from a random split: ragged last tiles again
    Workload("wide-narrow-k1", 22, T=600, d=192, d_ff=640, E=2, k=1),
    # decode-sized on the weight-streaming kernels with more tiles than
    # workgroups (the ring crosses tile boundaries), 2 K ranges of 512 in
    # GEMM1 and 10 in GEMM2
    Workload("stream-tiles", 23, T=24, d=1024, d_ff=5120),
    # 40 rows per expert with d too small for the wide tiles: the grouped
    # kernels with 128 x 64 tiles (bf16)
    Workload("grouped-bf16", 26, T=160, d=64, d_ff=1024),
    # 25-48 rows per expert: grouped GEMM1, then GEMM2 on the wide kernels
    # with 128-row token tiles and their split last round
    Workload("mixed-mid", 50, T=160, d=512, d_ff=1024),
    # degenerate routing: one expert (every gate is 1), and every token
    # taking all eight experts
    Workload("e1-k1", 27, T=50, d=256, d_ff=512, E=1, k=1),
    Workload("k-all", 28, T=40, d=256, d_ff=256, E=8, k=8),
    # the weight stream's even K split with few tiles (from nine tokens on;
    # fewer go to the column kernels below): GEMM1 8 tiles of 8 K ranges on
    # 64 workgroups (8 pieces a tile) ...
    Workload("split-8-pieces", 29, T=9, d=4096, d_ff=512, E=1, k=1),
    # ... GEMM2 8 tiles of 14 K ranges on 56 workgroups (7 pieces a tile)
    Workload("split-7-pieces", 30, T=9, d=512, d_ff=7168, E=2, k=1),
    # ... both GEMMs split, pieces of 1-3 ranges crossing tile boundaries
    Workload("split-9-tokens", 31, T=9, d=1024, d_ff=3584, E=8, k=2),
    # ... and in a layer of two experts with 24 rows each, where GEMM2 has 16
    # tiles (whole tiles would leave most CUs idle)
    Workload("split-two-experts", 32, T=24, d=1024, d_ff=2048, E=2, k=2),
    # one to four tokens: every workgroup streams its own columns of every
    # active expert (GEMM1 8 columns a stage, GEMM2 16) ...
    # ... one stage each on 64 and 256 workgroups, one expert active
    Workload("cols-one-token", 33, T=1, d=4096, d_ff=512, E=4, k=1),
    # ... GEMM1 3 or 4 stages on 256 workgroups, GEMM2 on 32
    Workload("cols-mixed-stages", 34, T=1, d=512, d_ff=7168, E=8, k=2),
    Workload("cols-three-tokens", 35, T=3, d=1024, d_ff=3584, E=8, k=2),
    # ... 32 assignments (the most), up to 32 experts active
    Workload("cols-e64-k8", 36, T=4, d=512, d_ff=1024, E=64, k=8),
    # ... one expert with four rows
    Workload("cols-e1-k1", 37, T=4, d=512, d_ff=1024, E=1, k=1),
    # ... GEMM2 two stages per workgroup (waves 0 and 1), 16 K ranges in GEMM1
    Workload("cols-two-stages", 38, T=2, d=8192, d_ff=512, E=4, k=2),
    # ... eight stages per workgroup (both accumulators of every wave):
    # GEMM2 (d = 32768, 64 K ranges in GEMM1), then GEMM1 (d_ff = 16384)
    Workload("cols-eight-stages-w2", 39, T=1, d=32768, d_ff=512, E=2, k=1),
    Workload("cols-eight-stages-w13", 40, T=2, d=512, d_ff=16384, E=2, k=1),
    # five to eight tokens: eight token rows per expert at most, two per wave
    Workload("cols-eight-tokens", 41, T=8, d=1024, d_ff=3584, E=8, k=2),
    Workload("cols-six-rows-e1", 43, T=6, d=512, d_ff=1024, E=1, k=1),
    Workload("cols-tok8-e64-k4", 44, T=8, d=512, d_ff=1024, E=64, k=4),
    # ... GEMM2 two and four stages per workgroup (its most at eight rows),
    # GEMM1 eight
    Workload("cols-tok8-two-stages", 45, T=7, d=8192, d_ff=512, E=4, k=2),
    Workload("cols-tok8-four-stages", 46, T=5, d=16384, d_ff=512, E=2, k=1),
    Workload("cols-tok8-eight-stages-w13", 47, T=6, d=512, d_ff=16384, E=2, k=1),
    # ... and past four GEMM2 stages the tile kernel takes the layer again
    Workload("cols-tok8-too-wide", 48, T=5, d=32768, d_ff=512, E=2, k=1),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_forward_small(w):
    L = _case(w)
    _forward_and_check(w, L)


@pytest.mark.parametrize("name", ["mid", "decode", "prefill"])
def test_layer_error_is_the_output_rounding(name):
    """With the SwiGLU intermediate quantised at the same point on both sides,
    the only differences left are fp32 versus fp64 summation and the final
    rounding of y to bf16: the GPU's normwise error is that of rounding the
    exact result once, within 25%."""
    w = {"mid": Workload("mid-bf16", 10, T=300, d=512, d_ff=1024)}.get(name) or WORKLOADS[name]
    L = _case(w)
    y = moe.moe_forward(L["x"], L["Wg"], L["W1"], L["W3"], L["W2"], w.k)
    idx, gw = moe.moe_route(L["x"], L["Wg"], w.k)
    torch.cuda.synchronize()
    rows = np.arange(w.T) if w.T <= 300 else np.random.default_rng(5).choice(w.T, 48, replace=False)
    ref = oracle.moe_rows(L["x"], L["Wg"], L["W1"], L["W3"], L["W2"], w.k, rows=rows,
                          round_mid=True)
    same, _, _ = check_routing(to_np(idx)[rows], to_np(gw)[rows], ref)
    err, floor = check_near_rounding_floor(to_np(y)[rows][same], ref["y"][same])
    log(f"  normwise {err:.3e} against a one-rounding floor of {floor:.3e}")


@pytest.mark.parametrize("w", [
    Workload("mid-bf16", 10, T=300, d=512, d_ff=1024),
    # from 1024 tokens on, Wg sits in LDS and each wave walks tokens
    Workload("many-bf16", 24, T=1100, d=512, d_ff=512),
    Workload("many-f32-e13", 25, T=1030, d=512, d_ff=256, E=13, k=3, dtype="f32"),
], ids=lambda w: w.name)
def test_route_scores_are_rounded_exact_dot_products(w):
    L = _case(w)
    T, E = w.T, w.E
    logits = torch.empty((T, E), dtype=torch.float32, device=DEV)
    idx, gw = moe.moe_route(L["x"], L["Wg"], w.k, logits=logits)
    torch.cuda.synchronize()
    ref = oracle.route(L["x"], L["Wg"], w.k)
    # fp64-accumulated scores, rounded once: equal to the oracle's scores
    # rounded to fp32 up to one unit in the last place
    want = ref["logits"].astype(np.float32)
    got = to_np(logits)
    ulp = np.spacing(np.abs(want))
    assert np.all(np.abs(got - want) <= ulp), np.abs(got - want).max()
    assert (got == want).mean() > 0.999
    check_routing(to_np(idx), to_np(gw), ref)
    np.testing.assert_allclose(to_np(gw).sum(1), 1.0, atol=2e-7)


@pytest.mark.parametrize("T", [300, 1100], ids=["four-wave", "lds"])
def test_exact_ties_go_to_the_lower_index(T):
    """Equal scores go to the lower expert index, for the set and the order.
    Duplicated gate rows give bit-identical scores on both sides (the same
    products summed in the same order), so the choice among them is decided
    by the tie rule alone: every token's indices must match the oracle's bit
    for bit with no exemption.  Wg[6] = Wg[1] and Wg[5] = Wg[2] give ties
    between first and second choice (1 and 6 on top) and between second and
    third (2 and 5 competing for the second place); Wg = 0 makes every score
    0, so every token takes experts 0 and 1 with gates 1/2.  Below 1024
    tokens the router splits a token's row over four waves, from 1024 on Wg
    sits in LDS; moe_route_balance routes through the one-wave form."""
    w = Workload(f"ties-{T}", 40, T=T, d=512, d_ff=512)
    L = _case(w)
    Wg = L["Wg"].clone()
    Wg[6] = Wg[1]
    Wg[5] = Wg[2]
    ref = oracle.route(L["x"], Wg, w.k)
    lg = ref["logits"]
    assert (lg[:, 6] == lg[:, 1]).all() and (lg[:, 5] == lg[:, 2]).all()
    top12 = int((np.sort(ref["idx"], 1) == [1, 6]).all(1).sum())
    second = int(((ref["idx"][:, 1] == 2) & (lg[:, 5] == lg[:, 2])).sum())
    log(f"  {top12} tokens with tied first and second choice (1, 6), {second} with expert 2 "
        f"second tied with 5")
    assert top12 > 0 and second > 0
    # where the tied pair holds the top two places the lower index comes first
    both = np.isin(ref["idx"], [1, 6]).all(1)
    assert (ref["idx"][both] == [1, 6]).all()
    for name, fn in (("route", lambda: moe.moe_route(L["x"], Wg, w.k)),
                     ("route_balance", lambda: moe.moe_route_balance(L["x"], Wg, w.k)[:2])):
        idx, gw = fn()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_np(idx), ref["idx"], name)
        np.testing.assert_allclose(to_np(gw), ref["gates"], atol=2e-6, err_msg=name)
        # tied first and second choice: equal gates of exactly 1/2
        assert (to_np(gw)[both] == 0.5).all(), name
    zero = torch.zeros_like(Wg)
    for idx, gw in (moe.moe_route(L["x"], zero, w.k), moe.moe_route_balance(L["x"], zero, w.k)[:2]):
        torch.cuda.synchronize()
        assert (to_np(idx) == [0, 1]).all()
        assert (to_np(gw) == 0.5).all()


def test_permute_is_the_oracles_stable_grouping():
    w = Workload("e13-k3", 13, T=1500, d=192, d_ff=448, E=13, k=3)
    L = _case(w)
    ref = oracle.route(L["x"], L["Wg"], w.k)
    # feed the oracle's own routing through the GPU dispatch
    idx = torch.from_numpy(ref["idx"]).to(DEV)
    P = moe.moe_permute(L["x"], idx, w.E)
    torch.cuda.synchronize()
    want = oracle.permute(ref["idx"], w.E)
    for key in ("counts", "offsets", "row_of", "token_of"):
        np.testing.assert_array_equal(to_np(P[key]).reshape(want[key].shape), want[key], key)
    # x_perm holds exact copies of the token rows
    xp = P["x_perm"].cpu()
    xs = L["x"].cpu()[torch.from_numpy(want["token_of"]).long()]
    assert torch.equal(xp, xs)


@pytest.mark.parametrize("T", [777, 5000])   # one workgroup; chunks over the chip
def test_permute_empty_and_skewed_groups(T):
    E, k, d = 8, 2, 128
    idx = torch.tensor([[3, 5]] * T, dtype=torch.int32, device=DEV)
    x = torch.randn((T, d), device=DEV).to(torch.bfloat16)
    P = moe.moe_permute(x, idx, E)
    torch.cuda.synchronize()
    want = oracle.permute(idx.cpu().numpy(), E)
    for key in ("counts", "offsets", "row_of", "token_of"):
        np.testing.assert_array_equal(to_np(P[key]).reshape(want[key].shape), want[key], key)
    P0 = moe.moe_permute(x[:0], idx[:0], E)
    torch.cuda.synchronize()
    assert to_np(P0["offsets"]).tolist() == [0] * (E + 1)


def _stable_grouping(idx, E):
    """Rows of the valid assignments in expert order, ties in assignment
    order (a stable sort by expert); entries outside [0, E) get row -1."""
    flat = idx.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    order = np.flatnonzero(valid)[np.argsort(flat[valid], kind="stable")]
    row_of = np.full(flat.shape, -1, np.int32)
    row_of[order] = np.arange(order.size, dtype=np.int32)
    return counts, offsets, row_of.reshape(idx.shape), (order // idx.shape[1]).astype(np.int32)


@pytest.mark.parametrize("T,E,k,bad", [
    (2048, 8, 2, False),     # 4096 assignments: the single-workgroup form
    (2049, 8, 2, False),     # 4098: the chunked form, a 2-assignment last chunk
    (700, 13, 3, True),      # single workgroup, out-of-range entries
    (1400, 13, 3, True),     # chunked, E = 13 (lane groups of 13), out-of-range entries
    (5000, 1, 1, False),     # one expert
    (3000, 64, 8, True),     # E = 64: one lane per expert
    (150000, 8, 2, False),   # 300000 assignments: 640 per chunk, 469 chunks
])
def test_permute_both_dispatch_forms(T, E, k, bad):
    rng = np.random.default_rng(T + E + k)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(min(T, 4096))])
    idx = np.resize(idx, (T, k)).astype(np.int32)
    if E > 1:
        # skew: a quarter of the tokens send their first choice to expert
        # E - 1 (a slot that held E - 1 takes the old first choice instead)
        sel = np.flatnonzero(rng.random(T) < 0.25)
        for j in range(1, k):
            hit = sel[idx[sel, j] == E - 1]
            idx[hit, j] = idx[hit, 0]
        idx[sel, 0] = E - 1
    if bad:
        idx.reshape(-1)[rng.choice(T * k, T * k // 50, replace=False)] = \
            rng.choice([-1, E, 1 << 30, -(1 << 30)], T * k // 50)
    need = moe.moe_permute_workspace_size(T, E, k)
    assert (need == 0) == (T * k <= 4096)
    x = torch.randn((T, 64), device=DEV).to(torch.bfloat16)
    P = moe.moe_permute(x, torch.from_numpy(idx).to(DEV), E)
    torch.cuda.synchronize()
    counts, offsets, row_of, token_of = _stable_grouping(idx, E)
    if not bad:
        want = oracle.permute(idx, E)
        np.testing.assert_array_equal(want["row_of"], row_of)
    np.testing.assert_array_equal(to_np(P["counts"]), counts)
    np.testing.assert_array_equal(to_np(P["offsets"]), offsets)
    np.testing.assert_array_equal(to_np(P["row_of"]), row_of)
    n = int(offsets[-1])
    np.testing.assert_array_equal(to_np(P["token_of"])[:n], token_of)
    # every placed row holds its token's row of x
    xp = P["x_perm"][:n].cpu()
    assert torch.equal(xp, x.cpu()[torch.from_numpy(token_of).long()])


def test_pieces_expert_ffn_and_combine():
    """moe_expert_ffn and moe_combine on their own, fed from the oracle's grouping."""
    w = Workload("mid-bf16", 10, T=300, d=512, d_ff=1024)
    L = _case(w)
    ref = oracle.route(L["x"], L["Wg"], w.k)
    grp = oracle.permute(ref["idx"], w.E)
    tok = torch.from_numpy(grp["token_of"]).long().to(DEV)
    x_perm = L["x"][tok].contiguous()
    offsets = torch.from_numpy(grp["offsets"]).to(DEV)
    out_perm = moe.moe_expert_ffn(x_perm, offsets, L["W1"], L["W3"], L["W2"], w.T, w.k)
    torch.cuda.synchronize()
    experts = np.repeat(np.arange(w.E), grp["counts"])
    rows = np.random.default_rng(0).choice(w.T * w.k, 40, replace=False)
    xr = to_np(x_perm).astype(np.float64)
    want = np.stack([oracle.swiglu_expert(xr[r], L["W1"], L["W3"], L["W2"], experts[r])
                     for r in rows])
    err = normwise(to_np(out_perm)[rows], want)
    log(f"  expert_ffn normwise {err:.3e}")
    assert err <= TOL["bf16"]
    # combine with the oracle's gates and rows
    row_of = torch.from_numpy(grp["row_of"]).to(DEV)
    gates = torch.from_numpy(ref["gates"].astype(np.float32)).to(DEV)
    y = moe.moe_combine(out_perm, row_of, gates)
    torch.cuda.synchronize()
    op = to_np(out_perm).astype(np.float64)
    want_y = np.einsum("tk,tkd->td", gates.cpu().double().numpy(), op[grp["row_of"]])
    assert normwise(to_np(y), want_y) < 4e-3   # one bf16 rounding of y
    # residual variant
    res = torch.randn_like(y)
    y2 = moe.moe_combine(out_perm, row_of, gates, residual=res)
    torch.cuda.synchronize()
    assert normwise(to_np(y2), want_y + to_np(res)) < 4e-3


def test_expert_ffn_leaves_rows_past_the_experts_untouched():
    """moe_expert_ffn writes exactly the rows the experts own.  At the
    smallest batches (fewer than four rows per expert) the weight-streaming
    kernels split tiles along K into pieces and sum them in a second pass;
    with offsets[E] below T*k the rows past it belong to no expert and must
    keep their contents bit for bit."""
    T, k, E, d, d_ff = 12, 2, 8, 2048, 2048
    w = Workload("ffn-rows", 41, T=T, d=d, d_ff=d_ff, E=E, k=k)
    assert moe.moe_expert_ffn_kernels(T, d, d_ff, E, k, torch.bfloat16) == "stream_gemm_kernel"
    L = _case(w)
    counts = np.array([3, 0, 4, 2, 0, 5, 1, 3], np.int32)   # 18 of the 24 rows
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    n = int(offsets[-1])
    x_perm = L["x"][np.arange(T * k) % T].contiguous()
    sentinel = torch.full((T * k, d), 7.0, dtype=torch.bfloat16, device=DEV)
    out = sentinel.clone()
    moe.moe_expert_ffn(x_perm, torch.from_numpy(offsets).to(DEV), L["W1"], L["W3"], L["W2"], T,
                       k, out_perm=out)
    torch.cuda.synchronize()
    assert torch.equal(out[n:], sentinel[n:])
    experts = np.repeat(np.arange(E), counts)
    xr = to_np(x_perm).astype(np.float64)
    want = np.stack([oracle.swiglu_expert(xr[r], L["W1"], L["W3"], L["W2"], experts[r])
                     for r in range(n)])
    err = normwise(to_np(out)[:n], want)
    log(f"  expert_ffn over {n} of {T * k} rows: normwise {err:.3e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("M", [8, 1024])
def test_expert_parallel_shard_at_the_mixtral_shape(M):
    """One GPU's share under expert parallelism (one expert per GPU): the
    expert GEMMs of one Mixtral-sized expert on the M rows it received (8 at
    decode, 1024 at prefill), every row (M = 8) or 24 sampled rows against
    the oracle's expert."""
    w = Workload("ep-shard", 5, T=M, d=4096, d_ff=14336, E=1, k=1)
    L = _case(w)
    offsets = torch.tensor([0, M], dtype=torch.int32, device=DEV)
    out = moe.moe_expert_ffn(L["x"], offsets, L["W1"], L["W3"], L["W2"], M, 1)
    torch.cuda.synchronize()
    rows = np.arange(M) if M <= 24 else np.sort(np.random.default_rng(M).choice(M, 24,
                                                                               replace=False))
    xr = to_np(L["x"]).astype(np.float64)
    want = np.stack([oracle.swiglu_expert(xr[r], L["W1"], L["W3"], L["W2"], 0) for r in rows])
    err = normwise(to_np(out)[rows], want)
    log(f"  ep shard M={M} ({moe.moe_expert_ffn_kernels(M, 4096, 14336, 1, 1, torch.bfloat16)}):"
        f" normwise {err:.3e} over {len(rows)} rows")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("w", [
    Workload("forced", 20, T=200, d=256, d_ff=512),
    # decode-sized (T*k/E <= 24): the weight-streaming kernels, here with
    # three token tiles of 32 rows for each of the two experts
    Workload("forced-stream", 21, T=96, d=512, d_ff=1024),
    # 32 tokens: GEMM2 on the column kernel, each expert's 32 rows in two
    # chunks of 16 (its W2 rows streamed once per chunk)
    Workload("forced-chunks", 49, T=32, d=512, d_ff=1024),
], ids=lambda w: w.name)
def test_all_tokens_to_two_experts_and_untouched_experts(w):
    """Every token routes to experts 3 and 5; the other six get no rows, and
    NaN in their weights must not reach y (their parameters are not read)."""
    L = _case(w)
    Wg = torch.zeros_like(L["Wg"])
    Wg[3, 0] = 10.0
    Wg[5, 0] = 5.0
    x = L["x"].clone()
    x[:, 0] = 4.0
    L = dict(L, Wg=Wg, x=x)
    y, ref = _forward_and_check(w, L)
    assert (ref["idx"] == np.array([3, 5])).all()
    P = {n: L[n].clone() for n in ("W1", "W3", "W2")}
    for e in (0, 1, 2, 4, 6, 7):
        for n in P:
            P[n][e] = float("nan")
    y_nan = moe.moe_forward(x, Wg, P["W1"], P["W3"], P["W2"], w.k)
    torch.cuda.synchronize()
    assert torch.equal(y_nan, y)


def test_zero_tokens_is_a_no_op():
    w = Workload("mid-bf16", 10, T=300, d=512, d_ff=1024)
    L = _case(w)
    y = torch.full((0, w.d), 7.0, device=DEV, dtype=torch.bfloat16)
    moe.moe_forward(L["x"][:0], L["Wg"], L["W1"], L["W3"], L["W2"], w.k, y=y)
    torch.cuda.synchronize()


def test_runs_are_bit_identical():
    w = Workload("mid-bf16", 10, T=300, d=512, d_ff=1024)
    L = _case(w)
    y1 = moe.moe_forward(L["x"], L["Wg"], L["W1"], L["W3"], L["W2"], w.k)
    y2 = moe.moe_forward(L["x"], L["Wg"], L["W1"], L["W3"], L["W2"], w.k)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("name", ["stream-tiles", "split-9-tokens", "cols-three-tokens",
                                  "cols-eight-tokens", "grouped-bf16", "wide-narrow"])
def test_side_streams_give_the_default_streams_result(name):
    """moe_forward on two side streams at once, each with its own output and
    workspace, matches the default stream's result bit for bit: every launch
    of the layer goes to the stream it is given, and nothing is shared
    between calls."""
    w = next(v for v in SMALL if v.name == name)
    L = _case(w)
    y0 = moe.moe_forward(L["x"], L["Wg"], L["W1"], L["W3"], L["W2"], w.k)
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    outs = []
    for s in (torch.cuda.Stream(), torch.cuda.Stream()):   # default priority
        s.wait_stream(cur)
        with torch.cuda.stream(s):
            y = torch.empty_like(L["x"])
            ws = moe.workspace(w.T, w.d, w.d_ff, w.E, w.k, L["x"].dtype, L["x"].device)
            moe.moe_forward(L["x"], L["Wg"], L["W1"], L["W3"], L["W2"], w.k, y=y, ws=ws,
                            stream=s)
            outs.append(y)
    torch.cuda.synchronize()
    for y in outs:
        assert torch.equal(y, y0)


@pytest.mark.parametrize("name", ["tiny", "stream-tiles", "split-9-tokens", "cols-three-tokens",
                                  "grouped-bf16", "mixed-mid", "wide-narrow", "wide-many"])
def test_profiled_layer_is_the_layer(name):
    """moe_forward_profiled, with all six stage events or only GEMM1's pair,
    gives moe_forward's output bit for bit, and its events are recorded in
    stage order on the launch stream (every elapsed time between consecutive
    ones is >= 0, GEMM1's > 0)."""
    import bench
    w = next(v for v in SMALL if v.name == name)
    L = _case(w)
    y0 = moe.moe_forward(L["x"], L["Wg"], L["W1"], L["W3"], L["W2"], w.k)
    ev = bench.HipEvents()
    e = [ev.create() for _ in range(6)]
    y1 = moe.moe_forward_profiled(L["x"], L["Wg"], L["W1"], L["W3"], L["W2"], w.k, e)
    torch.cuda.synchronize()
    gaps = [ev.elapsed_ms(e[i], e[i + 1]) for i in range(5)]
    g = [ev.create(), ev.create()]
    y2 = moe.moe_forward_profiled(L["x"], L["Wg"], L["W1"], L["W3"], L["W2"], w.k,
                                  [None, None, g[0], g[1], None, None])
    torch.cuda.synchronize()
    g1 = ev.elapsed_ms(g[0], g[1])
    for h in e + g:
        ev.destroy(h)
    log(f"  stage ms {[round(v, 4) for v in gaps]}, GEMM1 alone {g1:.4f}")
    assert torch.equal(y1, y0) and torch.equal(y2, y0)
    assert min(gaps) >= 0.0 and gaps[2] > 0.0 and g1 > 0.0


@pytest.mark.parametrize("name", ["stream-tiles", "split-9-tokens", "cols-three-tokens",
                                  "cols-eight-tokens", "grouped-bf16", "wide-narrow"])
def test_layer_replays_from_a_hip_graph(name):
    """moe_forward captured once in a HIP graph (no allocation, memset or
    synchronisation inside the layer) and replayed on new inputs copied into
    the captured x, with eager work and synchronisations between replays:
    every replay equals the eager layer on the same input bit for bit."""
    w = next(v for v in SMALL if v.name == name)
    L = _case(w)
    xs = [L["x"]] + [(torch.randn_like(L["x"].float()) * (1 + i)).to(L["x"].dtype)
                     for i in range(3)]
    x = xs[0].clone()
    y = torch.empty_like(x)
    ws = moe.workspace(w.T, w.d, w.d_ff, w.E, w.k, x.dtype, x.device)
    args = (L["Wg"], L["W1"], L["W3"], L["W2"], w.k)
    moe.moe_forward(x, *args, y=y, ws=ws)   # first launches set kernel attributes
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            moe.moe_forward(x, *args, y=y, ws=ws, stream=s)
    torch.cuda.synchronize()
    for xi in xs:
        want = moe.moe_forward(xi, *args)          # eager, own workspace
        torch.cuda.synchronize()
        x.copy_(xi)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, want)


def test_rmsnorm_matches_oracle_bit_for_bit():
    h = (torch.randn((333, 4096), device=DEV) * 3).to(torch.bfloat16)
    eps = float(np.float32(1e-5))
    out = moe.moe_rmsnorm(h, eps)
    torch.cuda.synchronize()
    want = oracle.rmsnorm_rows(to_np(h).astype(np.float64), eps, round_bf16=True)
    np.testing.assert_array_equal(to_np(out).astype(np.float64), want)


# ------------------------------------------------------------------ the stack


def _stack_check(w: Workload, blocks, h0, sample):
    """Run w.blocks block steps h <- h + moe(rms_norm(h)) on the GPU, keeping
    every block's input state, and check each block against the oracle's
    block taking that same bf16 state as its input (the state is an input
    of the block exactly as x is of a layer; the oracle's arithmetic stays
    its own, the plain fp64 definition with no intermediate rounding):

    * routing of every token in every block: the oracle routes the GPU's
      block input after its own rms_norm and bf16 rounding (bit-identical
      to the GPU's normalised rows), exact up to the near-tie exemptions;
    * the block output of the sampled tokens against the oracle's block
      step from the same input: normwise error within the bf16 bound.

    The free-running end-to-end distance (the oracle iterating its own
    states from h0) is reported, not gated: through 32 residual blocks a
    difference of one bf16 rounding grows, and a token that meets a
    near-tie takes another expert from there on."""
    eps = float(np.float32(w.eps))
    h = h0.clone()
    ws = moe.workspace(w.T, w.d, w.d_ff, w.E, w.k, h.dtype)
    states, routes = [], []
    for B in blocks:
        idx = torch.empty((w.T, w.k), dtype=torch.int32, device=DEV)
        gw = torch.empty((w.T, w.k), dtype=torch.float32, device=DEV)
        states.append(h.clone())
        moe.moe_block_forward(h, B["Wg"], B["W1"], B["W3"], B["W2"], w.k, eps, topk_idx=idx,
                              topk_w=gw, ws=ws)
        routes.append((idx, gw))
    states.append(h.clone())
    torch.cuda.synchronize()
    worst, exempt = 0.0, 0
    for b, B in enumerate(blocks):
        h_in = to_np(states[b]).astype(np.float64)
        xn = oracle.rmsnorm_rows(h_in, eps, round_bf16=True)
        r_all = oracle.route(torch.from_numpy(xn).float().to(torch.bfloat16), B["Wg"], w.k)
        same_all, ns, no = check_routing(to_np(routes[b][0]), to_np(routes[b][1]), r_all,
                                         label=f"block {b}")
        exempt += ns + no
        hb = h_in[sample].copy()
        r = oracle.block_step(hb, B["Wg"], B["W1"], B["W3"], B["W2"], w.k, eps)
        np.testing.assert_array_equal(r["idx"], r_all["idx"][sample])
        keep = same_all[sample]
        got = to_np(states[b + 1])[sample].astype(np.float64)
        err = normwise(got[keep], hb[keep])
        worst = max(worst, err)
        if b < 2 or b == len(blocks) - 1:
            log(f"  block {b}: output normwise {err:.3e} over {keep.sum()} tokens")
        assert err <= TOL["bf16"], (b, err)
    log(f"  stack: {len(blocks)} blocks, worst per-block output error {worst:.3e} "
        f"(bound {TOL['bf16']}), {exempt} near-tie routing exemptions")
    # report only: the oracle running free from h0 on the sample
    hR = to_np(h0)[sample].astype(np.float64).copy()
    split = np.zeros(len(sample), bool)
    for b, B in enumerate(blocks):
        r = oracle.block_step(hR, B["Wg"], B["W1"], B["W3"], B["W2"], w.k, eps)
        split |= (np.sort(r["idx"], 1) != np.sort(to_np(routes[b][0])[sample], 1)).any(1)
    got = to_np(h)[sample]
    log(f"  free-running end to end (reported, not gated): GPU vs oracle "
        f"{normwise(got, hR):.3e}; {split.sum()}/{len(sample)} sampled tokens left the "
        f"oracle's routing at some block; on the others "
        f"{normwise(got[~split], hR[~split]) if (~split).any() else float('nan'):.3e}")


def test_stack_small():
    w = Workload("stack-small", 21, T=96, d=256, d_ff=512, blocks=4)
    from sparse_mixture_experts_31_amd.inputs import make_stack
    log(f"case {w.name}")
    h0, blocks = make_stack(w, DEV, 0)
    _stack_check(w, blocks, h0, np.arange(w.T))


@pytest.mark.parametrize("T", [32, 12, 8, 3])
def test_stack_decode_sized(T):
    """Decoder blocks at decode sizes run on the weight-streaming kernels,
    where GEMM1 groups the assignments itself and (from four rows per
    expert on, T = 32 here) GEMM2 forms h + y in place; T = 12 keeps the
    pass that sums split tiles and combines; T = 8 and 3 run the column
    kernels (eight and four token rows per expert), whose GEMM2 forms h + y
    itself."""
    from sparse_mixture_experts_31_amd.inputs import make_stack
    w = Workload(f"stack-decode-{T}", 42, T=T, d=1024, d_ff=2048, blocks=3)
    assert moe.moe_expert_ffn_kernels(T, w.d, w.d_ff, w.E, w.k, torch.bfloat16) == \
        "stream_gemm_kernel"
    log(f"case {w.name}")
    h0, blocks = make_stack(w, DEV, 0)
    _stack_check(w, blocks, h0, np.arange(w.T))


# ------------------------------------------------------------------ full sizes


def _check_grouping_valid(idx, P, E):
    """Properties that define the stable grouping of any routing `idx`."""
    T, k = idx.shape
    flat = idx.reshape(-1)
    counts, offsets = to_np(P["counts"]), to_np(P["offsets"])
    row_of, token_of = to_np(P["row_of"]).reshape(-1), to_np(P["token_of"])
    assert (counts == np.bincount(flat, minlength=E)).all()
    assert (offsets == np.concatenate([[0], np.cumsum(counts)])).all()
    assert (token_of[row_of] == np.arange(T * k) // k).all()
    assert (np.sort(row_of) == np.arange(T * k)).all()
    for e in range(E):
        blk = np.nonzero(flat == e)[0]
        assert (row_of[blk] == np.arange(offsets[e], offsets[e + 1])).all()


def _sample_rows(T, ref_idx, n, seed):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(T, n, replace=False).tolist()) | {0, T - 1}
    for e in np.unique(ref_idx):   # at least one token per expert in use
        rows.add(int(np.nonzero((ref_idx == e).any(1))[0][0]))
    return np.array(sorted(rows))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["decode", "prefill", "skewed"])
def test_full_size_layer(name):
    """The full workloads: routing and grouping of every token; y of every
    token at decode and prefill, and at the skewed workload (16384 tokens) of
    1024 seeded tokens plus every token the oracle finds within 1e-6 of a
    routing tie."""
    w = WORKLOADS[name]
    L = _case(w)
    ref = oracle.route(L["x"], L["Wg"], w.k)
    idx, gw = moe.moe_route(L["x"], L["Wg"], w.k)
    torch.cuda.synchronize()
    same, _, _ = check_routing(to_np(idx), to_np(gw), ref)
    P = moe.moe_permute(L["x"], idx, w.E)
    torch.cuda.synchronize()
    if same.all():
        want = oracle.permute(ref["idx"], w.E)
        for key in ("counts", "offsets", "row_of", "token_of"):
            np.testing.assert_array_equal(to_np(P[key]).reshape(want[key].shape), want[key], key)
    else:
        # near-tie tokens routed differently: the grouping of the GPU's own
        # choice must still be the valid stable one
        _check_grouping_valid(to_np(idx), P, w.E)
    counts = to_np(P["counts"])
    log(f"  counts {counts.tolist()}; experts 0 and 1 hold "
        f"{counts[:2].sum() / counts.sum():.1%} of the assignments")
    if name == "skewed":
        assert 0.40 <= counts[:2].sum() / counts.sum() <= 0.60
        near = np.nonzero(np.minimum(ref["gap_set"], ref["gap_order"]) < NEAR_TIE)[0]
        rows = np.union1d(_sample_rows(w.T, ref["idx"], 1024, 1), near)
    else:
        rows = np.arange(w.T)
    log(f"  y compared on {len(rows)} of {w.T} tokens")
    _forward_and_check(w, L, rows=rows)


# ------------------------------------------- kernel-family thresholds, full shape

@pytest.fixture(scope="module")
def prefill_layer():
    w = WORKLOADS["prefill"]
    return w, _case(w)


MIXED = "grouped_gemm_kernel (128 x 64 tiles) + wide_gemm_kernel (128-row token tiles) (W2)"


@pytest.mark.parametrize("T,family", [
    (107, "stream_gemm_kernel"),                     # 26 rows per expert on average
    (108, MIXED),                                    # 27
    (195, MIXED),                                    # 48
    (196, "wide_gemm_kernel (128-row token tiles)"),  # 49
    (400, "wide_gemm_kernel (128-row token tiles)"),  # 100
    (401, "wide_gemm_kernel (256-row token tiles)"),  # 100.25
])
def test_kernel_family_thresholds_at_the_mixtral_shape(prefill_layer, T, family):
    """The layer on the full Mixtral shape at the batch sizes where the
    library switches expert kernels (by the average rows per expert, T k /
    E), on both sides of every switch: each side must match the oracle."""
    w0, L0 = prefill_layer
    w = w0.with_(name=f"threshold-T{T}", T=T)
    assert moe.moe_expert_ffn_kernels(T, w.d, w.d_ff, w.E, w.k, torch.bfloat16) == family
    L = dict(L0, x=L0["x"][:T].contiguous())
    rows = np.union1d(np.random.default_rng(T).choice(T, 40, replace=False), [0, T - 1])
    _forward_and_check(w, L, rows=rows)


# ------------------------------------------------------ decode sweep T = 1..16

@pytest.fixture(scope="module")
def decode16():
    """The decode workload's layer at T = 16; smaller batches take its first
    T token rows (the weights do not depend on T)."""
    w = WORKLOADS["decode"].with_(name="decode-sweep", T=16)
    return w, _case(w)


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 8, 12, 15, 16])
def test_decode_sweep(decode16, T):
    """Mixtral-shaped decode batches of 1..16 tokens: each token takes exactly
    two experts, so T tokens touch at most min(8, 2T) of them (expected
    8 (1 - 0.75^T) for independent uniform choices); empty experts must be
    skipped, and every token must match the oracle."""
    w0, L0 = decode16
    w = w0.with_(name=f"decode-T{T}", T=T)
    L = dict(L0, x=L0["x"][:T].contiguous())
    y, ref = _forward_and_check(w, L)
    counts = np.bincount(ref["idx"].ravel(), minlength=w.E)
    log(f"  T={T}: {int((counts > 0).sum())} experts active, counts {counts.tolist()}")
    assert (counts > 0).sum() <= min(w.E, 2 * T)


@pytest.fixture(scope="module")
def decode64():
    """The decode workload's layer at T = 64 (smaller batches take its first
    T token rows)."""
    w = WORKLOADS["decode"].with_(name="decode-64", T=64)
    return w, _case(w)


@pytest.mark.parametrize("T", [9, 17, 32, 33, 64])
def test_decode_batches_around_the_kernel_switches(decode64, T):
    """Mixtral-shaped batches on both sides of the switches: nine to 32
    tokens run GEMM1 on the tile kernel and GEMM2 on the column kernel (16
    token rows per chunk); from 33 on both GEMMs run on the tile kernel,
    whose GEMM2 forms y in its tail.  Every token must match the oracle."""
    w0, L0 = decode64
    w = w0.with_(name=f"decode-T{T}", T=T)
    L = dict(L0, x=L0["x"][:T].contiguous())
    want = "stream_gemm_kernel + stream_cols_kernel (W2)" if T <= 32 else "stream_gemm_kernel"
    assert moe.moe_forward_kernels(T, w.d, w.d_ff, w.E, w.k, torch.bfloat16) == want
    y, ref = _forward_and_check(w, L)
    counts = np.bincount(ref["idx"].ravel(), minlength=w.E)
    log(f"  T={T}: rows per expert {counts.tolist()}")


def test_weight_stream_at_every_small_batch():
    """Every batch of 1..48 tokens (2..96 assignments over 8 experts) on a
    small shape the weight-streaming kernels take: the even K split, whole
    tiles, and the rule between them meet every token count; each layer
    against the oracle on all its tokens."""
    w0 = Workload("stream-every-T", 33, T=48, d=512, d_ff=1536)
    L0 = _case(w0)
    for T in range(1, 49):
        w = w0.with_(name=f"stream-T{T}", T=T)
        assert moe.moe_expert_ffn_kernels(T, w.d, w.d_ff, w.E, w.k,
                                          torch.bfloat16) == "stream_gemm_kernel"
        _forward_and_check(w, dict(L0, x=L0["x"][:T].contiguous()))


def test_decode_single_token_reads_only_its_two_experts(decode16):
    """T = 1: NaN in the six experts the token does not choose must leave y
    bit for bit unchanged (their weights are never read)."""
    w0, L0 = decode16
    w = w0.with_(name="decode-T1", T=1)
    x = L0["x"][:1].contiguous()
    y = moe.moe_forward(x, L0["Wg"], L0["W1"], L0["W3"], L0["W2"], w.k)
    idx, _ = moe.moe_route(x, L0["Wg"], w.k)
    torch.cuda.synchronize()
    chosen = set(to_np(idx).ravel().tolist())
    assert len(chosen) == 2
    P = {n: L0[n].clone() for n in ("W1", "W3", "W2")}
    for e in range(w.E):
        if e not in chosen:
            for n in P:
                P[n][e] = float("nan")
    y_nan = moe.moe_forward(x, L0["Wg"], P["W1"], P["W3"], P["W2"], w.k)
    torch.cuda.synchronize()
    assert torch.equal(y_nan, y)


@pytest.mark.timeout(900)
def test_full_size_stack():
    from sparse_mixture_experts_31_amd.inputs import make_stack
    w = WORKLOADS["stack"]
    log(f"case {w.name}: generating {w.blocks} blocks")
    h0, blocks = make_stack(w, DEV, 0)
    rng = np.random.default_rng(7)
    sample = np.union1d(rng.choice(w.T, 62, replace=False), [0, w.T - 1])
    _stack_check(w, blocks, h0, sample)


# ------------------------------------------------ load statistics of the router

@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "skewed"])
def test_route_balance_matches_oracle(name):
    """f (share routed per expert), P (mean full-softmax probability) and
    Laux = E sum f P against the oracle; the routing outputs are those of
    moe_route bit for bit, and two runs give the same bits."""
    w = WORKLOADS[name]
    L = _case(w)
    idx, gw, f, P, laux = moe.moe_route_balance(L["x"], L["Wg"], w.k)
    idx0, gw0 = moe.moe_route(L["x"], L["Wg"], w.k)
    _, _, f2, P2, laux2 = moe.moe_route_balance(L["x"], L["Wg"], w.k)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx0) and torch.equal(gw, gw0)
    assert torch.equal(f, f2) and torch.equal(P, P2) and torch.equal(laux, laux2)
    ref = oracle.route(L["x"], L["Wg"], w.k)
    check_routing(to_np(idx), to_np(gw), ref)
    # f from the GPU's own choices is exact (an integer count over T*k)
    counts = np.bincount(to_np(idx).ravel(), minlength=w.E)
    np.testing.assert_array_equal(to_np(f), (counts / (w.T * w.k)).astype(np.float32))
    b = oracle.balance(ref["logits"], ref["idx"])
    # near-tie tokens may route differently: f then differs by those tokens
    n_diff = int((to_np(idx) != ref["idx"]).any(1).sum())
    assert np.abs(to_np(f).astype(np.float64) - b["f"]).max() <= (n_diff + 0.5) / (w.T * w.k)
    # P from fp32-rounded scores, summed in fp64 and rounded once to fp32
    np.testing.assert_allclose(to_np(P), b["P"], rtol=2e-6, atol=1e-8)
    assert abs(float(laux[0]) - b["laux"]) <= 2e-6 * b["laux"] + 2.0 * n_diff / (w.T * w.k)
    log(f"  Laux {float(laux[0]):.6f} (oracle {b['laux']:.6f}), f {np.round(to_np(f), 4).tolist()}")


def test_route_balance_rejects_empty_batch():
    x = torch.empty((0, 128), dtype=torch.bfloat16, device=DEV)
    Wg = torch.zeros((8, 128), dtype=torch.float32, device=DEV)
    with pytest.raises(moe.MoeError):
        moe.moe_route_balance(x, Wg, 2, ws=torch.empty(256, dtype=torch.uint8, device=DEV))


# ------------------------------------------------------ random shapes

def _random_workload(seed):
    """A seeded random layer shape within the library's limits: any expert
    count and k, d and d_ff multiples of 64, a quarter fp32; odd seeds take
    shapes the weight-streaming kernels accept (d, d_ff multiples of 512,
    small batches)."""
    rng = np.random.default_rng(1000 + seed)
    E = int(rng.choice([1, 2, 3, 4, 8, 8, 13, 16, 64]))
    k = int(rng.integers(1, min(E, 8) + 1))
    if seed % 2:
        d = int(rng.choice([512, 1024, 1536]))
        d_ff = int(rng.choice([512, 1024, 1536, 2048]))
        T = int(rng.choice([1, 3, 8, 24, 48, 96]))
    else:
        d = int(rng.integers(1, 17)) * 64
        d_ff = int(rng.integers(1, 33)) * 64
        T = int(rng.choice([2, 17, 64, 150, 400, 1100]))
    dt = "f32" if rng.random() < 0.25 else "bf16"
    return Workload(f"random-{seed}", 200 + seed, T=T, d=d, d_ff=d_ff, E=E, k=k, dtype=dt)


@pytest.mark.parametrize("seed", range(40))
def test_random_shapes(seed):
    """moe_forward on seeded random shapes (every kernel family and their
    thresholds) against the oracle on up to 48 sampled tokens."""
    w = _random_workload(seed)
    L = _case(w)
    rows = None if w.T <= 48 else np.sort(np.random.default_rng(seed).choice(w.T, 48, replace=False))
    _forward_and_check(w, L, rows=rows)


@pytest.mark.parametrize("seed", range(20))
def test_random_tile_stream_shapes(seed):
    """9 to 32 tokens on weight-stream shapes (d, d_ff multiples of 512): the
    layer's GEMM1 on the tile kernel, which sums the pieces of the tiles it
    splits itself (the last workgroup to count a tile's piece), and GEMM2 on
    the column kernel; random E and k, every token checked against the
    oracle."""
    rng = np.random.default_rng(5000 + seed)
    E = int(rng.choice([2, 4, 8, 8, 16, 64]))
    k = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.integers(9, 33))
    k = min(k, 64 // T)
    w = Workload(f"tile-stream-{seed}", 300 + seed, T=T, d=int(rng.choice([512, 1024, 2048])),
                 d_ff=int(rng.choice([512, 1024, 1536, 2048, 3584])), E=E, k=k)
    L = _case(w)
    _forward_and_check(w, L)
