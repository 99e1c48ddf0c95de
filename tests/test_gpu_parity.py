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
from parity import (NEAR_TIE, TOL, bf16_rne, check_near_rounding_floor, check_routing, log,
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
    # 25-48 rows per expert: the grouped kernels with 128 x 64 tiles (bf16)
    Workload("grouped-bf16", 26, T=160, d=512, d_ff=1024),
    # degenerate routing: one expert (every gate is 1), and every token
    # taking all eight experts
    Workload("e1-k1", 27, T=50, d=256, d_ff=512, E=1, k=1),
    Workload("k-all", 28, T=40, d=256, d_ff=256, E=8, k=8),
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


def test_permute_empty_and_skewed_groups():
    T, E, k, d = 777, 8, 2, 128
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


@pytest.mark.parametrize("w", [
    Workload("forced", 20, T=200, d=256, d_ff=512),
    # decode-sized (T*k/E <= 24): the weight-streaming kernels, here with
    # three token tiles of 32 rows for each of the two experts
    Workload("forced-stream", 21, T=96, d=512, d_ff=1024),
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


def test_rmsnorm_matches_oracle_bit_for_bit():
    h = (torch.randn((333, 4096), device=DEV) * 3).to(torch.bfloat16)
    eps = float(np.float32(1e-5))
    out = moe.moe_rmsnorm(h, eps)
    torch.cuda.synchronize()
    want = oracle.rmsnorm_rows(to_np(h).astype(np.float64), eps, round_bf16=True)
    np.testing.assert_array_equal(to_np(out).astype(np.float64), want)


# ------------------------------------------------------------------ the stack


def _rms_bf16(h, eps):
    """Test-side rmsnorm + bf16 rounding (used only to size the state
    difference between the two trajectories, never as an expected value)."""
    h = np.asarray(h, np.float64)
    xn = h / np.sqrt((h * h).mean(axis=1, keepdims=True) + eps)
    m, e = np.frexp(xn)   # one rounding to 8 significant bits, ties to even
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def _gate_spread(Wg):
    """max over expert pairs of ||Wg_e - Wg_e'||_2: by Cauchy-Schwarz, an
    input change of norm D moves any score difference by at most this * D."""
    W = Wg.double().cpu().numpy()
    diff = W[:, None, :] - W[None, :, :]
    return float(np.sqrt((diff * diff).sum(-1)).max())


def _stack_check(w: Workload, blocks, h0, sample):
    """Run w.blocks block steps on the GPU against the oracle, free-running.

    Block 0: the normalised inputs are bit-identical on both sides, so all
    tokens' routing must match (fp32 near-ties excepted) and the block output
    must sit at the bf16 rounding floor of the exact step.

    Blocks 1..: the two trajectories differ by bf16 roundings, and the
    stacked residual blocks amplify such differences.  A routing difference
    is accepted only where the oracle's set gap lies within what the measured
    input difference can move a score difference (Cauchy-Schwarz); the token
    is then followed no further.  The end-to-end criterion is relative to the
    problem's own conditioning: the oracle is run twice, with the SwiGLU
    intermediate quantised to bf16 (R, the GPU's data path) and kept in fp64
    (S); both are valid arithmetic, and the GPU's distance to R may not exceed
    max(bf16 tolerance, 2 x the distance between S and R)."""
    eps = float(np.float32(w.eps))
    h = h0.clone()
    ws = moe.workspace(w.T, w.d, w.d_ff, w.E, w.k, h.dtype)
    sel = torch.from_numpy(np.asarray(sample)).long().to(DEV)
    idxs, h_in = [], []
    for b, B in enumerate(blocks):
        idx = torch.empty((w.T, w.k), dtype=torch.int32, device=DEV)
        gw = torch.empty((w.T, w.k), dtype=torch.float32, device=DEV)
        h_in.append(h[sel].clone())
        moe.moe_block_forward(h, B["Wg"], B["W1"], B["W3"], B["W2"], w.k, eps, topk_idx=idx,
                              topk_w=gw, ws=ws)
        idxs.append((idx, gw))
    torch.cuda.synchronize()
    # block 0 sees bit-identical normalised inputs on both sides: all tokens
    xn0 = oracle.rmsnorm_rows(to_np(h0).astype(np.float64), eps, round_bf16=True)
    xn0 = torch.from_numpy(xn0).float().to(torch.bfloat16)
    r0 = oracle.route(xn0, blocks[0]["Wg"], w.k)
    check_routing(to_np(idxs[0][0]), to_np(idxs[0][1]), r0)
    # free-running oracle on the sample, two quantisation choices
    hR = to_np(h0)[sample].astype(np.float64).copy()
    hS = hR.copy()
    diverged = np.zeros(len(sample), bool)
    worst_drift = 0.0
    for b, B in enumerate(blocks):
        spread = _gate_spread(B["Wg"])
        dx = np.linalg.norm(_rms_bf16(to_np(h_in[b]), eps) - _rms_bf16(hR, eps), axis=1)
        worst_drift = max(worst_drift, float(dx[~diverged].max(initial=0.0)))
        r = oracle.block_step(hR, B["Wg"], B["W1"], B["W3"], B["W2"], w.k, eps, round_mid=True)
        oracle.block_step(hS, B["Wg"], B["W1"], B["W3"], B["W2"], w.k, eps)
        if b == 0:
            got1 = to_np(h_in[1] if len(blocks) > 1 else h[sel])
            e1 = normwise(got1, hR)
            floor = normwise(bf16_rne(hR), hR)   # hR is already bf16: floor 0
            log(f"  block 0 output: normwise {e1:.3e} (exact step rounded: {floor:.1e})")
            assert e1 <= 1e-3
        gi = to_np(idxs[b][0])[sample]
        for n in range(len(sample)):
            if diverged[n]:
                continue
            if set(gi[n].tolist()) != set(r["idx"][n].tolist()):
                tol = NEAR_TIE + spread * dx[n]
                assert r["gap_set"][n] < tol, (b, sample[n], r["gap_set"][n], tol)
                log(f"  block {b} token {sample[n]}: routing split at set gap "
                    f"{r['gap_set'][n]:.2e} (bound {tol:.2e})")
                diverged[n] = True
    log(f"  largest normalised-input drift on the oracle's path: {worst_drift:.3e}")
    got = to_np(h)[sample]
    e_gpu = normwise(got, hR)
    e_ref = normwise(hS, hR)
    keep = ~diverged
    e_path = normwise(got[keep], hR[keep]) if keep.any() else float("nan")
    log(f"  stack: {w.blocks} blocks; GPU vs oracle {e_gpu:.3e}, oracle vs its fp64-"
        f"intermediate variant {e_ref:.3e}; {keep.sum()}/{len(sample)} tokens on the "
        f"oracle's routing path (normwise {e_path:.3e})")
    assert e_gpu <= max(TOL["bf16"], 2.0 * e_ref)


def test_stack_small():
    w = Workload("stack-small", 21, T=96, d=256, d_ff=512, blocks=4)
    from sparse_mixture_experts_31_amd.inputs import make_stack
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


@pytest.mark.parametrize("name", ["decode", "prefill", "skewed"])
def test_full_size_layer(name):
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
    log(f"  counts {to_np(P['counts']).tolist()}")
    rows = np.arange(w.T) if w.T <= 64 else _sample_rows(w.T, ref["idx"], 40, 1)
    _forward_and_check(w, L, rows=rows)


# ------------------------------------------------------ decode sweep T = 1..16

@pytest.fixture(scope="module")
def decode16():
    """The decode workload's layer at T = 16; smaller batches take its first
    T token rows (the weights do not depend on T)."""
    w = WORKLOADS["decode"].with_(name="decode-sweep", T=16)
    return w, _case(w)


@pytest.mark.parametrize("T", [1, 2, 4, 8, 16])
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
    sample = np.array([0, 1, 100, 333, 517, 777, 901, 1024, 1300, 1500, 1650, 1800, 1901, 2000,
                       2046, 2047])
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


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes(seed):
    """moe_forward on seeded random shapes (every kernel family and their
    thresholds) against the oracle on up to 48 sampled tokens."""
    w = _random_workload(seed)
    L = _case(w)
    rows = None if w.T <= 48 else np.sort(np.random.default_rng(seed).choice(w.T, 48, replace=False))
    _forward_and_check(w, L, rows=rows)
