#!/usr/bin/env python
"""Throughput of the Mixtral sparse-MoE layer on one MI355X.

A step is one whole layer (router, dispatch, the two expert GEMMs, combine)
over one batch of the workload's synthetic tokens, inputs resident in HBM.
For the stack workload a step is all of its h + moe(rms_norm(h)) blocks.

Prints one JSON line.  `roofline` covers the dominant kernel (the W1/W3
GEMM with the SwiGLU epilogue), timed live with HIP events recorded by the
library on the launch stream around that kernel in every timed step.
`cpu_baseline` times the fp64 CPU oracle on a bounded sample of the same
workload (rank 0, one GPU only).

    python bench.py [--steps K] [--warmup W] [--workload decode|prefill|skewed|stack|tiny]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s (d4096,ff14336,E8,k2); %MFMA peak prefill, %HBM BW decode"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 (matrix and vector)


class HipEvents:
    """hipEvent_t handles from the HIP runtime (the library records them)."""

    # Timing-only events: no system-scope fence (cache writeback and
    # invalidate) when they complete, so recording them inside the timed
    # loop costs the kernels around them nothing measurable.
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                     ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self) -> int:
        e = ctypes.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        return e.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a),
                                          ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def destroy(self, e: int):
        self.hip.hipEventDestroy(ctypes.c_void_p(e))

    def record(self, e: int, stream):
        """Record e on a torch stream (the stream the timed work runs on)."""
        rc = self.hip.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")


def gemm1_work(w, counts):
    """Algorithmic work of the W1/W3 + SwiGLU GEMM for one launch.

    bytes: W1 and W3 rows of every expert that received tokens (2*d_ff*d
    elements each), the A = T*k gathered token rows (d elements each) and
    the A SwiGLU rows written (d_ff elements each).
    flops: 2 multiply-adds' worth per weight per assignment: 2 * A * d * 2*d_ff.
    """
    es = 4 if w.dtype == "f32" else 2
    A = w.T * w.k
    n_active = int((counts > 0).sum())
    nbytes = n_active * 2 * w.d_ff * w.d * es + A * w.d * es + A * w.d_ff * es
    flops = 2 * A * w.d * 2 * w.d_ff
    return nbytes, flops, n_active


def layer_work(w, n_active):
    """Whole-layer algorithmic work: FLOPs = T(2*k*3*d*d_ff + 2*d*E); bytes =
    active experts' weights + x read + y written + the fp32 gate matrix."""
    es = 4 if w.dtype == "f32" else 2
    flops = w.T * (2 * w.k * 3 * w.d * w.d_ff + 2 * w.d * w.E)
    nbytes = n_active * 3 * w.d * w.d_ff * es + 2 * w.T * w.d * es + w.E * w.d * 4
    return nbytes, flops


def measured_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel, from the committed
    rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE scaled by a plain
    copy of known size), or None when there is none or the kernel source has
    changed since the counters were taken."""
    import glob
    import hashlib

    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as f:
            for line in f:
                if not line.startswith("bench-traffic "):
                    continue
                rec = json.loads(line[len("bench-traffic "):])
                if rec.get("workload") != workload:
                    continue
                src = os.path.join(ROOT, rec["source"])
                if not os.path.exists(src):
                    return None
                with open(src, "rb") as s:
                    if hashlib.sha1(s.read()).hexdigest() != rec["source_sha1"]:
                        return None
                return int(rec["traffic_bytes"])
    return None


def cpu_baseline(w, L, budget_tokens, budget_s=10.0):
    """The oracle, as it stands, on a bounded token sample of the same layer:
    chunks of `budget_tokens` consecutive tokens until about `budget_s`
    seconds of wall time have passed (tokens are independent, so tokens per
    second over the sample is the layer's rate)."""
    import numpy as np

    import oracle

    host = {n: L[n].cpu() for n in ("x", "Wg", "W1", "W3", "W2")}
    threads = oracle.default_threads()
    chunk = min(w.T, budget_tokens)
    done, start, elapsed = 0, 0, 0.0
    while elapsed < budget_s and done < 64 * w.T:
        rows = (np.arange(chunk, dtype=np.int64) + start) % w.T
        t0 = time.perf_counter()
        oracle.moe_rows(host["x"], host["Wg"], host["W1"], host["W3"], host["W2"], w.k,
                        rows=rows, nthreads=threads)
        elapsed += time.perf_counter() - t0
        done += chunk
        start = (start + chunk) % w.T
    return {"value": round(done / elapsed, 3), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done} tokens of the {w.name} workload (T={w.T}) in chunks of {chunk}, "
                      f"{elapsed:.1f} s wall on {threads} threads"}


def decode_sweep(w, L, moe, np, torch, stream, steps):
    """The decode layer at T = 1, 2, 4, 8, 16 tokens (the first T rows of the
    batch, same weights): time per layer, the experts the batch activates and
    the HBM rate of reading their weights.  Only active experts are read, so
    the bytes grow with T until all eight are in use."""
    res = {}
    ev = torch.cuda.Event
    for T in (1, 2, 4, 8, 16):
        x = L["x"][:T].contiguous()
        ws = moe.workspace(T, w.d, w.d_ff, w.E, w.k, x.dtype, x.device)
        y = torch.empty_like(x)

        def run():
            moe.moe_forward(x, L["Wg"], L["W1"], L["W3"], L["W2"], w.k, y=y, ws=ws,
                            stream=stream)

        for _ in range(3):
            run()
        a, b = ev(enable_timing=True), ev(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            run()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        idx, _ = moe.moe_route(x, L["Wg"], w.k)
        n_active = int((np.bincount(idx.cpu().numpy().reshape(-1), minlength=w.E) > 0).sum())
        wbytes = n_active * 3 * w.d * w.d_ff * 2
        res[str(T)] = {"ms": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
                       "active_experts": n_active,
                       "weight_GBps": round(wbytes / (ms * 1e-3) / 1e9, 1),
                       "hbm_frac": round(wbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        print(f"[bench] decode sweep T={T}: {ms:.3f} ms, {n_active} experts", file=sys.stderr,
              flush=True)
    return res


def routing_summary(w, L, moe, np, torch):
    """What the batch's routing looks like, from the GPU router's own fp32
    scores: experts in use, the share of assignments on experts 0 and 1 (the
    skewed workload aims at about half), and the tokens whose k-th and
    (k+1)-th scores (set) or kept scores (order) are closer than 1e-6 --
    the near ties that the exact routing comparison exempts."""
    T, E, k = w.T, w.E, w.k
    logits = torch.empty((T, E), dtype=torch.float32, device=L["x"].device)
    idx, _ = moe.moe_route(L["x"], L["Wg"], k, logits=logits)
    torch.cuda.synchronize()
    lg = np.sort(logits.cpu().numpy().astype(np.float64), axis=1)[:, ::-1]
    counts = np.bincount(idx.cpu().numpy().reshape(-1), minlength=E)
    gap_set = lg[:, k - 1] - lg[:, k] if k < E else np.full(T, np.inf)
    gap_order = (np.diff(-lg[:, :k], axis=1).min(axis=1) if k > 1 else np.full(T, np.inf))
    return counts, {"active_experts": int((counts > 0).sum()),
                    "experts01_share": round(float(counts[:2].sum() / counts.sum()), 4),
                    "near_ties_set": int((gap_set < 1e-6).sum()),
                    "near_ties_order": int((gap_order < 1e-6).sum())}


def gemm1_roofline(w, counts, gemm1_ms, kernel):
    """The dominant kernel (the W1/W3 + SwiGLU GEMM) against its roofline:
    HBM when its arithmetic intensity on the weights (2 flop per weight
    element per row of the expert) is below the chip's ridge, else MFMA."""
    g_bytes, g_flops, _ = gemm1_work(w, counts)
    es = 4 if w.dtype == "f32" else 2
    peak_fl = PEAK_F32_TFLOPS if w.dtype == "f32" else PEAK_BF16_TFLOPS
    per_expert = (w.T * w.k) // w.E
    if 2 * per_expert / es < peak_fl * 1e12 / (PEAK_HBM_GBS * 1e9):
        achieved = g_bytes / (gemm1_ms * 1e-3) / 1e9
        r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
             "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        achieved = g_flops / (gemm1_ms * 1e-3) / 1e12
        r = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak_fl,
             "unit": "TFLOP/s", "frac": round(achieved / peak_fl, 4)}
    r["traffic"] = measured_traffic(w.name)
    # the family of GEMM1 (where the two GEMMs differ, the label names GEMM1's first)
    r["kernel"] = kernel.split(" + ")[0] + " GEMM1 (W1/W3 + silu*v)"
    r["kernel_ms"] = round(gemm1_ms, 4)
    r["alg_bytes"] = g_bytes
    r["alg_flops"] = g_flops
    return r


def layer_roofline(w, n_active, ms_per_step):
    l_bytes, l_flops = layer_work(w, n_active)
    nblk = max(1, w.blocks)
    step_s = ms_per_step * 1e-3
    peak_fl = PEAK_F32_TFLOPS if w.dtype == "f32" else PEAK_BF16_TFLOPS
    return {"alg_bytes": l_bytes * nblk, "alg_flops": l_flops * nblk,
            "hbm_frac": round(l_bytes * nblk / step_s / 1e9 / PEAK_HBM_GBS, 4),
            "mfma_frac": round(l_flops * nblk / step_s / 1e12 / peak_fl, 4),
            "active_experts": n_active}


def time_layer(w, L, moe, np, torch, ev, stream, steps, warmup, blocks=None):
    """W untimed layers, then K timed ones between two synchronisations.
    Returns (ms per step, mean GEMM1 ms from the library's events around
    that kernel in every timed step, stage breakdown in us or None)."""
    dev = L["x"].device
    ws = moe.workspace(w.T, w.d, w.d_ff, w.E, w.k, L["x"].dtype, dev)
    y = torch.empty_like(L["x"])
    eps = float(np.float32(w.eps))

    def step(marks):
        if blocks is None:
            moe.moe_forward_profiled(L["x"], L["Wg"], L["W1"], L["W3"], L["W2"], w.k, marks,
                                     y=y, ws=ws, stream=stream)
        else:
            h = y
            h.copy_(L["x"])
            for B in blocks:
                moe.moe_block_forward(h, B["Wg"], B["W1"], B["W3"], B["W2"], w.k, eps, ws=ws,
                                      stream=stream)

    none6 = [None] * 6
    for _ in range(warmup):
        step(none6)
    torch.cuda.synchronize()
    print(f"[bench] {w.name}: warmup done", file=sys.stderr, flush=True)

    pairs = [(ev.create(), ev.create()) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step([None, None, pairs[i][0], pairs[i][1], None, None] if blocks is None else none6)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps
    print(f"[bench] {w.name}: timed {steps} steps, {ms_per_step:.3f} ms/step", file=sys.stderr,
          flush=True)
    gemm1_ms = None
    if blocks is None:
        gemm1_ms = float(np.mean([ev.elapsed_ms(a, b) for a, b in pairs]))
    for a, b in pairs:
        ev.destroy(a)
        ev.destroy(b)

    # Where a layer's time goes: a few more layers, outside the timed region,
    # with the library's events around every stage (recording all six costs
    # the layer about 10 us, so the timed steps carry only GEMM1's pair).
    breakdown = None
    if blocks is None:
        marks = [[ev.create() for _ in range(6)] for _ in range(10)]
        for _ in range(10):   # back to the steady state after the pause above
            step(none6)
        for m in marks:
            step(m)
        torch.cuda.synchronize()
        names = ["router", "dispatch", "gemm1", "gemm2", "combine"]
        breakdown = {n: round(float(np.mean([ev.elapsed_ms(m[i], m[i + 1]) for m in marks])) * 1e3, 1)
                     for i, n in enumerate(names)}
        for m in marks:
            for e in m:
                ev.destroy(e)
    return ms_per_step, gemm1_ms, breakdown


def ep_shard(Ms, steps, warmup, dev, seed, moe, np, torch, ev, stream):
    """One GPU's share under expert parallelism (one expert per GPU): the
    expert GEMMs of a single Mixtral-sized expert (E = 1) on M received rows,
    timed with HIP events around every call of moe_expert_ffn."""
    from sparse_mixture_experts_31_amd.inputs import Workload, make_layer
    res = {}
    for M in Ms:
        w = Workload("ep-shard", 5, T=M, d=4096, d_ff=14336, E=1, k=1)
        L = make_layer(w, dev, seed)
        offsets = torch.tensor([0, M], dtype=torch.int32, device=dev)
        ws = moe.workspace(M, w.d, w.d_ff, 1, 1, L["x"].dtype, dev)
        out = torch.empty_like(L["x"])

        def call():
            moe.moe_expert_ffn(L["x"], offsets, L["W1"], L["W3"], L["W2"], M, 1, out_perm=out,
                               ws=ws, stream=stream)

        for _ in range(warmup):
            call()
        pairs = [(ev.create(), ev.create()) for _ in range(steps)]
        for a, b in pairs:
            ev.record(a, stream)
            call()
            ev.record(b, stream)
        torch.cuda.synchronize()
        ms = float(np.mean([ev.elapsed_ms(a, b) for a, b in pairs]))
        for a, b in pairs:
            ev.destroy(a)
            ev.destroy(b)
        flops = 2.0 * M * 3 * w.d * w.d_ff
        nbytes = 3.0 * w.d * w.d_ff * 2 + 2.0 * M * w.d * 2
        res[str(M)] = {"kernel": moe.moe_expert_ffn_kernels(M, w.d, w.d_ff, 1, 1, w.torch_dtype),
                       "ms": round(ms, 4),
                       "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                       "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                       "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                       "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        del L, ws, out
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the first few dozen layers of a fresh process run slower (decode: 0.52 ms
    # for the first ten, 0.45 from about the thirtieth on), so the default
    # warm-up covers them
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="decode",
                    choices=["tiny", "decode", "prefill", "skewed", "stack"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode-sweep", action="store_true",
                    help="skip the T = 1..16 small-batch lines of the decode workload")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill (T = 4096) layer the decode run also times")
    ap.add_argument("--cpu-tokens", type=int, default=None,
                    help="oracle sample size (default sized to ~10-30 s)")
    ap.add_argument("--ep-shard", default=None, metavar="M1,M2,...",
                    help="only time one GPU's share under expert parallelism: the expert "
                         "GEMMs of one Mixtral-sized expert on M rows, for each M, and exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device 3 times (a plain copy of known "
                         "size, to scale the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs the layer on one GPU only; --gpus {args.gpus} / WORLD_SIZE {world} "
              "is not supported (the layer has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from sparse_mixture_experts_31_amd import moe
    from sparse_mixture_experts_31_amd.inputs import WORKLOADS, make_layer, make_stack

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)
        return
    if args.ep_shard:
        ev = HipEvents()
        Ms = [int(m) for m in args.ep_shard.split(",")]
        res = ep_shard(Ms, args.steps, min(args.warmup, 20), dev, args.seed, moe, np, torch, ev,
                       torch.cuda.current_stream())
        print(json.dumps({"ep_shard": res, "d": 4096, "d_ff": 14336, "dtype": "bf16",
                          "steps": args.steps, "data": "synthetic"}), flush=True)
        return
    w = WORKLOADS[args.workload]
    print(f"[bench] workload {w.name}: T={w.T} d={w.d} d_ff={w.d_ff} E={w.E} k={w.k} "
          f"{w.dtype} blocks={w.blocks}", file=sys.stderr, flush=True)
    ev = HipEvents()
    stream = torch.cuda.current_stream()

    if w.blocks > 1:
        h0, blocks = make_stack(w, dev, args.seed)
        L = dict(x=h0, **blocks[0])
    else:
        L = make_layer(w, dev, args.seed)
        blocks = None
    torch.cuda.synchronize()
    print("[bench] inputs ready", file=sys.stderr, flush=True)

    ms_per_step, gemm1_ms, breakdown = time_layer(w, L, moe, np, torch, ev, stream, args.steps,
                                                  args.warmup, blocks)
    tokens_per_s = w.T / (ms_per_step * 1e-3)

    counts, routing = routing_summary(w, L, moe, np, torch)
    kernel = moe.moe_forward_kernels(w.T, w.d, w.d_ff, w.E, w.k, w.torch_dtype)
    roofline = gemm1_roofline(w, counts, gemm1_ms, kernel) if blocks is None else None
    layer = layer_roofline(w, routing["active_experts"], ms_per_step)

    sweep = None
    if w.name == "decode" and not args.no_decode_sweep:
        sweep = decode_sweep(w, L, moe, np, torch, stream, args.steps)

    # The compute-bound half of the metric: the prefill layer (T = 4096) timed
    # the same way, reported beside the decode headline.
    prefill = None
    if w.name == "decode" and not args.no_prefill:
        wp = WORKLOADS["prefill"]
        Lp = make_layer(wp, dev, args.seed)
        torch.cuda.synchronize()
        p_ms, p_g1, p_stages = time_layer(wp, Lp, moe, np, torch, ev, stream, args.steps,
                                          args.warmup)
        p_counts, p_routing = routing_summary(wp, Lp, moe, np, torch)
        p_kernel = moe.moe_forward_kernels(wp.T, wp.d, wp.d_ff, wp.E, wp.k, wp.torch_dtype)
        prefill = {"config": {"workload": wp.name, "T": wp.T, "d": wp.d, "d_ff": wp.d_ff,
                              "E": wp.E, "k": wp.k, "act_dtype": wp.dtype},
                   "ms_per_step": round(p_ms, 4),
                   "tokens_per_s": round(wp.T / (p_ms * 1e-3), 1),
                   "roofline": gemm1_roofline(wp, p_counts, p_g1, p_kernel),
                   "layer_roofline": layer_roofline(wp, p_routing["active_experts"], p_ms),
                   "stage_us": p_stages, "routing": p_routing}
        del Lp
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline and blocks is None:
        budget = args.cpu_tokens or max(8, min(w.T, 48))
        print(f"[bench] oracle baseline on {budget} tokens", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, L, budget)

    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32" if w.dtype == "f32" else "bf16", "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "d_ff": w.d_ff, "E": w.E, "k": w.k,
                   "blocks": w.blocks, "act_dtype": w.dtype, "router_dtype": "f32",
                   "seed": args.seed},
        "roofline": roofline, "cpu_baseline": cpu, "layer_roofline": layer, "routing": routing,
    }
    if breakdown is not None:
        out["stage_us"] = breakdown
    if sweep is not None:
        out["decode_sweep"] = sweep
    if prefill is not None:
        out["prefill"] = prefill
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
