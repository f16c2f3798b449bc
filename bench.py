#!/usr/bin/env python3
"""Benchmark of the SERQ linear layer on one MI355X.

A step is one pass of the whole runtime path -- per-token activation
quantization, the packed 4-bit main GEMM with the fused rank-r residual, the
dequant epilogue -- over one batch of synthetic input already resident in HBM:
LLaMA-2-7B attention-projection shape, 2048 tokens, 4096 -> 4096, r = 128,
INT4 (W4A4).  Prints one JSON line with

  value        serq_linear throughput in TOPS: 2*M*d_out*(d_in + r) / step time
  roofline     the fused GEMM kernel's algorithmic ops / its average launch time
               (HIP events on the launch stream) against the int8 MFMA peak
  residual     the GEMM's time at rank r versus the same kernel at rank 0
  cpu_baseline the CPU oracle on a bounded sample of the same workload

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from rank_error_compensated_amd import binding as B  # noqa: E402
from rank_error_compensated_amd import workloads as WL  # noqa: E402

PEAK = {  # MI355X published dense peaks
    "int4": ("mfma", 5000.0, "TFLOP/s"),    # int8 MFMA, 5.0 POP/s (4-bit codes run on it)
    "w4a8": ("mfma", 5000.0, "TFLOP/s"),
    "mxfp4": ("mfma", 10100.0, "TFLOP/s"),  # FP4 MFMA
}
HBM_PEAK_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "rank_error_compensated_amd", "csrc", "serq_kernels.hip")

WORKLOADS = {
    "attn_proj_int4": lambda: WL.attn_proj_int4()[0],
}


def kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profiles(name: str):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, each scaled by a copy of
    known size) from the committed rocprofv3 counter summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_src_sha256_16") != kernel_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def time_launches(fn, n: int, torch) -> float:
    """Average duration (s) of fn() over n back-to-back launches, by HIP
    events recorded on torch's current stream (the stream the library
    launches on)."""
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(n):
        fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) * 1e-3 / n


def cpu_baseline(c, r, fmt, budget_s: float = 10.0) -> dict:
    """The CPU oracle, as it stands, on 128-token blocks of the same layer
    (cycling through its 2048 tokens) until the time budget is spent:
    per-token quantization + exact integer products + epilogue.  Offline
    preparation is not timed."""
    from oracle import serq_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    p = O.prepare(c.W, c.X_cal, r, fmt)
    Xh = O.flatten_acts(c.X, p["s"], p["perm"])
    blk, done, t0 = 128, 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        lo = done % c.M
        O.serq_linear(Xh[lo:lo + blk], p)
        done += blk
    dt = time.perf_counter() - t0
    ops = 2.0 * done * c.d_out * (c.d_in + r)
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} tokens ({blk}-token blocks cycling through the {c.M} tokens) of the same "
                      f"{c.d_in}->{c.d_out}, r={r} layer in {dt:.1f} s; numpy, fp64 BLAS for the exact integer "
                      f"products"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="attn_proj_int4", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the SERQ layer needs no collective and this build runs on a "
              f"single MI355X (asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    B.lib()
    dev = torch.device("cuda:0")

    c = WORKLOADS[args.workload]()
    fmt, r, M, K, N = c.fmt, c.r, c.M, c.d_in, c.d_out
    layer = B.PreparedLayer.prepare(c.W, c.X_cal, r, fmt, dev)
    layer0 = B.PreparedLayer.prepare(c.W, c.X_cal, 0, fmt, dev)
    Xh = torch.from_numpy(B.serq_flatten_act(c.X, layer.host["perm"], layer.host["s"])).to(dev)
    Y = torch.empty((M, N), dtype=torch.float32, device=dev)
    ws = layer.workspace(M)
    nq, ns = B.serq_act_bytes(M, K, fmt)
    xq, xs = torch.empty(nq, dtype=torch.uint8, device=dev), torch.empty(ns, dtype=torch.uint8, device=dev)
    d, d0 = layer.dev, layer0.dev

    step = lambda: layer(Xh, Y, ws)                                               # noqa: E731
    quant = lambda: B.serq_quant_act(Xh, fmt, xq, xs)                            # noqa: E731
    gemm = lambda: B.serq_linear_q(layer.L, xq, xs, M, d["wq"], d["wscale"], d["rq"], d["rscale"], Y)  # noqa: E731
    gemm0 = lambda: B.serq_linear_q(layer0.L, xq, xs, M, d0["wq"], d0["wscale"], d0["rq"], d0["rscale"], Y)  # noqa: E731

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: exactly K steps, synchronized on both sides
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps

    # per-kernel averages by HIP events (quantizer, fused GEMM at r and at 0)
    n_ev = max(50, args.steps)
    quant(); gemm(); gemm0()
    torch.cuda.synchronize()
    t_quant = time_launches(quant, n_ev, torch)
    t_gemm = time_launches(gemm, n_ev, torch)
    t_gemm0 = time_launches(gemm0, n_ev, torch)

    ops = 2.0 * M * N * (K + r)
    bound, peak, unit = PEAK[fmt]
    achieved = ops / t_gemm / 1e12
    kname = "gemm_int" if fmt in ("int4", "w4a8") else "gemm_mx"
    quant_bytes = M * K * 4 + nq + ns
    out = {
        "metric": "serq_linear TOPS & % of MFMA peak (prefill); residual overhead vs rank-0 (%)",
        "value": round(ops / dt / 1e12, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dt * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": fmt,
        "data": "synthetic",
        "config": {"workload": "LLaMA-2-7B attention projection, 2048 tokens, 4096->4096, r=128, W4A4 INT4",
                   "M": M, "d_in": K, "d_out": N, "r": r, "fmt": fmt, "x_dtype": "f32",
                   "parallelism": "single GPU"},
        "pct_of_peak": round(100.0 * ops / dt / 1e12 / peak, 2),
        "residual_overhead_pct": round(100.0 * (t_gemm / t_gemm0 - 1.0), 2),
        "residual_overhead_target_pct": round(100.0 * r / K + 3.0, 2),
        "kernels_us": {"quant_act": round(t_quant * 1e6, 3), kname: round(t_gemm * 1e6, 3),
                       kname + "_r0": round(t_gemm0 * 1e6, 3)},
        "quant_act_hbm_gbs": round(quant_bytes / t_quant / 1e9, 1),
        "roofline": {"kernel": kname, "bound": bound, "achieved": round(achieved, 2), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": traffic_from_profiles(f"{kname}_{args.workload}")},
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(c, r, fmt, args.cpu_seconds)
        out["cpu_baseline"]["value"] = round(out["cpu_baseline"]["value"], 5)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
