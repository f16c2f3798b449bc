#!/usr/bin/env python3
"""Benchmark of the SERQ linear layer on one MI355X.

A step is one pass of the whole runtime path -- per-token activation
quantization, the packed 4-bit main GEMM with the fused rank-r residual, the
dequant epilogue -- over one batch of synthetic input already resident in
HBM, for every layer of the workload.  The default workload is the largest
prefill set: the LLaMA-3-8B decoder layer's linears (q|k|v, o, gate|up, down)
at 2048 tokens, r = 128, MXFP4.
Prints one JSON line with

  value        serq_linear throughput in TOPS: sum of 2*M*d_out*(d_in + r)
               over the workload's layers / step time
  roofline     the dominant kernel's algorithmic ops (or bytes, for decode)
               per launch / its average launch time (HIP events on the launch
               stream) against the int8 / FP4 MFMA peak (or HBM), published
               and as sustained on this GPU (measured_peaks)
  residual     the GEMM's time at rank r versus the same kernel at rank 0
  cpu_baseline the CPU oracle on a bounded sample of the same workload
  producer_quant  beside the step, not in it: the fused producer kernels
               (RMSNorm or SwiGLU + flatten + quantization) that emit each
               layer's quantized input from its producer's input

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from rank_error_compensated_amd import binding as B  # noqa: E402
from rank_error_compensated_amd import workloads as WL  # noqa: E402
from rank_error_compensated_amd.profiling import kernel_hash  # noqa: E402
from rank_error_compensated_amd import peaks as PK  # noqa: E402

# MI355X dense, 10^12 ops/s; an FP4 x FP8 product issues at the FP8 rate
MFMA_PEAK = {"int4": 5000.0, "w4a8": 5000.0, "mxfp4": 10100.0, "mxw4a8": 5000.0}
HBM_PEAK_GBS = 8000.0


WORKLOADS = WL.NAMED


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


def residual_from_profiles(name: str):
    """The dominant layer's residual overhead against rank 0 from the
    committed rocprofv3 kernel-trace summary (profiling.py --residual), if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{name}_residual.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_src_sha256_16") != kernel_hash():
        return None
    return {"layer": rec["layer"], "overhead_pct": round(rec["residual_overhead_pct"], 2),
            "target_pct": round(rec["target_pct"], 2), "rank_r_us": round(rec["rank_r"]["avg_us"], 2),
            "rank_0_us": round(rec["rank_0"]["avg_us"], 2)}


def capture(fn, n: int, torch):
    """A HIP graph holding n consecutive calls of fn (the library only enqueues
    kernels on the current stream: no allocation, no memset, no sync)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    return g


def time_launches(fn, n: int, torch, reps: int = 5) -> float:
    """Average duration (s) of one fn() launch: n launches captured in a HIP
    graph, replayed reps times between HIP events recorded on torch's current
    stream, the stream the graph runs on (host launch overhead excluded)."""
    g = capture(fn, n, torch)
    g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        g.replay()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) * 1e-3 / (n * reps)


def cpu_baseline(c, r, fmt, budget_s: float = 10.0) -> dict:
    """The CPU oracle, as it stands, on 128-token blocks of one layer of the
    workload (cycling through its tokens) until the time budget is spent:
    per-token quantization + exact products (fp64 BLAS on integer-valued
    arrays, every BLAS thread) + epilogue.  Offline preparation is not timed.

    Beside it, the semantic reference on a slice of the same layer, on one
    thread: for INT formats numpy's np.int32 matmul of the codes (no BLAS),
    for MX formats the block-scaled sum with exact integer block products;
    both are checked equal to the timed form."""
    from oracle import serq_oracle as O
    affinity = len(os.sched_getaffinity(0))
    blas_threads = None
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"]
                           + [1])
    except Exception:
        pass
    p = O.prepare(c.W, c.X_cal, r, fmt)
    Xh = O.flatten_acts(c.X, p["s"], p["perm"])
    blk = min(128, c.M)
    done, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        lo = done % c.M
        O.serq_linear(Xh[lo:lo + blk], p)
        done += blk
    dt = time.perf_counter() - t0
    ops = 2.0 * done * c.d_out * (c.d_in + r)

    # semantic reference on a slice (one thread), cross-checked against the timed form
    mx = fmt in O.MX_FORMATS
    rows, cols = (8, min(c.d_out, 2048)) if mx else (min(128, c.M), min(c.d_out, 1024))
    sub = dict(p)
    sub["wq"], sub["rq"] = p["wq"][:, :cols], p["rq"][:, :cols]
    if mx:
        sub["we"], sub["re"] = p["we"][:, :cols], p["re"][:, :cols]
    else:
        sub["sw"], sub["sR"] = p["sw"][:cols], p["sR"][:cols]
    out = O.serq_linear(Xh[:rows], sub)
    t1 = time.perf_counter()
    if mx:
        Yn = O.linear_mx_blocks(out["xq"], out["xscale"], sub)
        same = bool(np.allclose(Yn, out["Y"], rtol=1e-12, atol=1e-12 * np.abs(out["Y"]).max()))
        kind = "block-scaled sum, exact integer block products (numpy int64 matmul, one thread)"
    else:
        Am = O.int_matmul_naive(out["xq"], sub["wq"])
        Ar = O.int_matmul_naive(out["xq"][:, :r], sub["rq"])
        same = bool(np.array_equal(Am, out["A_main"]) and np.array_equal(Ar, out["A_res"]))
        kind = "np.int32 matmul of the codes (numpy integer matmul, one thread, no BLAS)"
    tn = time.perf_counter() - t1
    ops_n = 2.0 * rows * cols * (c.d_in + r)
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": int(blas_threads or affinity), "kind": "oracle",
            "sample": f"{done} tokens ({blk}-token blocks cycling through the {c.M} tokens) of the "
                      f"{c.d_in}->{c.d_out}, r={r} {fmt} layer '{c.name}' in {dt:.1f} s; numpy, fp64 BLAS "
                      f"for the exact products",
            "blas_threads": blas_threads, "affinity_cpus": affinity,
            "semantic_reference": {"kind": kind, "slice": f"{rows} tokens x {cols} channels",
                                   "seconds": round(tn, 3), "tops": round(ops_n / tn / 1e12, 6),
                                   "equal_to_timed_oracle": same}}


class Layer:
    """One prepared layer on the device: weight copies, input, output,
    workspace and the launch closures the bench times."""

    def __init__(self, c, copies: int, torch, dev):
        self.c = c
        self.fmt, self.r, self.M, self.K, self.N = c.fmt, c.r, c.M, c.d_in, c.d_out
        main = B.PreparedLayer.prepare(c.W, c.X_cal, c.r, c.fmt, dev)
        zero = B.PreparedLayer.prepare(c.W, c.X_cal, 0, c.fmt, dev)
        self.L, self.L0 = main.L, zero.L
        self.host = {"perm": main.host["perm"], "s": main.host["s"]}
        self.copies = [main.dev] + [{k: v.clone() for k, v in main.dev.items()} for _ in range(copies - 1)]
        # the rank-0 layer rotates as many copies, so both sides read from HBM alike
        self.zeros = [zero.dev] + [{k: v.clone() for k, v in zero.dev.items()} for _ in range(copies - 1)]
        self.X = torch.from_numpy(B.serq_flatten_act(c.X, main.host["perm"], main.host["s"])).to(dev)
        self.Y = torch.empty((self.M, self.N), dtype=torch.float32, device=dev)
        self.ws = main.workspace(self.M)
        nq, ns = B.serq_act_bytes(self.M, self.K, self.fmt)
        self.xq = torch.empty(nq, dtype=torch.uint8, device=dev)
        self.xs = torch.empty(ns, dtype=torch.uint8, device=dev)
        self.nq, self.ns = nq, ns
        self.i = 0

    def ops(self) -> float:
        return 2.0 * self.M * self.N * (self.K + self.r)

    def weight_bytes(self, L) -> int:
        return L.wq_bytes + L.wscale_bytes + L.rq_bytes + L.rscale_bytes

    def step(self):
        d = self.copies[self.i % len(self.copies)]
        self.i += 1
        B.serq_linear(self.L, self.X, d["wq"], d["wscale"], d["rq"], d["rscale"], self.Y, self.ws)

    def quant(self):
        B.serq_quant_act(self.X, self.fmt, self.xq, self.xs)

    def gemm(self):
        d = self.copies[self.i % len(self.copies)]
        self.i += 1
        B.serq_linear_q(self.L, self.xq, self.xs, self.M, d["wq"], d["wscale"], d["rq"], d["rscale"], self.Y)

    def gemm0(self):
        d = self.zeros[self.i % len(self.zeros)]
        self.i += 1
        B.serq_linear_q(self.L0, self.xq, self.xs, self.M, d["wq"], d["wscale"], d["rq"], d["rscale"], self.Y)


def O_pairs(Wg: np.ndarray, Wu: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """[W_gate | W_up] with its columns in (gate, up) pairs in the order perm
    (column 2j: gate channel perm[j]; 2j + 1: up channel perm[j])."""
    W = np.empty((Wg.shape[0], 2 * Wg.shape[1]), np.float32)
    W[:, 0::2], W[:, 1::2] = Wg[:, perm], Wu[:, perm]
    return W


def lowrank_factors(E: np.ndarray, k: int, seed: int = 0):
    """Rank-k factors of the weight error for the L2QER comparator: a
    randomized range finder with two power steps, then an SVD of the small
    projected matrix, split evenly (L1 = Q U sqrt(S), L2 = sqrt(S) V^T).  The
    timing does not depend on the factor values; this keeps the offline step
    to seconds at the MLP's 4096 x 28672."""
    rng = np.random.default_rng(seed)
    E64 = E.astype(np.float64)
    Q, _ = np.linalg.qr(E64 @ rng.standard_normal((E.shape[1], k)))
    for _ in range(2):
        Q, _ = np.linalg.qr(E64 @ (E64.T @ Q))
    U, S, Vt = np.linalg.svd(Q.T @ E64, full_matrices=False)
    h = np.sqrt(S)
    return ((Q @ U) * h).astype(np.float32), (h[:, None] * Vt).astype(np.float32)


class L2qerLayer:
    """The L2QER comparator on the same layer: Y = X_q W_q + Q(X_q L1_q) L2_q
    with rank-r factors, sharing the SERQ layer's quantized input."""

    def __init__(self, lay, torch, dev):
        self.lay, self.k = lay, lay.r
        E = B.serq_weight_error(lay.L0, lay.c.W, lay.c.X_cal)
        L1, L2 = lowrank_factors(E, self.k)
        f = B.serq_l2qer_prepare(lay.L0, L1, L2)
        self.f = {n: torch.from_numpy(f[n]).to(dev) for n in ("l1q", "l1scale", "l2q", "l2scale")}
        kp = (self.k + 127) // 128 * 128
        self.tq = torch.empty(lay.M * kp // 2, dtype=torch.uint8, device=dev)
        nts = lay.M * kp // 32 if lay.fmt == "mxfp4" else lay.M * 4 * (1 + kp // 128)   # E8M0 bytes / INT4 xscale
        self.ts = torch.empty(nts, dtype=torch.uint8, device=dev)
        self.ws = torch.empty(B.serq_l2qer_workspace_bytes(lay.L0, lay.M, self.k), dtype=torch.uint8, device=dev)

    def intermediate(self):
        lay = self.lay
        B.serq_l2qer_intermediate(lay.L0, self.k, lay.xq, lay.xs, lay.M, self.f["l1q"], self.f["l1scale"], None,
                                  self.tq, self.ts)

    def gemm(self):
        lay = self.lay
        d = lay.zeros[0]
        B.serq_l2qer_linear_q(lay.L0, self.k, lay.xq, lay.xs, lay.M, d["wq"], d["wscale"], self.tq, self.ts,
                              self.f["l2q"], self.f["l2scale"], lay.Y)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama3_layer_mxfp4", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--gptq", action="store_true",
                    help="also prepare the layers with GPTQ (offline, host) and report the output error "
                         "of round to nearest and GPTQ against the unquantized product")
    ap.add_argument("--skip-r0", action="store_true",
                    help="omit the rank-0 comparison (residual overhead), e.g. under a kernel-trace profiler, so "
                         "that every dispatch of the fused kernel is at rank r")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the SERQ layer needs no collective and this build runs on a "
              f"single MI355X (asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    B.lib()
    dev = torch.device("cuda:0")
    desc, factory, bound, copies = WORKLOADS[args.workload]
    cases = factory()
    layers = [Layer(c, copies, torch, dev) for c in cases]
    fmt = layers[0].fmt

    def step():
        for lay in layers:
            lay.step()

    # The steps run as HIP graphs, as a serving loop would capture them: a
    # graph of G consecutive steps (a multiple of the rotated weight copies,
    # up to 100 steps) replayed steps // G times, then one graph holding the
    # remaining steps % G, so that exactly `steps` steps are timed.
    steps = max(1, args.steps)
    G = max(copies, min(steps, 100) // copies * copies)
    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    graph = capture(step, G, torch)
    graph.replay()
    rest = capture(step, steps % G, torch) if steps % G else None
    if rest is not None:
        rest.replay()
    torch.cuda.synchronize()
    # timed region: exactly `steps` steps, synchronized on both sides
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps // G):
        graph.replay()
    if rest is not None:
        rest.replay()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps

    # per-kernel averages by HIP events (quantizer, fused GEMM at r and at 0)
    n_ev = max(50, args.steps)
    per = []
    for lay in layers:
        lay.quant(); lay.gemm()
        torch.cuda.synchronize()
        tq = time_launches(lay.quant, n_ev, torch)
        if args.skip_r0:
            tg, t0_ = time_launches(lay.gemm, n_ev, torch), None
        else:
            # rank r, rank 0, rank 0, rank r: a clock drift linear in time
            # falls on both sides of the residual overhead alike
            ta = time_launches(lay.gemm, n_ev, torch)
            t0_ = 0.5 * (time_launches(lay.gemm0, n_ev, torch) + time_launches(lay.gemm0, n_ev, torch))
            tg = 0.5 * (ta + time_launches(lay.gemm, n_ev, torch))
        per.append((lay, tq, tg, t0_))

    # Producers fused with quantization (RMSNorm in front of attention and MLP
    # inputs, SwiGLU in front of the down projection): time per layer input,
    # on synthetic producer inputs of the layer's shape.
    prod = {}
    rng = np.random.default_rng(0)
    for lay in layers:
        swiglu = lay.c.group == "down_in"
        perm = torch.from_numpy(np.ascontiguousarray(lay.host["perm"])).to(dev)
        sd = torch.from_numpy(np.ascontiguousarray(lay.host["s"][lay.host["perm"]])).to(dev)   # s in saliency order
        if swiglu:
            src = torch.from_numpy(rng.standard_normal((lay.M, 2 * lay.K)).astype(np.float32)).to(dev)
            fn = lambda lay=lay, src=src, perm=perm, sd=sd: B.serq_swiglu_quant(src, perm, sd, lay.fmt, lay.xq, lay.xs)
        else:
            src = torch.from_numpy(rng.standard_normal((lay.M, lay.K)).astype(np.float32)).to(dev)
            gamma = torch.ones(lay.K, dtype=torch.float32, device=dev)
            fn = lambda lay=lay, src=src, perm=perm, sd=sd, gamma=gamma: B.serq_rmsnorm_quant(
                src, gamma, 1e-5, perm, sd, lay.fmt, lay.xq, lay.xs)
        fn()
        torch.cuda.synchronize()
        tp = time_launches(fn, n_ev, torch)
        nbytes = src.numel() * 4 + lay.nq + lay.ns
        prod[lay.c.name] = {"kernel": "swiglu_quant" if swiglu else "rmsnorm_quant", "us": round(tp * 1e6, 3),
                            "hbm_gbs": round(nbytes / tp / 1e9, 1)}
        if swiglu:   # the permutation folded into gate|up: no gather
            ff = lambda lay=lay, src=src, sd=sd: B.serq_swiglu_quant(src, None, sd, lay.fmt, lay.xq, lay.xs)
            ff()
            torch.cuda.synchronize()
            tf = time_launches(ff, n_ev, torch)
            prod[lay.c.name].update({"us_perm_folded": round(tf * 1e6, 3),
                                     "hbm_gbs_perm_folded": round(nbytes / tf / 1e9, 1)})

    # The L2QER comparator on the same prefill layers (INT4 or MXFP4): its
    # intermediate (the extra GEMM and the on-the-fly quantization) plus its
    # output GEMM, against the same rank-0 GEMM that SERQ's residual overhead
    # uses.
    l2 = None
    l2_ok = {"int4": lambda lay: lay.M > 128 and lay.K % 256 == 0,
             "mxfp4": lambda lay: lay.M > 16 and lay.K % 512 == 0 and lay.r % 32 == 0 and 32 <= lay.r <= 128}
    if fmt in l2_ok and not args.skip_r0 and all(l2_ok[fmt](lay) for lay in layers):
        rows = {}
        for (lay, tq, tg, t0_) in per:
            cmp_ = L2qerLayer(lay, torch, dev)
            cmp_.intermediate(); cmp_.gemm()
            torch.cuda.synchronize()
            ti = time_launches(cmp_.intermediate, n_ev, torch)
            tl = time_launches(cmp_.gemm, n_ev, torch)
            rows[lay.c.name] = (ti, tl, tg, t0_)
        t0s = sum(v[3] for v in rows.values())
        l2_over = 100.0 * ((sum(v[0] + v[1] for v in rows.values())) / t0s - 1.0)
        serq_over = 100.0 * (sum(v[2] for v in rows.values()) / t0s - 1.0)
        l2 = {"rank": layers[0].r, "overhead_pct": round(l2_over, 2), "serq_residual_overhead_pct": round(serq_over, 2),
              "overhead_ratio_l2qer_over_serq": round(l2_over / serq_over, 2) if serq_over > 0 else None,
              "kernels_us": {n: {"intermediate": round(v[0] * 1e6, 3), "gemm_l2qer": round(v[1] * 1e6, 3),
                                 "gemm_serq": round(v[2] * 1e6, 3), "gemm_r0": round(v[3] * 1e6, 3)}
                             for n, v in rows.items()},
              "factors": "rank-r randomized range finder of the weight error (timing is value-independent)"}

    # The MLP with SwiGLU in the gate|up GEMM's epilogue (INT4): the gate|up
    # layer with its columns in (gate, up) pairs in the down projection's
    # saliency order writes the down projection's flattened input H, which
    # the down layer then quantizes, against the unfused chain with the same
    # permutation folded -- gate|up in [gate | up] saliency order, the fused
    # SwiGLU + flatten + quantize producer on its output, the down GEMM.
    mlp = None
    byname = {lay.c.name: lay for lay in layers}
    gu, dn = byname.get("gate_up"), byname.get("down")
    int4_ok = fmt == "int4" and gu is not None and gu.M > 128 and gu.K % 256 == 0
    mx_ok = fmt == "mxfp4" and gu is not None and gu.M > 16 and gu.K % 512 == 0 and gu.r <= 128 and gu.N % 256 == 0
    if dn is not None and (int4_ok or mx_ok):
        d = gu.N // 2
        perm = dn.host["perm"]
        sd = torch.from_numpy(np.ascontiguousarray(dn.host["s"][perm])).to(dev)
        Wg, Wu = gu.c.W[:, :d], gu.c.W[:, d:]
        pair = B.PreparedLayer.prepare(O_pairs(Wg, Wu, perm), gu.c.X_cal, gu.r, fmt, dev)
        block = B.PreparedLayer.prepare(np.concatenate([Wg[:, perm], Wu[:, perm]], axis=1), gu.c.X_cal, gu.r, fmt,
                                        dev)
        Xp = torch.from_numpy(B.serq_flatten_act(gu.c.X, pair.host["perm"], pair.host["s"])).to(dev)
        H = torch.empty((gu.M, d), dtype=torch.float32, device=dev) if int4_ok else None
        Ygu = torch.empty((gu.M, gu.N), dtype=torch.float32, device=dev)
        ws_gu, ws_dn = pair.workspace(gu.M), dn.ws
        dd, pd, bd = dn.copies[0], pair.dev, block.dev

        if int4_ok:   # the epilogue writes H, which the down layer then quantizes
            def gate_up_fused():
                B.serq_linear_swiglu(pair.L, Xp, pd["wq"], pd["wscale"], pd["rq"], pd["rscale"], sd, H, ws_gu)

            def fused():
                gate_up_fused()
                B.serq_linear(dn.L, H, dd["wq"], dd["wscale"], dd["rq"], dd["rscale"], dn.Y, ws_dn)
            steps_txt = "fused: quant_act + gate|up GEMM writing H + quant_act(H) + down GEMM"
        else:         # MXFP4: the epilogue writes the down layer's quantized input
            def gate_up_fused():
                B.serq_linear_swiglu_q(pair.L, Xp, pd["wq"], pd["wscale"], pd["rq"], pd["rscale"], sd, dn.xq, dn.xs,
                                       ws_gu)

            def fused():
                gate_up_fused()
                B.serq_linear_q(dn.L, dn.xq, dn.xs, dn.M, dd["wq"], dd["wscale"], dd["rq"], dd["rscale"], dn.Y)
            steps_txt = "fused: quant_act + gate|up GEMM writing the down layer's MXFP4 codes and scales + down GEMM"

        def unfused():
            B.serq_linear(block.L, Xp, bd["wq"], bd["wscale"], bd["rq"], bd["rscale"], Ygu, ws_gu)
            B.serq_swiglu_quant(Ygu, None, sd, fmt, dn.xq, dn.xs)
            B.serq_linear_q(dn.L, dn.xq, dn.xs, dn.M, dd["wq"], dd["wscale"], dd["rq"], dd["rscale"], dn.Y)

        fused(); unfused()
        torch.cuda.synchronize()
        n_m = max(20, args.steps // 5)
        tf, tu = time_launches(fused, n_m, torch), time_launches(unfused, n_m, torch)
        tk = time_launches(gate_up_fused, n_m, torch)
        tq = time_launches(lambda: B.serq_swiglu_quant(Ygu, None, sd, fmt, dn.xq, dn.xs), n_m, torch)
        tg = time_launches(lambda: B.serq_linear(block.L, Xp, bd["wq"], bd["wscale"], bd["rq"], bd["rscale"], Ygu,
                                                 ws_gu), n_m, torch)
        mlp = {"fused_us": round(tf * 1e6, 2), "unfused_us": round(tu * 1e6, 2),
               "speedup": round(tu / tf, 3),
               "gate_up_swiglu_epilogue_us": round(tk * 1e6, 2), "gate_up_plain_us": round(tg * 1e6, 2),
               "swiglu_quant_folded_us": round(tq * 1e6, 2),
               "steps": steps_txt + "; unfused: quant_act + gate|up GEMM writing Y + swiglu_quant (perm folded) + "
                                    "down GEMM"}

    # GPTQ against round to nearest (opt-in): offline preparation time and the
    # layer output's relative error against the unquantized product
    # X-hat . W-hat (fp64, on a sample of tokens), both through the GPU path,
    # for the workload's own activations (independent channels) and for
    # correlated ones (a rank-64 latent factor, 2048 calibration tokens).
    gq = None
    if args.gptq:
        gq = {}
        rng = np.random.default_rng(7)

        def rel_errs(c, layer_r, layer_g, X, rows):
            perm, sv = layer_r.host["perm"], layer_r.host["s"]
            W_hat = (sv[perm][:, None].astype(np.float32) * c.W[perm]).astype(np.float64)
            ref = X[rows].cpu().numpy().astype(np.float64) @ W_hat
            Y = torch.empty((X.shape[0], c.d_out), dtype=torch.float32, device=dev)
            out = {}
            for name, layer in (("rtn", layer_r), ("gptq", layer_g)):
                layer(X, Y)
                torch.cuda.synchronize()
                out[name] = round(float(np.linalg.norm(Y[rows].cpu().numpy() - ref) / np.linalg.norm(ref)), 5)
            return out

        for lay in layers:
            if lay.N > 8192:
                # the widest layers are left out to keep the leg short (four
                # preparations and an fp64 reference product per layer)
                gq[lay.c.name] = {"skipped": f"{lay.K - lay.r} non-salient rows x {lay.N} channels"}
                continue
            entry = {}
            for label, c in (("independent", lay.c), ("correlated", WL.correlated_case(lay.c))):
                layer_r = B.PreparedLayer.prepare(c.W, c.X_cal, c.r, c.fmt, dev)
                t0 = time.perf_counter()
                layer_g = B.PreparedLayer.prepare(c.W, c.X_cal, c.r, c.fmt, dev, gptq_damp=0.01)
                prep_s = time.perf_counter() - t0
                print(f"gptq: {lay.c.name} ({label}) prepared in {prep_s:.1f} s", file=sys.stderr, flush=True)
                X = torch.from_numpy(B.serq_flatten_act(c.X, layer_r.host["perm"], layer_r.host["s"])).to(dev)
                rows = np.sort(rng.choice(c.M, min(256, c.M), replace=False))
                e = rel_errs(c, layer_r, layer_g, X, rows)
                entry[label] = {"n_cal": int(c.X_cal.shape[0]), "gptq_prep_s": round(prep_s, 2),
                                "rel_err_rtn": e["rtn"], "rel_err_gptq": e["gptq"]}
            gq[lay.c.name] = entry

    ops = sum(lay.ops() for lay in layers)
    t_gemm = sum(p[2] for p in per)
    t_gemm0 = None if args.skip_r0 else sum(p[3] for p in per)
    dom, tq_d, tg_d, _ = max(per, key=lambda p: p[2])
    if dom.M <= 16:   # the decode kernels
        kname = "decode_mx" if fmt in ("mxfp4", "mxw4a8") else "decode_int"
    else:
        kname = {"mxfp4": "gemm_mx", "mxw4a8": "gemm_mx8"}.get(fmt, "gemm_int")
    if bound == "mfma":
        peak = MFMA_PEAK[fmt]
        achieved = dom.ops() / tg_d / 1e12
        roof = {"kernel": kname, "layer": dom.c.name, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
        pct = 100.0 * ops / dt / 1e12 / peak
    else:
        nbytes = dom.weight_bytes(dom.L) + dom.nq + dom.ns + dom.M * dom.N * 4
        achieved = nbytes / tg_d / 1e9
        roof = {"kernel": kname, "layer": dom.c.name, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
        pct = None
    roof["traffic"] = traffic_from_profiles(f"{kname}_{args.workload}")
    # the same fraction against what the chip sustains (libserq_peaks: MFMA
    # loops on register operands, the better of one and two waves per SIMD;
    # a 1 GiB streaming read)
    measured = PK.measure()
    if bound == "mfma":
        unit_kind = {"int4": "int8", "w4a8": "int8", "mxfp4": "fp4", "mxw4a8": "fp4xfp8"}[fmt]
        sustained = max(measured["mfma"][f"{unit_kind}_{w}wave_per_simd"]["tera_ops_per_s"] for w in (1, 2))
    else:
        sustained = measured["hbm_read_gbs"]
    roof["peak_sustained"] = sustained
    roof["frac_of_sustained"] = round(roof["achieved"] / sustained, 4)
    r = layers[0].r
    out = {
        "metric": "serq_linear TOPS & % of MFMA peak (prefill); residual overhead vs rank-0 (%)",
        "value": round(ops / dt / 1e12, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(dt * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": fmt,
        "data": "synthetic",
        "config": {"workload": desc, "layers": [f"{l.c.name} {l.M}x{l.K}->{l.N}" for l in layers], "r": r,
                   "fmt": fmt, "x_dtype": "f32", "parallelism": "single GPU",
                   "weight_copies_rotated": copies, "launch": f"HIP graphs: {steps // G} x {G} steps" + (f" + {steps % G}" if steps % G else "")},
        "pct_of_peak": None if pct is None else round(pct, 2),
        "residual_overhead_pct": None if t_gemm0 is None else round(100.0 * (t_gemm / t_gemm0 - 1.0), 2),
        "residual_overhead_target_pct": round(100.0 * r / min(l.K for l in layers) + 3.0, 2),
        "residual_overhead_rocprof": residual_from_profiles(f"{kname}_{args.workload}"),
        "kernels_us": {l.c.name: {"quant_act": round(tq * 1e6, 3), kname: round(tg * 1e6, 3),
                                  kname + "_r0": None if t0_ is None else round(t0_ * 1e6, 3)}
                       for l, tq, tg, t0_ in per},
        "quant_act_hbm_gbs": round(sum(l.M * l.K * 4 + l.nq + l.ns for l in layers)
                                   / sum(p[1] for p in per) / 1e9, 1),
        "producer_quant": prod,
        "l2qer_comparator": l2,
        "mlp_swiglu_epilogue": mlp,
        "gptq": gq,
        "roofline": roof,
        "measured_peaks": measured,
    }
    if not args.no_cpu:
        cb = cpu_baseline(dom.c, dom.r, fmt, args.cpu_seconds)
        cb["value"] = round(cb["value"], 5)
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
