"""Hardware-counter runs of the library's kernels (for rocprofv3 --pmc).

Run under the profiler, this module drives the dominant layer of a named
benchmark workload (the one with the most operations): it quantizes the
activations and runs the fused linear layer `reps` times, then performs one
plain device copy of 64 MiB.  The copy calibrates the counters: FETCH_SIZE
and WRITE_SIZE of a kernel are scaled by (copied bytes / what the copy's own
counter reads), which turns them into HBM bytes per dispatch.

    rocprofv3 --pmc FETCH_SIZE -d <dir>/FETCH_SIZE -o FETCH_SIZE --output-format csv \\
        -- python3 -m rank_error_compensated_amd.profiling --workload attn_proj_int4
    rocprofv3 --pmc WRITE_SIZE -d <dir>/WRITE_SIZE -o WRITE_SIZE --output-format csv \\
        -- python3 -m rank_error_compensated_amd.profiling --workload attn_proj_int4
    python3 -m rank_error_compensated_amd.profiling --workload attn_proj_int4 --summarize <dir>

--summarize (no GPU needed) reads the two counter CSVs and prints a JSON
record: per-dispatch counters of the fused kernel, the calibration factors,
HBM bytes per launch and the kernel source hash they belong to.

Instruction and stall counters of the fused kernel (two passes within the
per-pass counter limits, then a summary with derived ratios):

    rocprofv3 --pmc SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU \
        SQ_ACTIVE_INST_LDS SQ_WAIT_INST_LDS SQ_LDS_BANK_CONFLICT SQ_INSTS_MFMA GRBM_GUI_ACTIVE \
        -d <dir>/A -o A --output-format csv -- python3 -m rank_error_compensated_amd.profiling --workload W
    rocprofv3 --pmc SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_VALU_MFMA_COEXEC_CYCLES \
        SQ_INSTS_VALU SQ_INSTS_LDS SQ_CYCLES SQ_LDS_DATA_FIFO_FULL \
        -d <dir>/B -o B --output-format csv -- python3 -m rank_error_compensated_amd.profiling --workload W
    python3 -m rank_error_compensated_amd.profiling --workload W --counters-summarize <dir>

The residual overhead against rank 0, from a kernel trace:

    rocprofv3 --kernel-trace -d <dir> -o run --output-format csv \
        -- python3 -m rank_error_compensated_amd.profiling --workload attn_proj_int4 --residual
    python3 -m rank_error_compensated_amd.profiling --workload attn_proj_int4 --residual-summarize <dir>

--residual runs the fused layer prepared at rank r and at rank 0 in runs of
back-to-back launches (rotating six weight copies for decode layers of at
most 16 tokens), one activation quantization marking the end of each run:
a warm-up run of each (at least 50 ms), then rank r, rank 0, rank 0, rank r,
so that a clock drift that is linear in time falls on both sides alike.  The summary splits the trace
into runs of consecutive fused-kernel dispatches, drops the warm-up runs and
the first launches of every run, and reports the mean of the rank-r runs
over that of the rank-0 runs.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sys
import time

from . import binding as B
from . import workloads as WL

COPY_BYTES = 64 << 20
KERNEL_SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "serq_kernels.hip")


def kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def dominant(name: str):
    cases = WL.NAMED[name][1]()
    return max(cases, key=lambda c: c.M * c.d_out * (c.d_in + c.r))


def drive(name: str, reps: int) -> None:
    import torch
    assert torch.cuda.is_available(), "the counter run needs a GPU"
    c = dominant(name)
    layer = B.PreparedLayer.prepare(c.W, c.X_cal, c.r, c.fmt, "cuda")
    Xh = torch.from_numpy(B.serq_flatten_act(c.X, layer.host["perm"], layer.host["s"])).cuda()
    nq, ns = B.serq_act_bytes(c.M, c.d_in, c.fmt)
    xq = torch.empty(nq, dtype=torch.uint8, device="cuda")
    xs = torch.empty(ns, dtype=torch.uint8, device="cuda")
    Y = torch.empty((c.M, c.d_out), dtype=torch.float32, device="cuda")
    d = layer.dev
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for i in range(reps):
        B.serq_quant_act(Xh, c.fmt, xq, xs)
        B.serq_linear_q(layer.L, xq, xs, c.M, d["wq"], d["wscale"], d["rq"], d["rscale"], Y)
        torch.cuda.synchronize()
        print(f"rep {i} done", flush=True)
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"{name}: layer {c.name} {c.M}x{c.d_in}->{c.d_out} r={c.r} {c.fmt}, {reps} reps, 64 MiB copy", flush=True)


RESIDUAL_WARM = 3                    # launches dropped at the start of every run
RESIDUAL_ORDER = (0, 1, 0, 1, 1, 0)  # runs: 0 = rank r, 1 = rank 0; the first two warm up
RESIDUAL_WARM_S = 0.05               # seconds of each warm-up run, at least


def drive_residual(name: str, reps: int) -> None:
    import torch
    assert torch.cuda.is_available(), "the trace run needs a GPU"
    c = dominant(name)
    runs = []
    for r in (c.r, 0):
        layer = B.PreparedLayer.prepare(c.W, c.X_cal, r, c.fmt, "cuda")
        Xh = torch.from_numpy(B.serq_flatten_act(c.X, layer.host["perm"], layer.host["s"])).cuda()
        nq, ns = B.serq_act_bytes(c.M, c.d_in, c.fmt)
        xq = torch.empty(nq, dtype=torch.uint8, device="cuda")
        xs = torch.empty(ns, dtype=torch.uint8, device="cuda")
        B.serq_quant_act(Xh, c.fmt, xq, xs)
        Y = torch.empty((c.M, c.d_out), dtype=torch.float32, device="cuda")
        runs.append((r, layer, Xh, xq, xs, Y))
    torch.cuda.synchronize()
    # decode layers stream their weights from HBM: rotate copies, as the bench
    # does, so that the memory-side cache does not hold them between launches
    copies = 6 if c.M <= 16 else 1
    ds = {r: [layer.dev] + [{k: v.clone() for k, v in layer.dev.items()} for _ in range(copies - 1)]
          for r, layer, *_ in runs}
    for phase, which in enumerate(RESIDUAL_ORDER):
        r, layer, Xh, xq, xs, Y = runs[which]
        n, t0 = 0, time.perf_counter()
        while True:
            for _ in range(RESIDUAL_WARM + reps if n == 0 else reps):
                d = ds[r][n % copies]
                B.serq_linear_q(layer.L, xq, xs, c.M, d["wq"], d["wscale"], d["rq"], d["rscale"], Y)
                n += 1
            torch.cuda.synchronize()
            # the two warm-up runs last at least RESIDUAL_WARM_S each, long
            # enough for the clocks to settle
            if phase >= 2 or time.perf_counter() - t0 >= RESIDUAL_WARM_S:
                break
        B.serq_quant_act(Xh, c.fmt, xq, xs)   # marker: ends this run of fused launches
        torch.cuda.synchronize()
        print(f"run {phase}: rank {r}, {n} launches", flush=True)
    print(f"{name}: layer {c.name} {c.M}x{c.d_in}->{c.d_out} r={c.r} {c.fmt}", flush=True)


def summarize_residual(name: str, root: str) -> dict:
    files = glob.glob(os.path.join(root, "**", "*kernel_trace.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"expected one kernel trace CSV under {root}, found {files}")
    rows = sorted(csv.DictReader(open(files[0])), key=lambda r: int(r["Start_Timestamp"]))
    blocks, cur = [], []
    for r in rows:
        name_k = r["Kernel_Name"]
        if "serq::" not in name_k:
            continue                                   # torch's own kernels
        if "k_gemm" in name_k or "k_decode" in name_k:
            cur.append((name_k, (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3))
        elif cur:
            blocks.append(cur)
            cur = []
    if cur:
        blocks.append(cur)
    if len(blocks) != len(RESIDUAL_ORDER):
        raise SystemExit(f"expected {len(RESIDUAL_ORDER)} runs of fused launches, found {len(blocks)}")
    out = {}
    for key, side in (("rank_r", 0), ("rank_0", 1)):
        us, kern, per_run = [], set(), []
        for blk in [b for b, which in list(zip(blocks, RESIDUAL_ORDER))[2:] if which == side]:
            kern |= {k for k, _ in blk}
            if len(blk) <= RESIDUAL_WARM:
                raise SystemExit(f"{key}: a run of {len(blk)} launches")
            t = [x for _, x in blk[RESIDUAL_WARM:]]
            per_run.append(sum(t) / len(t))
            us += t
        if len(kern) != 1:
            raise SystemExit(f"{key}: expected one fused kernel, found {kern}")
        out[key] = {"kernel": kern.pop(), "launches": len(us), "avg_us": sum(us) / len(us), "min_us": min(us),
                    "max_us": max(us), "run_avgs_us": per_run}
    c = dominant(name)
    return {
        "workload": name, "layer": f"{c.name} {c.M}x{c.d_in}->{c.d_out} r={c.r} {c.fmt}",
        "kernel_src_sha256_16": kernel_hash(),
        "command": "rocprofv3 --kernel-trace -- python3 -m rank_error_compensated_amd.profiling "
                   f"--workload {name} --residual",
        **out,
        "residual_overhead_pct": 100.0 * (out["rank_r"]["avg_us"] / out["rank_0"]["avg_us"] - 1.0),
        "target_pct": 100.0 * c.r / c.d_in + 3.0,
    }


# MI355X: 8 XCDs (GRBM_GUI_ACTIVE sums their busy cycles), 256 CUs of 4 SIMDs
N_XCD, N_SIMD = 8, 256 * 4


def summarize_counters(name: str, root: str) -> dict:
    files = glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter CSV under {root}")
    vals = collections.defaultdict(list)
    kernels = set()
    for f in files:
        for r in csv.DictReader(open(f)):
            k = r["Kernel_Name"]
            if "k_gemm" in k or "k_decode" in k:
                kernels.add(k)
                vals[r["Counter_Name"]].append(float(r["Counter_Value"]))
    if len(kernels) != 1:
        raise SystemExit(f"expected one fused kernel, found {kernels}")
    m = {c: sum(v) / len(v) for c, v in vals.items()}
    out = {"workload": name, "kernel": kernels.pop(), "kernel_src_sha256_16": kernel_hash(),
           "counters_mean_per_dispatch": m}
    d = {}
    if "GRBM_GUI_ACTIVE" in m and "SQ_VALU_MFMA_BUSY_CYCLES" in m:
        cycles = m["GRBM_GUI_ACTIVE"] / N_XCD
        d["kernel_cycles"] = cycles
        d["mfma_busy_fraction_per_simd"] = m["SQ_VALU_MFMA_BUSY_CYCLES"] / N_SIMD / cycles
    if "SQ_INSTS_MFMA" in m:
        n = m["SQ_INSTS_MFMA"]
        if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
            d["mfma_busy_cycles_per_mfma"] = m["SQ_VALU_MFMA_BUSY_CYCLES"] / n
        if "SQ_INSTS_VALU" in m:
            d["other_valu_per_mfma"] = (m["SQ_INSTS_VALU"] - n) / n
        if "SQ_INSTS_LDS" in m:
            d["lds_instr_per_mfma"] = m["SQ_INSTS_LDS"] / n
    if "SQ_WAVE_CYCLES" in m:   # both in quad-cycles, summed over waves
        for c in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
                  "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS"):
            if c in m:
                d[c.lower().replace("sq_", "") + "_fraction_of_wave_cycles"] = m[c] / m["SQ_WAVE_CYCLES"]
    if "SQ_VALU_MFMA_COEXEC_CYCLES" in m and "SQ_VALU_MFMA_BUSY_CYCLES" in m:
        d["valu_coexec_fraction_of_mfma_busy"] = m["SQ_VALU_MFMA_COEXEC_CYCLES"] / m["SQ_VALU_MFMA_BUSY_CYCLES"]
    out["derived"] = d
    return out


def summarize(name: str, root: str) -> dict:
    per = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        files = glob.glob(os.path.join(root, ctr, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter CSV under {root}/{ctr}")
        rows = collections.defaultdict(list)
        for r in csv.DictReader(open(files[0])):
            rows[r["Kernel_Name"]].append((int(r.get("Dispatch_Id") or 0), float(r["Counter_Value"])))
        per[ctr] = {k: [v for _, v in sorted(vals)] for k, vals in rows.items()}
    copy_k = [k for k in per["FETCH_SIZE"] if "copy" in k.lower()]
    fused = [k for k in per["FETCH_SIZE"] if "k_gemm" in k or "k_decode" in k]
    if len(copy_k) != 1 or len(fused) != 1:
        raise SystemExit(f"expected one copy and one fused kernel, found {copy_k} {fused}")
    ck, fk = copy_k[0], fused[0]
    scale = {ctr: COPY_BYTES / (per[ctr][ck][-1] * 1024.0) for ctr in per}
    kib = {ctr: per[ctr][fk] for ctr in per}
    mean = {ctr: sum(v) / len(v) for ctr, v in kib.items()}
    read_b = mean["FETCH_SIZE"] * 1024.0 * scale["FETCH_SIZE"]
    write_b = mean["WRITE_SIZE"] * 1024.0 * scale["WRITE_SIZE"]
    c = dominant(name)
    L = B.serq_query_layout(c.d_in, c.d_out, c.r, c.fmt)
    nq, ns = B.serq_act_bytes(c.M, c.d_in, c.fmt)
    return {
        "kernel": fk, "workload": name, "layer": f"{c.name} {c.M}x{c.d_in}->{c.d_out} r={c.r} {c.fmt}",
        "kernel_src_sha256_16": kernel_hash(),
        "command": "rocprofv3 --pmc <FETCH_SIZE | WRITE_SIZE> -- python3 -m rank_error_compensated_amd.profiling "
                   f"--workload {name}",
        "fetch_size_kib_per_dispatch": kib["FETCH_SIZE"], "write_size_kib_per_dispatch": kib["WRITE_SIZE"],
        "copy_64MiB_kib": {ctr: per[ctr][ck][-1] for ctr in per},
        "fetch_scale": scale["FETCH_SIZE"], "write_scale": scale["WRITE_SIZE"],
        "hbm_read_bytes_per_launch": read_b, "hbm_write_bytes_per_launch": write_b,
        "hbm_bytes_per_launch": read_b + write_b,
        "algorithmic_read_bytes": L.wq_bytes + L.wscale_bytes + L.rq_bytes + L.rscale_bytes + nq + ns,
        "algorithmic_write_bytes": c.M * c.d_out * 4,
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="attn_proj_int4", choices=sorted(WL.NAMED))
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--summarize", metavar="DIR", help="read the two counter runs under DIR")
    ap.add_argument("--residual", action="store_true", help="drive rank r, then rank 0, for a kernel trace")
    ap.add_argument("--residual-summarize", metavar="DIR", help="read the kernel trace of a --residual run")
    ap.add_argument("--counters-summarize", metavar="DIR", help="read SQ counter runs under DIR")
    args = ap.parse_args()
    if args.summarize:
        print(json.dumps(summarize(args.workload, args.summarize), indent=1))
    elif args.counters_summarize:
        print(json.dumps(summarize_counters(args.workload, args.counters_summarize), indent=1))
    elif args.residual_summarize:
        print(json.dumps(summarize_residual(args.workload, args.residual_summarize), indent=1))
    elif args.residual:
        drive_residual(args.workload, max(args.reps, 20))
    else:
        drive(args.workload, args.reps)
    return 0


if __name__ == "__main__":
    sys.exit(main())
