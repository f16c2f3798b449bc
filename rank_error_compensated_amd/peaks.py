"""Sustained MFMA and HBM rates of the GPU, measured with libserq_peaks.so
(include/serq_peaks.h), for reading the layer's roofline fractions against
what the chip sustains beside AMD's published peaks.

    python -m rank_error_compensated_amd.peaks        # prints one JSON record

MFMA probes: one workgroup per compute unit with one or two waves per SIMD,
each wave issuing back-to-back MFMAs on 8 independent register accumulators;
rate = MFMAs x ops per MFMA / time (HIP events around several launches on
the current stream).  The shader clock under each load comes from the first
wave's cycle counter against the constant-rate wall clock.  HBM: a 1 GiB
streaming read and a 512 MiB copy (larger than the 256 MB memory-side cache).
"""
from __future__ import annotations

import ctypes
import json
import os
import sys

from ._build import PEAKS_LIB

OPS = {0: 32768, 1: 65536, 2: 65536, 3: 65536}            # per MFMA instruction
KIND = {"int8": 0, "fp4": 1, "fp8": 2, "fp4xfp8": 3}
PUBLISHED = {"int8": 5000.0, "fp4": 10100.0, "fp8": 5000.0, "fp4xfp8": 5000.0, "hbm_gbs": 8000.0}

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(PEAKS_LIB):
            raise RuntimeError(f"{PEAKS_LIB} is missing: build it with `python -m rank_error_compensated_amd._build`")
        L = ctypes.CDLL(PEAKS_LIB)
        vp = ctypes.c_void_p
        L.serq_peak_sink_floats.argtypes = [ctypes.c_int]
        L.serq_peak_wall_khz.argtypes = []
        L.serq_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp]
        L.serq_peak_read.argtypes = [vp, ctypes.c_size_t, vp, vp]
        L.serq_peak_copy.argtypes = [vp, vp, ctypes.c_size_t, vp]
        _lib = L
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what} returned {rc}")


def _time(fn, torch, reps: int) -> float:
    fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) * 1e-3 / reps


def measure(iters: int = 20000, reps: int = 5) -> dict:
    import torch
    assert torch.cuda.is_available(), "the peak probes need a GPU"
    L = lib()
    cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    wall_khz = L.serq_peak_wall_khz()
    out = {"compute_units": cus, "mfma": {}}
    clocks = torch.zeros(2, dtype=torch.int64, device="cuda")
    stream = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for name, kind in KIND.items():
        for wps in (1, 2):
            sink = torch.empty(L.serq_peak_sink_floats(wps), dtype=torch.float32, device="cuda")
            fn = lambda: _check(L.serq_peak_mfma(kind, wps, iters, ctypes.c_void_p(sink.data_ptr()),
                                                 ctypes.c_void_p(clocks.data_ptr()), stream()), "serq_peak_mfma")
            t = _time(fn, torch, reps)
            waves = cus * 4 * wps
            rate = waves * iters * 8 * OPS[kind] / t / 1e12
            cyc, ticks = (int(v) for v in clocks.cpu())
            rec = {"tera_ops_per_s": round(rate, 1), "of_published": round(rate / PUBLISHED[name], 3)}
            if wall_khz:
                # the first wave's shader clock over its loop; SIMD cycles per
                # MFMA over the whole launch at that clock
                mhz = cyc / (ticks / wall_khz) / 1e3
                rec["sclk_mhz"] = round(mhz, 0)
                rec["simd_cycles_per_mfma"] = round(t * mhz * 1e6 / (iters * 8 * wps), 2)
            out["mfma"][f"{name}_{wps}wave_per_simd"] = rec
    gib = 1 << 30
    src = torch.empty(gib, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    sink = torch.empty(cus * 8 * 256, dtype=torch.int32, device="cuda")
    t = _time(lambda: _check(L.serq_peak_read(ctypes.c_void_p(src.data_ptr()), gib, ctypes.c_void_p(sink.data_ptr()),
                                              stream()), "serq_peak_read"), torch, reps)
    out["hbm_read_gbs"] = round(gib / t / 1e9, 1)
    half = gib // 2
    dst = torch.empty(half, dtype=torch.uint8, device="cuda")
    t = _time(lambda: _check(L.serq_peak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), half,
                                              stream()), "serq_peak_copy"), torch, reps)
    out["hbm_copy_gbs"] = round(2 * half / t / 1e9, 1)
    out["published"] = PUBLISHED
    del src, dst
    torch.cuda.empty_cache()
    return out


def main() -> int:
    print(json.dumps(measure()), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
