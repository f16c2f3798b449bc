"""Host-side logic of the profiling summaries (no GPU): the residual-overhead
summary of a kernel trace splits it into runs of fused-kernel launches
separated by the library's other kernels, drops warm-up launches and
reports rank r over rank 0; malformed traces are refused."""
import csv
import os

import pytest

from rank_error_compensated_amd import profiling as P

FIELDS = ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]
GEMM = "void serq::(anonymous namespace)::k_decode_int<false, 4, 4, 2>(serq::(anonymous namespace)::IntArgs)"
QUANT = "void serq::(anonymous namespace)::k_quant_int<7, false, 1, 1024>(void const*, int, unsigned char*, float*, int*)"
TORCH = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>>"


def write_trace(path, seq):
    t = 1000
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for name, us in seq:
            w.writerow({"Kind": "KERNEL_DISPATCH", "Kernel_Name": name, "Start_Timestamp": t,
                        "End_Timestamp": t + int(us * 1000)})
            t += int(us * 1000) + 500


def residual_trace(r_us, r0_us, n=10):
    """Quantizer launches, then the runs in the driver's order (rank r or
    rank 0), each ended by a quantizer launch; the two warm-up runs are slow."""
    warm = P.RESIDUAL_WARM
    seq = [(QUANT, 3.0), (TORCH, 1.0), (QUANT, 3.0)]
    for phase, which in enumerate(P.RESIDUAL_ORDER):
        us = (r_us, r0_us)[which]
        body = [(GEMM, 99.0)] * 2 * n if phase < 2 else [(GEMM, us)] * (n // 2) + [(TORCH, 1.0)] + [(GEMM, us)] * (n - n // 2)
        seq += [(GEMM, 50.0)] * warm + body + [(QUANT, 3.0)]
    return seq


def test_residual_summary_from_trace(tmp_path):
    d = tmp_path / "trace"
    d.mkdir()
    write_trace(d / "run_kernel_trace.csv", residual_trace(11.0, 10.0))
    out = P.summarize_residual("decode_int4_m16", str(d))
    n_runs = (len(P.RESIDUAL_ORDER) - 2) // 2
    assert out["rank_r"]["launches"] == 10 * n_runs and out["rank_0"]["launches"] == 10 * n_runs
    assert out["rank_r"]["avg_us"] == pytest.approx(11.0)
    assert out["rank_0"]["avg_us"] == pytest.approx(10.0)
    assert out["residual_overhead_pct"] == pytest.approx(10.0)
    assert out["target_pct"] == pytest.approx(100.0 * 256 / 4096 + 3.0)
    assert len(out["quad_overheads_pct"]) == P.RESIDUAL_QUADS
    assert out["quad_mean_pct"] == pytest.approx(10.0) and out["quad_sd_pct"] == pytest.approx(0.0, abs=1e-9)
    md = P.render_markdown(out)
    assert "10.00 % mean over the quads" in md and "target r/d_in + 3 % = 9.25 %" in md


def test_residual_quads_cancel_a_linear_drift(tmp_path):
    """Kernel times growing linearly with the run index (a clock drift) leave
    every (r, 0, 0, r) quad's overhead at the true ratio."""
    warm = P.RESIDUAL_WARM
    seq = [(QUANT, 3.0)]
    for phase, which in enumerate(P.RESIDUAL_ORDER):
        base = 1.0 + 0.01 * phase
        us = (11.0, 10.0)[which] * base
        seq += [(GEMM, 50.0)] * warm + [(GEMM, us)] * 6 + [(QUANT, 3.0)]
    d = tmp_path / "trace"
    d.mkdir()
    write_trace(d / "run_kernel_trace.csv", seq)
    out = P.summarize_residual("decode_int4_m16", str(d), layer="down")
    assert out["layer"].startswith("down ")
    assert "--layer down" in out["command"]
    for q in out["quad_overheads_pct"]:
        assert q == pytest.approx(10.0, abs=0.02)


def test_residual_summary_refuses_a_missing_run(tmp_path):
    seq = residual_trace(11.0, 10.0)[:-14]
    d = tmp_path / "trace"
    d.mkdir()
    write_trace(d / "run_kernel_trace.csv", seq)
    with pytest.raises(SystemExit):
        P.summarize_residual("decode_int4_m16", str(d))


def test_counter_summary_from_csv(tmp_path):
    """--counters-summarize averages each counter over the fused kernel's
    dispatches (other kernels ignored) and derives the ratios from them."""
    rows = []
    for disp in range(2):
        for name, val in (("GRBM_GUI_ACTIVE", 8 * 1000.0), ("SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 250.0),
                          ("SQ_INSTS_MFMA", 100.0 + disp * 2), ("SQ_INSTS_VALU", 301.0 + disp * 6),
                          ("SQ_INSTS_LDS", 50.0), ("SQ_WAVE_CYCLES", 400.0), ("SQ_WAIT_ANY", 100.0)):
            rows.append({"Kernel_Name": GEMM, "Counter_Name": name, "Counter_Value": val})
        rows.append({"Kernel_Name": QUANT, "Counter_Name": "SQ_INSTS_MFMA", "Counter_Value": 9999.0})
    d = tmp_path / "sq" / "A"
    d.mkdir(parents=True)
    with open(d / "A_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        w.writerows(rows)
    out = P.summarize_counters("decode_int4_m16", str(tmp_path / "sq"))
    dv = out["derived"]
    assert out["counters_mean_per_dispatch"]["SQ_INSTS_MFMA"] == pytest.approx(101.0)
    assert dv["kernel_cycles"] == pytest.approx(1000.0)
    assert dv["mfma_busy_fraction_per_simd"] == pytest.approx(0.25)
    assert dv["other_valu_per_mfma"] == pytest.approx((304.0 - 101.0) / 101.0)
    assert dv["wait_any_fraction_of_wave_cycles"] == pytest.approx(0.25)
