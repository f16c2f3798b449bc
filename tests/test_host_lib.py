"""CPU tests of libserq.so's host half: exported symbols, argument checks that
must fail before any HIP call, and bit-exact agreement of the library's
offline preparation and activation fold with the oracle."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import serq_oracle as O
from rank_error_compensated_amd import binding as B
from rank_error_compensated_amd import workloads as WL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return B.lib()


def test_exports_every_declared_symbol(lib):
    hdr = open(os.path.join(ROOT, "include", "serq.h")).read()
    names = set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(serq_\w+)\s*\(", hdr, re.M))
    assert names >= set(B.EXPORTS) and len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n


@pytest.mark.parametrize("args,status", [
    ((100, 128, 0, "int4"), B.SERQ_ERR_SHAPE),      # d_in not a multiple of 128
    ((0, 128, 0, "int4"), B.SERQ_ERR_SHAPE),
    ((256, 40, 0, "int4"), B.SERQ_ERR_SHAPE),       # d_out not a multiple of 16
    ((256, 128, 257, "int4"), B.SERQ_ERR_SHAPE),    # r > d_in
    ((256, 128, -1, "int4"), B.SERQ_ERR_SHAPE),
    ((256, 128, 16, "mxfp4"), B.SERQ_ERR_SHAPE),    # MX needs r % 32 == 0
    ((256, 128, 48, "mxw4a8"), B.SERQ_ERR_SHAPE),
    ((256, 128, 16, 7), B.SERQ_ERR_INVALID_ARG),    # unknown format
])
def test_layout_errors(args, status):
    with pytest.raises(B.SerqError) as e:
        B.serq_query_layout(*args)
    assert e.value.status == status
    assert B.lib().serq_last_error()


def test_layout_sizes():
    L = B.serq_query_layout(4096, 4096, 128, "int4")
    assert (L.r_pad, L.wq_bytes, L.rq_bytes, L.wscale_bytes, L.rscale_bytes) == (128, 4096 * 2048, 4096 * 64, 32768, 32768)
    L = B.serq_query_layout(4096, 4096, 128, "w4a8")
    assert (L.wscale_bytes, L.rscale_bytes) == (16384, 16384)
    L = B.serq_query_layout(256, 128, 16, "int4")
    assert L.r_pad == 128
    L = B.serq_query_layout(4096, 1024, 128, "mxfp4")      # E8M0 in 16-byte groups of four K steps a row
    assert (L.wscale_bytes, L.rscale_bytes, L.layout_version) == (1024 * 128, 1024 * 16, 4)
    L = B.serq_query_layout(640, 64, 256, "mxfp4")           # 5 and 2 K steps: one padded group each more
    assert (L.wscale_bytes, L.rscale_bytes) == (64 * 32, 64 * 16)
    L = B.serq_query_layout(256, 32, 0, "mxfp4")
    assert L.r_pad == 0 and L.rq_bytes == 0 and L.rscale_bytes == 0
    assert B.serq_act_bytes(16, 256, "int4") == (16 * 128, 64 + 16 * 2 * 4)
    assert B.serq_act_bytes(16, 256, "w4a8") == (16 * 256, 64)
    assert B.serq_act_bytes(16, 256, "mxfp4") == (16 * 128, 16 * 8)
    L = B.serq_query_layout(4096, 1024, 128, "mxw4a8")      # weights exactly as MXFP4
    assert (L.wq_bytes, L.rq_bytes, L.wscale_bytes, L.rscale_bytes) == (1024 * 2048, 1024 * 64, 1024 * 128, 1024 * 16)
    assert B.serq_act_bytes(16, 256, "mxw4a8") == (16 * 256, 16 * 8)


FAKE = 1 << 20      # a 16-byte aligned non-null address that is never dereferenced


def _L(fmt="int4", d_in=256, d_out=128, r=16):
    return B.serq_query_layout(d_in, d_out, r, fmt)


def test_device_entry_points_reject_bad_arguments_before_any_hip_call(lib):
    L = _L()
    lp = ctypes.byref(L)
    # null input / output
    assert lib.serq_linear(lp, None, 0, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == B.SERQ_ERR_INVALID_ARG
    assert lib.serq_linear(lp, FAKE, 0, 4, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, None) == B.SERQ_ERR_INVALID_ARG
    # M < 1
    assert lib.serq_linear(lp, FAKE, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == B.SERQ_ERR_SHAPE
    # undersized workspace
    need = lib.serq_linear_workspace_bytes(lp, 4)
    assert need > 0
    assert lib.serq_linear(lp, FAKE, 0, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == B.SERQ_ERR_BUFFER
    # misaligned input
    assert lib.serq_linear(lp, FAKE + 4, 0, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == B.SERQ_ERR_INVALID_ARG
    # unknown dtype
    assert lib.serq_linear(lp, FAKE, 9, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == B.SERQ_ERR_INVALID_ARG
    # a layout that serq_query_layout did not produce
    bad = _L()
    bad.r_pad = 64
    assert lib.serq_linear(ctypes.byref(bad), FAKE, 0, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == B.SERQ_ERR_SHAPE
    # the allocation-free form: null pointers, M < 1, misalignment, and more
    # quantized activations than its device array holds
    nl = lib.serq_linear_noalloc
    assert nl(lp, None, 0, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None) == B.SERQ_ERR_INVALID_ARG
    assert nl(lp, FAKE, 0, 4, FAKE, FAKE, FAKE, FAKE, None, None) == B.SERQ_ERR_INVALID_ARG
    assert nl(lp, FAKE, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None) == B.SERQ_ERR_SHAPE
    assert nl(lp, FAKE + 4, 0, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None) == B.SERQ_ERR_INVALID_ARG
    assert nl(lp, FAKE, 9, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None) == B.SERQ_ERR_INVALID_ARG
    m_big = B.NOALLOC_SCRATCH_BYTES // (L.d_in // 2) + 1
    assert lib.serq_linear_workspace_bytes(lp, m_big) > B.NOALLOC_SCRATCH_BYTES
    assert nl(lp, FAKE, 0, m_big, FAKE, FAKE, FAKE, FAKE, FAKE, None) == B.SERQ_ERR_BUFFER
    assert b"64" in lib.serq_last_error() or b"holds at most" in lib.serq_last_error()
    # the SwiGLU epilogue: NULL H or scales, formats and shapes off the large-tile kernel
    sw_ = lib.serq_linear_swiglu
    Lp = _L("int4", d_in=256, d_out=128, r=16)
    lpp = ctypes.byref(Lp)
    ws_need = lib.serq_linear_workspace_bytes(lpp, 256)
    assert sw_(lpp, FAKE, 0, 256, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws_need, None) == B.SERQ_ERR_INVALID_ARG
    assert sw_(lpp, FAKE, 0, 256, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, ws_need, None) == B.SERQ_ERR_INVALID_ARG
    assert sw_(lpp, FAKE, 0, 100, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws_need, None) == B.SERQ_ERR_UNSUPPORTED
    Lm2 = _L("mxfp4", d_in=256, d_out=128, r=32)
    assert sw_(ctypes.byref(Lm2), FAKE, 0, 256, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 24,
               None) == B.SERQ_ERR_UNSUPPORTED
    assert sw_(lpp, FAKE, 0, 256, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws_need - 1, None) == B.SERQ_ERR_BUFFER
    # the quantizing SwiGLU epilogue (MXFP4): NULL outputs, other formats,
    # a next-layer width that is not whole MX blocks, shapes off the
    # LDS-direct kernel, an undersized workspace, misaligned outputs
    sq_ = lib.serq_linear_swiglu_q
    Lq = _L("mxfp4", d_in=512, d_out=256, r=32)
    lq = ctypes.byref(Lq)
    wq_need = lib.serq_linear_workspace_bytes(lq, 64)
    assert sq_(lq, FAKE, 0, 64, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, wq_need, None) == B.SERQ_ERR_INVALID_ARG
    assert sq_(lq, FAKE, 0, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, wq_need, None) == B.SERQ_ERR_INVALID_ARG
    assert sq_(lpp, FAKE, 0, 256, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws_need,
               None) == B.SERQ_ERR_UNSUPPORTED                        # INT4
    Lq128 = _L("mxfp4", d_in=512, d_out=128, r=32)
    assert sq_(ctypes.byref(Lq128), FAKE, 0, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, wq_need,
               None) == B.SERQ_ERR_SHAPE                              # a 64-wide next layer
    assert sq_(lq, FAKE, 0, 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, wq_need,
               None) == B.SERQ_ERR_UNSUPPORTED                        # decode-sized
    Lq256 = _L("mxfp4", d_in=256, d_out=256, r=32)
    assert sq_(ctypes.byref(Lq256), FAKE, 0, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, wq_need,
               None) == B.SERQ_ERR_UNSUPPORTED                        # d_in % 512
    assert sq_(lq, FAKE, 0, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, wq_need - 1, None) == B.SERQ_ERR_BUFFER
    assert sq_(lq, FAKE, 0, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 2, FAKE, FAKE, wq_need,
               None) == B.SERQ_ERR_INVALID_ARG
    # null R with r > 0
    assert lib.serq_linear_q(lp, FAKE, FAKE, 4, FAKE, FAKE, None, FAKE, FAKE, None, None, None) == B.SERQ_ERR_INVALID_ARG
    # only one of the two accumulator buffers
    assert lib.serq_linear_q(lp, FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == B.SERQ_ERR_INVALID_ARG
    # accumulators requested for MX
    Lm = _L("mxfp4", r=32)
    assert lib.serq_linear_q(ctypes.byref(Lm), FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == B.SERQ_ERR_INVALID_ARG
    # quant_act: bad shapes and pointers
    assert lib.serq_quant_act(None, 0, 4, 256, 0, FAKE, FAKE, None) == B.SERQ_ERR_INVALID_ARG
    assert lib.serq_quant_act(FAKE, 0, 4, 200, 0, FAKE, FAKE, None) == B.SERQ_ERR_SHAPE
    assert lib.serq_quant_act(FAKE, 0, 0, 256, 0, FAKE, FAKE, None) == B.SERQ_ERR_SHAPE
    assert lib.serq_quant_act(FAKE, 0, 4, 256, 5, FAKE, FAKE, None) == B.SERQ_ERR_INVALID_ARG
    # producers: pointers, shapes, the row limit, eps, alignment
    rq_ = lib.serq_rmsnorm_quant
    assert rq_(None, 0, 4, 256, FAKE, 1e-5, FAKE, FAKE, 0, FAKE, FAKE, None) == B.SERQ_ERR_INVALID_ARG
    assert rq_(FAKE, 0, 4, 256, None, 1e-5, FAKE, FAKE, 0, FAKE, FAKE, None) == B.SERQ_ERR_INVALID_ARG
    assert rq_(FAKE, 0, 4, 256, FAKE, 1e-5, None, FAKE, 0, FAKE, FAKE, None) == B.SERQ_ERR_INVALID_ARG
    assert rq_(FAKE, 0, 4, 200, FAKE, 1e-5, FAKE, FAKE, 0, FAKE, FAKE, None) == B.SERQ_ERR_SHAPE
    assert rq_(FAKE, 0, 0, 256, FAKE, 1e-5, FAKE, FAKE, 0, FAKE, FAKE, None) == B.SERQ_ERR_SHAPE
    assert rq_(FAKE, 0, 4, 16512, FAKE, 1e-5, FAKE, FAKE, 0, FAKE, FAKE, None) == B.SERQ_ERR_UNSUPPORTED
    assert rq_(FAKE, 0, 4, 256, FAKE, -1.0, FAKE, FAKE, 0, FAKE, FAKE, None) == B.SERQ_ERR_INVALID_ARG
    assert rq_(FAKE, 0, 4, 256, FAKE, float("nan"), FAKE, FAKE, 0, FAKE, FAKE, None) == B.SERQ_ERR_INVALID_ARG
    assert rq_(FAKE, 0, 4, 256, FAKE, 1e-5, FAKE + 4, FAKE, 0, FAKE, FAKE, None) == B.SERQ_ERR_INVALID_ARG
    assert rq_(FAKE, 0, 4, 256, FAKE + 4, 1e-5, FAKE, FAKE, 0, FAKE, FAKE, None) == B.SERQ_ERR_INVALID_ARG
    assert rq_(FAKE, 7, 4, 256, FAKE, 1e-5, FAKE, FAKE, 0, FAKE, FAKE, None) == B.SERQ_ERR_INVALID_ARG
    sq_ = lib.serq_swiglu_quant
    assert sq_(None, 0, 4, 256, FAKE, FAKE, 0, FAKE, FAKE, None) == B.SERQ_ERR_INVALID_ARG
    assert sq_(FAKE, 0, 4, 256, FAKE, None, 0, FAKE, FAKE, None) == B.SERQ_ERR_INVALID_ARG
    assert sq_(FAKE, 0, 4, 256, None, None, 0, FAKE, FAKE, None) == B.SERQ_ERR_INVALID_ARG
    assert sq_(FAKE, 0, 4, 320, FAKE, FAKE, 0, FAKE, FAKE, None) == B.SERQ_ERR_SHAPE
    assert sq_(FAKE, 0, 4, 32768, FAKE, FAKE, 1, FAKE, FAKE, None) == B.SERQ_ERR_UNSUPPORTED
    assert sq_(FAKE, 0, 4, 256, FAKE, FAKE, 9, FAKE, FAKE, None) == B.SERQ_ERR_INVALID_ARG
    assert sq_(FAKE + 8, 0, 4, 256, FAKE, FAKE, 0, FAKE, FAKE, None) == B.SERQ_ERR_INVALID_ARG
    # host prep: null pointers, bad n_cal
    W = np.zeros((256, 128), np.float32)
    with pytest.raises(B.SerqError) as e:
        B.serq_prepare_weights(L, W, np.zeros((0, 256), np.float32))
    assert e.value.status == B.SERQ_ERR_SHAPE


def _compare_prep(case, fmt=None):
    fmt = fmt or case.fmt
    p = O.prepare(case.W, case.X_cal, case.r, fmt)
    want = O.packed_weights(p)
    L = B.serq_query_layout(case.d_in, case.d_out, case.r, fmt)
    got = B.serq_prepare_weights(L, case.W, case.X_cal, want_R=True)
    np.testing.assert_array_equal(got["s"], want["s"])
    np.testing.assert_array_equal(got["perm"], want["perm"])
    np.testing.assert_array_equal(got["wq"], want["wq"])
    np.testing.assert_array_equal(got["wscale"], want["wscale"])
    np.testing.assert_array_equal(got["rq"], want["rq"])
    np.testing.assert_array_equal(got["rscale"], want["rscale"])
    np.testing.assert_array_equal(got["R"], p["R"])
    return p, got


@pytest.mark.parametrize("fmt", ["int4", "w4a8", "mxfp4", "mxw4a8"])
@pytest.mark.parametrize("r", [0, 32, 128, 256])
def test_prepare_matches_oracle_bit_exactly(fmt, r):
    c = WL.random_case(100 + r, 8, 256, 48, r, fmt, n_out=5, factor=50.0, n_cal=40)
    _compare_prep(c)


def test_prepare_ties_zero_rows_and_zero_columns():
    c = WL.random_case(7, 4, 128, 32, 64, "int4", n_out=2, factor=40.0, n_cal=8)
    c.W[5] = 0.0                      # a zero weight row: s = 1
    c.W[:, 3] = 0.0                   # a zero output column: sw = 0, codes 0
    c.X_cal[:, 9] = 0.0               # a channel never active in calibration
    c.W[10] = c.W[11]                 # equal rows and equal activations -> tied s
    c.X_cal[:, 10] = c.X_cal[:, 11]
    for fmt in ("int4", "mxfp4", "mxw4a8"):
        _compare_prep(c, fmt)


def test_prepare_tiny_workload_matches_oracle():
    _compare_prep(WL.tiny_int4()[0])


@pytest.mark.slow
def test_prepare_attention_projection_matches_oracle():
    c = WL.attn_proj_int4(M=16)[0]
    _compare_prep(c)
    _compare_prep(c, "mxfp4")


def test_flatten_act_matches_oracle_bit_exactly():
    c = WL.random_case(31, 20, 256, 32, 16, "int4", n_out=4, factor=50.0, n_cal=16)
    s = O.saf_scales(c.W, c.X_cal)
    perm = O.saliency_perm(s)
    np.testing.assert_array_equal(B.serq_flatten_act(c.X, perm, s), O.flatten_acts(c.X, s, perm))
    with pytest.raises(B.SerqError):
        B.serq_flatten_act(c.X, np.full(256, 999, np.int32), s)


# ---------------------------------------------------------------- GPTQ preparation

@pytest.mark.parametrize("fmt,r", [("int4", 0), ("int4", 64), ("w4a8", 128), ("int4", 256), ("mxfp4", 0),
                                   ("mxfp4", 64), ("mxw4a8", 128)])
def test_gptq_prepare_matches_oracle_bit_exactly(fmt, r):
    """The library's GPTQ (lazy block updates from the Cholesky factor of the
    reversed Hessian, no inverse formed; threads over output channels)
    against the oracle's textbook form (numpy inverse and Cholesky, row by
    row), for What_q's non-salient rows and for Q(R): every code and every MX
    group scale is decided on an fp64 row rounded to fp32, so the two fp64
    routes agree unless a value sits within ~1e-11 of a rounding tie."""
    c = WL.random_case(200 + r, 8, 384, 80, r, fmt, n_out=5, factor=40.0, n_cal=96)
    L = B.serq_query_layout(c.d_in, c.d_out, r, fmt)
    got = B.serq_prepare_weights(L, c.W, c.X_cal, gptq_damp=0.01)
    want = O.packed_weights(O.prepare_gptq(c.W, c.X_cal, r, fmt))
    for k in ("perm", "s", "wq", "wscale", "rq", "rscale"):
        np.testing.assert_array_equal(got[k], want[k], err_msg=k)
    rtn = B.serq_prepare_weights(L, c.W, c.X_cal)
    assert np.any(rtn["wq"] != got["wq"])


def test_gptq_prepare_dead_channels_and_errors():
    c = WL.random_case(9, 8, 256, 32, 32, "int4", n_out=3, factor=40.0, n_cal=64)
    c.X_cal[:, 40:60] = 0.0
    L = B.serq_query_layout(c.d_in, c.d_out, 32, "int4")
    got = B.serq_prepare_weights(L, c.W, c.X_cal, gptq_damp=0.01)
    want = O.packed_weights(O.prepare_gptq(c.W, c.X_cal, 32, "int4"))
    np.testing.assert_array_equal(got["wq"], want["wq"])
    for bad, status in ((-1.0, B.SERQ_ERR_INVALID_ARG), (float("nan"), B.SERQ_ERR_INVALID_ARG)):
        with pytest.raises(B.SerqError) as e:
            B.serq_prepare_weights(L, c.W, c.X_cal, gptq_damp=bad)
        assert e.value.status == status
    # d_in beyond 32768 (a Hessian factor of more than 8 GiB): refused before any work
    W = np.zeros((32896, 16), np.float32)
    Lb = B.serq_query_layout(32896, 16, 128, "mxfp4")
    with pytest.raises(B.SerqError) as e:
        B.serq_prepare_weights(Lb, W, np.ones((2, 32896), np.float32), gptq_damp=0.01)
    assert e.value.status == B.SERQ_ERR_UNSUPPORTED


def test_peaks_library_exports_and_rejects_bad_arguments():
    """libserq_peaks.so (include/serq_peaks.h): every declared symbol is
    exported, and invalid arguments return -1 before any HIP call."""
    from rank_error_compensated_amd import peaks as PK
    L = PK.lib()
    hdr = open(os.path.join(ROOT, "include", "serq_peaks.h")).read()
    names = set(re.findall(r"^\s*int\s+(serq_peak_\w+)\s*\(", hdr, re.M))
    assert names == {"serq_peak_sink_floats", "serq_peak_wall_khz", "serq_peak_mfma", "serq_peak_read",
                     "serq_peak_copy"}
    for n in names:
        assert hasattr(L, n), n
    vp = ctypes.c_void_p
    assert L.serq_peak_mfma(4, 1, 10, vp(FAKE), vp(FAKE), None) == -1        # unknown kind
    assert L.serq_peak_mfma(0, 3, 10, vp(FAKE), vp(FAKE), None) == -1        # waves per SIMD
    assert L.serq_peak_mfma(0, 1, 0, vp(FAKE), vp(FAKE), None) == -1         # iterations
    assert L.serq_peak_mfma(0, 1, 10, None, vp(FAKE), None) == -1
    assert L.serq_peak_read(None, 1 << 20, vp(FAKE), None) == -1
    assert L.serq_peak_read(vp(FAKE), 100, vp(FAKE), None) == -1             # not a multiple of 16
    assert L.serq_peak_copy(vp(FAKE + 4), vp(FAKE), 1 << 20, None) == -1     # misaligned
