"""L2QER comparator, host side: the offline entry points against the oracle
(bit for bit) and the argument checks of the device entry points, which all
run before any HIP call.  No GPU needed."""
import ctypes

import numpy as np
import pytest

from oracle import serq_oracle as O
from rank_error_compensated_amd import binding as B
from rank_error_compensated_amd import workloads as WL

FAKE = 1 << 20      # a 16-byte aligned non-null address that is never dereferenced


@pytest.fixture(scope="module")
def lib():
    return B.lib()


def _case(seed=21, d_in=256, d_out=48):
    return WL.random_case(seed, 8, d_in, d_out, 0, "int4", n_out=4, factor=40.0, n_cal=24)


@pytest.mark.parametrize("fmt", ["int4", "w4a8", "mxfp4", "mxw4a8"])
def test_weight_error_matches_oracle_bit_exactly(fmt):
    c = _case()
    L = B.serq_query_layout(c.d_in, c.d_out, 32, fmt)
    got = B.serq_weight_error(L, c.W, c.X_cal)
    want = O.weight_error(O.prepare(c.W, c.X_cal, 0, fmt))
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("k", [1, 31, 128, 200, 256])
def test_l2qer_prepare_matches_oracle_bit_exactly(k):
    c = _case(seed=22 + k, d_in=384, d_out=272)
    L = B.serq_query_layout(c.d_in, c.d_out, 0, "int4")
    E = O.weight_error(O.prepare(c.W, c.X_cal, 0, "int4"))
    L1, L2 = O.l2qer_factors(E, k)
    got = B.serq_l2qer_prepare(L, L1, L2)
    want = O.packed_l2qer(O.l2qer_prepare(L1, L2))
    for name in ("l1q", "l1scale", "l2q", "l2scale"):
        np.testing.assert_array_equal(got[name], want[name], err_msg=name)


@pytest.mark.parametrize("k", [32, 96, 128])
def test_l2qer_prepare_mx_matches_oracle_bit_exactly(k):
    """MXFP4 factors: E2M1 codes and E8M0 per 32 along each column, packed
    as an MXFP4 d_in -> k_pad layer (L1) and an MXFP4 Q(R) (L2)."""
    c = _case(seed=40 + k, d_in=640, d_out=272)
    L = B.serq_query_layout(c.d_in, c.d_out, 0, "mxfp4")
    E = O.weight_error(O.prepare(c.W, c.X_cal, 0, "mxfp4"))
    L1, L2 = O.l2qer_factors(E, k)
    got = B.serq_l2qer_prepare(L, L1, L2)
    want = O.packed_l2qer(O.l2qer_prepare_mx(L1, L2))
    for name in ("l1q", "l1scale", "l2q", "l2scale"):
        np.testing.assert_array_equal(got[name], want[name], err_msg=name)


def test_l2qer_sizes_and_offline_errors():
    L = B.serq_query_layout(512, 64, 0, "int4")
    assert B.serq_l2qer_sizes(L, 100) == (128 * 256, 8 * 128, 64 * 64, 8 * 64)
    assert B.serq_l2qer_sizes(L, 129) == (256 * 256, 8 * 256, 64 * 128, 8 * 64)
    for k in (0, 257, -3):
        with pytest.raises(B.SerqError) as e:
            B.serq_l2qer_sizes(L, k)
        assert e.value.status == B.SERQ_ERR_SHAPE
    for fmt, r in (("w4a8", 0), ("mxw4a8", 32)):
        with pytest.raises(B.SerqError) as e:
            B.serq_l2qer_sizes(B.serq_query_layout(512, 64, r, fmt), 32)
        assert e.value.status == B.SERQ_ERR_UNSUPPORTED
    Lm = B.serq_query_layout(640, 64, 0, "mxfp4")       # 5 K steps of L1: two E8M0 groups a row
    assert B.serq_l2qer_sizes(Lm, 96) == (128 * 320, 128 * 32, 64 * 64, 64 * 16)
    for k in (16, 100, 160):
        with pytest.raises(B.SerqError) as e:
            B.serq_l2qer_sizes(Lm, k)
        assert e.value.status == B.SERQ_ERR_SHAPE


def test_l2qer_device_entry_points_reject_bad_arguments_before_any_hip_call(lib):
    L = B.serq_query_layout(512, 64, 0, "int4")
    lp = ctypes.byref(L)
    need = lib.serq_l2qer_workspace_bytes(lp, 256, 128)
    assert need > 0 and lib.serq_l2qer_workspace_bytes(lp, 256, 0) == 0
    lin = lib.serq_l2qer_linear
    # null pointers, bad k, M < 1, unknown dtype
    assert lin(lp, 128, None, 0, 256, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == B.SERQ_ERR_INVALID_ARG
    assert lin(lp, 0, FAKE, 0, 256, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == B.SERQ_ERR_SHAPE
    assert lin(lp, 128, FAKE, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == B.SERQ_ERR_SHAPE
    assert lin(lp, 128, FAKE, 7, 256, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == B.SERQ_ERR_INVALID_ARG
    # undersized workspace, misaligned buffers
    assert lin(lp, 128, FAKE, 0, 256, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == B.SERQ_ERR_BUFFER
    assert lin(lp, 128, FAKE, 0, 256, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 8, FAKE, need, None) == B.SERQ_ERR_INVALID_ARG
    # outside the large-tile envelope: 128 tokens or fewer
    small = lib.serq_l2qer_workspace_bytes(lp, 128, 128)
    assert lin(lp, 128, FAKE, 0, 128, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, small, None) == B.SERQ_ERR_UNSUPPORTED
    linq = lib.serq_l2qer_linear_q
    assert linq(lp, 128, FAKE, FAKE, 100, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == B.SERQ_ERR_UNSUPPORTED
    assert linq(lp, 128, FAKE, FAKE, 256, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, None) == B.SERQ_ERR_INVALID_ARG
    # a non-INT4 layer
    Lw = B.serq_query_layout(512, 64, 0, "w4a8")
    assert linq(ctypes.byref(Lw), 128, FAKE, FAKE, 256, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == B.SERQ_ERR_UNSUPPORTED
    inter = lib.serq_l2qer_intermediate
    assert inter(lp, 128, FAKE, FAKE, 256, FAKE, FAKE, None, None, FAKE, None) == B.SERQ_ERR_INVALID_ARG
    assert inter(lp, 128, FAKE, FAKE, 256, FAKE, FAKE, FAKE + 4, FAKE, FAKE, None) == B.SERQ_ERR_INVALID_ARG
    assert inter(lp, 300, FAKE, FAKE, 256, FAKE, FAKE, None, FAKE, FAKE, None) == B.SERQ_ERR_SHAPE
    assert lib.serq_last_error()


def test_l2qer_mx_intermediate_rejects_activations_past_2_gib(lib):
    """The buffer-resource kernels address 32-bit offsets and mark lanes past a
    buffer with offset 2^31: activations of 2 GiB or more are refused before
    any HIP call."""
    L = B.serq_query_layout(16384, 64, 0, "mxfp4")
    M = (1 << 31) // (16384 // 2)
    st = lib.serq_l2qer_intermediate(ctypes.byref(L), 128, FAKE, FAKE, M, FAKE, FAKE, None, FAKE, FAKE, None)
    assert st == B.SERQ_ERR_UNSUPPORTED
    assert b"2 GiB" in lib.serq_last_error()
