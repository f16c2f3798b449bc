"""Pins for the CPU oracle: each test checks it against something other than
itself -- hand-worked vectors, exact rational arithmetic, rounding-error
bounds, algebraic identities, brute force on tiny shapes, a second
independent formulation.  No GPU needed."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import serq_oracle as O
from rank_error_compensated_amd import workloads as WL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- quantizer

@pytest.mark.parametrize("case", _load("quantizer_vectors.json")["cases"], ids=lambda c: c["note"][:30])
def test_quantizer_hand_vectors(case):
    x = np.array([case["x"]], np.float32)
    q, s = O.sym_quant(x, case["n_bits"], axis=1)
    assert s[0] == np.float32(case["s"])
    assert q[0].tolist() == case["q"]


def _exact_rne(fr: Fraction) -> int:
    fl = math.floor(fr)
    d = fr - fl
    if d > Fraction(1, 2):
        return fl + 1
    if d < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


@pytest.mark.parametrize("n_bits", [4, 8])
def test_quantizer_against_exact_rationals(n_bits):
    """Codes equal round-half-even of the exact rational x / s, except where
    the exact quotient lies within one fp32 ulp of a half-integer (there the
    fp32 quotient may land on either side and both codes are accepted)."""
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((40, 64)) * rng.uniform(0.01, 30, (40, 1))).astype(np.float32)
    x[3, 5] *= 60.0                       # an outlier row
    x[11] = 0.0                           # an all-zero row
    q, s = O.sym_quant(x, n_bits, axis=1)
    Q = 2 ** (n_bits - 1) - 1
    for m in range(x.shape[0]):
        amax = max(abs(Fraction(float(v))) for v in x[m])
        assert Fraction(float(s[m])) == Fraction(float(np.float32(float(amax) / Q))) or amax == 0
        if s[m] == 0:
            assert np.all(q[m] == 0)
            continue
        S = Fraction(float(s[m]))
        for k in range(x.shape[1]):
            ex = Fraction(float(x[m, k])) / S
            want = max(-Q, min(Q, _exact_rne(ex)))
            if want != q[m, k]:
                near = abs(abs(ex - math.floor(ex)) - Fraction(1, 2)) < Fraction(2, 1) ** -20 * max(1, abs(ex))
                assert near, (m, k, float(ex), int(q[m, k]), want)


# ---------------------------------------------------------------- MX codec

@pytest.mark.parametrize("case", _load("mx_vectors.json")["cases"], ids=lambda c: c["note"][:30])
def test_mx_hand_vectors(case):
    x = np.zeros((1, 32), np.float32)
    x[0, : len(case["x"])] = case["x"]
    codes, e8 = O.mx_quant(x, axis=1)
    assert e8.shape == (1, 1) and int(e8[0, 0]) == case["e8m0"]
    # "v" lists the E2M1 element values (before the block scale)
    assert O.e2m1_value(codes)[0, : len(case["v"])].tolist() == case["v"]
    xd = O.mx_dequant(codes, e8, axis=1)[0, : len(case["v"])]
    assert xd.tolist() == [math.ldexp(v, case["e8m0"] - 127) for v in case["v"]]


def _e2m1_closed_form(v):
    """Round to a float with 1 mantissa bit: step 0.5 below 2, 1 in [2, 4),
    2 in [4, 8), ties to even multiples of the step; saturate at 6."""
    mag = np.abs(v)
    step = np.where(mag < 2, 0.5, np.where(mag < 4, 1.0, 2.0))
    r = np.rint(mag / step) * step
    return np.copysign(np.minimum(r, 6.0), v)


def test_e2m1_against_closed_form():
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.uniform(-8, 8, 20000), np.arange(-32, 33) / 4.0])
    got = O.e2m1_value(O.e2m1_code(v))
    np.testing.assert_array_equal(got, _e2m1_closed_form(v))


def test_mx_scale_exponent_from_fp32_bits():
    rng = np.random.default_rng(4)
    a = np.abs(rng.standard_normal(5000) * 10.0 ** rng.integers(-6, 6, 5000)).astype(np.float32)
    a = a[a > np.float32(1e-30)]
    a = np.concatenate([a, np.ldexp(np.float32(1), np.arange(-20, 20)).astype(np.float32)])
    bits = a.view(np.uint32)
    floor_log2 = ((bits >> 23) & 0xFF).astype(np.int64) - 127
    np.testing.assert_array_equal(O.mx_scale_exponent(a), floor_log2 - 2)


def test_mx_blocks_reconstruct_within_half_step():
    """Every element is within half of its local E2M1 step (times the block
    scale) of its input, unless it saturates at 6 -- which only the block
    maximum can reach within 2^e * 8."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((8, 256)) * 3).astype(np.float32)
    codes, e8 = O.mx_quant(x, axis=1)
    xd = O.mx_dequant(codes, e8, axis=1)
    scale = np.repeat(np.ldexp(1.0, e8.astype(np.int64) - 127), 32, axis=1)
    v = np.abs(x) / scale
    step = np.where(v < 2, 0.5, np.where(v < 4, 1.0, 2.0))
    assert np.all(v < 8)
    allowed = np.maximum(step / 2, v - 6.0)          # saturation above 6
    assert np.all(np.abs(xd - x) <= allowed * scale + 1e-12)
    assert np.any(v > 6)                             # the case is exercised


# ---------------------------------------------------------------- SAF + permutation

def test_saf_identity_in_fp64():
    """X . W == (X diag(s)^-1 P^T)(P diag(s) W) up to the two fp32 roundings
    of each operand: |diff| <= 2.5e-7 * (|X| @ |W|) elementwise."""
    c = WL.random_case(11, 24, 256, 96, 16, "int4", n_out=5, factor=50.0, n_cal=64)
    s = O.saf_scales(c.W, c.X_cal)
    perm = O.saliency_perm(s)
    Xh = O.flatten_acts(c.X, s, perm).astype(np.float64)
    Wh = O.flatten_weights(c.W, s, perm).astype(np.float64)
    X, W = c.X.astype(np.float64), c.W.astype(np.float64)
    bound = 2.5e-7 * (np.abs(X) @ np.abs(W)) + 1e-30
    assert np.all(np.abs(Xh @ Wh - X @ W) <= bound)
    # a wrong permutation of either side is caught
    assert not np.all(np.abs(Xh[:, ::-1] @ Wh - X @ W) <= bound)


def test_saf_balances_channel_maxima():
    """With alpha = 1/2 the flattened calibration maximum and the flattened
    weight-row maximum of every channel are both sqrt(max|X_j| * max|W_j|)."""
    c = WL.random_case(12, 8, 128, 64, 0, "int4", n_out=4, factor=40.0, n_cal=32)
    s = O.saf_scales(c.W, c.X_cal)
    ax = np.abs(c.X_cal).max(0).astype(np.float64)
    aw = np.abs(c.W).max(1).astype(np.float64)
    ax_f = ax / s
    aw_f = aw * s
    np.testing.assert_allclose(ax_f, np.sqrt(ax * aw), rtol=3e-7)
    np.testing.assert_allclose(aw_f, np.sqrt(ax * aw), rtol=3e-7)


def test_saf_zero_channels_get_unit_scale():
    W = np.ones((4, 3), np.float32)
    W[2] = 0
    Xc = np.ones((5, 4), np.float32)
    Xc[:, 1] = 0
    assert O.saf_scales(W, Xc).tolist() == [1.0, 1.0, 1.0, 1.0]


def test_saliency_order_is_descending_and_stable():
    s = np.array([1.0, 3.0, 2.0, 3.0, 0.5, 2.0], np.float32)
    assert O.saliency_perm(s).tolist() == [1, 3, 2, 5, 0, 4]
    rng = np.random.default_rng(1)
    s = rng.integers(0, 5, 1000).astype(np.float32)
    p = O.saliency_perm(s)
    assert sorted(p.tolist()) == list(range(1000))
    sp = s[p]
    assert np.all(sp[:-1] >= sp[1:])
    for v in np.unique(s):                # ties keep the original order
        idx = p[sp == v]
        assert np.all(np.diff(idx) > 0)


# ---------------------------------------------------------------- residual R

@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
def test_salient_rows_decompose_exactly(fmt):
    """W-tilde_s = Q(W-tilde_s) + R holds exactly: R is an exact fp32
    difference (Sterbenz) for INT, and exactly representable for MX."""
    c = WL.random_case(13, 8, 256, 64, 64, fmt, n_out=5, factor=40.0, n_cal=32)
    p = O.prepare(c.W, c.X_cal, c.r, fmt)
    lhs = p["D"].astype(np.float64) + p["R"].astype(np.float64)
    np.testing.assert_array_equal(lhs, p["W_hat"][: c.r].astype(np.float64))
    if fmt == "int4":
        assert np.all(np.abs(p["R"]) <= p["sw"][None, :] / 2 * (1 + 1e-6))


def test_full_rank_residual_reconstruction_bound():
    """r = d_in: every row is salient; after the residual the weight error is
    at most sR/2 <= sw/28 per channel."""
    c = WL.random_case(14, 4, 128, 48, 128, "int4", n_out=3, factor=40.0, n_cal=16)
    p = O.prepare(c.W, c.X_cal, c.r, "int4")
    W_eff = p["D"].astype(np.float64) + p["rq"].astype(np.float64) * p["sR"][None, :]
    err = np.abs(p["W_hat"] - W_eff)
    assert np.all(err <= p["sR"][None, :] / 2 * (1 + 1e-6) + 1e-12)
    assert np.all(p["sR"] <= p["sw"] / 14 * (1 + 1e-6))


# ---------------------------------------------------------------- accumulation

def test_int_matmul_brute_force():
    rng = np.random.default_rng(2)
    a = rng.integers(-127, 128, (5, 64))
    b = rng.integers(-7, 8, (64, 6))
    want = np.zeros((5, 6), np.int64)
    for i in range(5):
        for j in range(6):
            acc = 0
            for k in range(64):
                acc += int(a[i, k]) * int(b[k, j])
            want[i, j] = acc
    np.testing.assert_array_equal(O.int_matmul(a, b), want)
    np.testing.assert_array_equal(O.int_matmul(a, b), a.astype(np.int64) @ b.astype(np.int64))
    np.testing.assert_array_equal(O.int_matmul_naive(a, b), want)


def test_accumulators_fit_int32_at_largest_shape():
    # worst case magnitudes the layer can reach: A8 x 4-bit over d_in = 14336
    assert 127 * 7 * 14336 < 2 ** 31 and 7 * 7 * 14336 < 2 ** 24


# ---------------------------------------------------------------- whole layer

def _error_bound_int(p, xq, sx, X_hat):
    """Rounding bound of the quantized layer against X-hat . W-hat:
    sum_k |x_k| |w_k - w_eff_k| + |x_k - xq_k sx| |w_eff_k|, with the
    effective weight error <= sR/2 on salient rows and sw/2 elsewhere."""
    r = p["r"]
    Xh = np.abs(X_hat.astype(np.float64))
    w_err = np.repeat(p["sw"][None, :].astype(np.float64) / 2, Xh.shape[1], axis=0)
    if r:
        w_err[:r] = p["sR"][None, :] / 2
    W_eff = p["wq"].astype(np.float64) * p["sw"][None, :]
    if r:
        W_eff[:r] = p["D"] + p["rq"].astype(np.float64) * p["sR"][None, :]
    x_err = (sx.astype(np.float64) / 2)[:, None] * np.ones_like(Xh)
    return Xh @ w_err + x_err @ np.abs(W_eff)


@pytest.mark.parametrize("r", [0, 16, 64])
def test_layer_within_quantization_error_bound(r):
    c = WL.random_case(15, 32, 256, 64, r, "int4", n_out=4, factor=40.0, n_cal=64)
    p = O.prepare(c.W, c.X_cal, r, "int4")
    Xh = O.flatten_acts(c.X, p["s"], p["perm"])
    out = O.serq_linear(Xh, p)
    exact = Xh.astype(np.float64) @ p["W_hat"].astype(np.float64)
    bound = _error_bound_int(p, out["xq"], out["xscale"], Xh)
    assert np.all(np.abs(out["Y"] - exact) <= bound * (1 + 1e-5) + 1e-9)
    if r:
        # The residual term sx * sR * A_res reproduces X-tilde_{s,q} . R (the
        # exact salient-row weight error) within R's rounding bound ...
        xs = out["xq"][:, :r].astype(np.float64) * out["xscale"][:, None]
        res_term = out["xscale"][:, None].astype(np.float64) * p["sR"][None, :] * out["A_res"]
        res_bound = np.abs(xs) @ np.full((r, p["sR"].size), 1.0) * p["sR"][None, :] / 2
        assert np.all(np.abs(res_term - xs @ p["R"].astype(np.float64)) <= res_bound * (1 + 1e-6))
        # ... which a residual of the wrong sign does not
        assert not np.all(np.abs(-res_term - xs @ p["R"].astype(np.float64)) <= res_bound * (1 + 1e-6))


def test_rank_zero_is_plain_w4a4_and_main_path_independent_of_r():
    c = WL.random_case(16, 16, 256, 32, 64, "int4", n_out=3, factor=40.0, n_cal=32)
    p0 = O.prepare(c.W, c.X_cal, 0, "int4")
    p64 = O.prepare(c.W, c.X_cal, 64, "int4")
    Xh = O.flatten_acts(c.X, p0["s"], p0["perm"])
    o0, o64 = O.serq_linear(Xh, p0), O.serq_linear(Xh, p64)
    np.testing.assert_array_equal(o0["A_main"], o64["A_main"])
    assert o0["A_res"].shape == (16, 32) and not o0["A_res"].any()
    resid = out_res = o64["xscale"][:, None].astype(np.float64) * p64["sR"][None, :] * o64["A_res"]
    np.testing.assert_allclose(o64["Y"] - out_res, o0["Y"], rtol=0, atol=1e-12 * np.abs(o0["Y"]).max())
    del resid


def test_permutation_consistency_at_rank_zero():
    """At r = 0 the saliency order cannot change any code: accumulators of the
    permuted layer equal those computed in original channel order."""
    c = WL.random_case(17, 12, 128, 40, 0, "int4", n_out=3, factor=40.0, n_cal=32)
    p = O.prepare(c.W, c.X_cal, 0, "int4")
    ident = np.arange(128, dtype=np.int32)
    Wh_id = O.flatten_weights(c.W, p["s"], ident)
    Xh_id = O.flatten_acts(c.X, p["s"], ident)
    wq_id, _ = O.sym_quant(Wh_id, 4, axis=0)
    xq_id, _ = O.sym_quant(Xh_id, 4, axis=1)
    Xh = O.flatten_acts(c.X, p["s"], p["perm"])
    out = O.serq_linear(Xh, p)
    np.testing.assert_array_equal(out["A_main"], O.int_matmul(xq_id, wq_id))


def test_mx_linear_matches_blockwise_formulation():
    """fp64 product of exactly dequantized MX operands equals the block-scaled
    sum  sum_b 2^(ex+ew-254) sum_{k in b} e2m1 * e2m1  (main + residual)."""
    c = WL.random_case(18, 6, 128, 8, 64, "mxfp4", n_out=3, factor=40.0, n_cal=16)
    p = O.prepare(c.W, c.X_cal, 64, "mxfp4")
    Xh = O.flatten_acts(c.X, p["s"], p["perm"])
    out = O.serq_linear(Xh, p)
    xv, wv, rv = O.e2m1_value(out["xq"]), O.e2m1_value(p["wq"]), O.e2m1_value(p["rq"])
    xe, we, re = out["xscale"].astype(int), p["we"].astype(int), p["re"].astype(int)
    Y = np.zeros((6, 8))
    for m in range(6):
        for o in range(8):
            acc = 0.0
            for b in range(128 // 32):
                dot = sum(xv[m, k] * wv[k, o] for k in range(32 * b, 32 * b + 32))
                acc += math.ldexp(float(dot), int(xe[m, b] + we[b, o] - 254))
            for b in range(64 // 32):
                dot = sum(xv[m, k] * rv[k, o] for k in range(32 * b, 32 * b + 32))
                acc += math.ldexp(float(dot), int(xe[m, b] + re[b, o] - 254))
            Y[m, o] = acc
    np.testing.assert_allclose(out["Y"], Y, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O.linear_mx_blocks(out["xq"], out["xscale"], p), Y, rtol=1e-12, atol=1e-12)


def test_residual_reduces_layer_error_on_outlier_data():
    """Sanity trend (not a pin): larger rank never makes the weight
    reconstruction worse on the salient rows."""
    c = WL.random_case(19, 64, 256, 64, 0, "int4", n_out=6, factor=50.0, n_cal=64)
    errs = []
    for r in (0, 16, 64, 128):
        p = O.prepare(c.W, c.X_cal, r, "int4")
        Xh = O.flatten_acts(c.X, p["s"], p["perm"])
        Y = O.serq_linear(Xh, p)["Y"]
        exact = c.X.astype(np.float64) @ c.W.astype(np.float64)
        errs.append(np.linalg.norm(Y - exact) / np.linalg.norm(exact))
    assert errs[-1] < errs[0]


# ---------------------------------------------------------------- storage layout

def test_nibble_packing_round_trip_and_byte_order():
    codes = np.array([[1, -2, 7, -7, 0, -1]], np.int8)
    packed = O.pack_nibbles(codes)
    # element k in byte k/2, low nibble for even k, two's complement
    assert packed.tolist() == [[0xE1, 0x97, 0xF0]]
    np.testing.assert_array_equal(O.unpack_int4(packed), codes)


def test_packed_weights_shapes():
    c = WL.random_case(20, 4, 256, 32, 16, "w4a8", n_out=2, factor=40.0, n_cal=8)
    p = O.prepare(c.W, c.X_cal, 16, "w4a8")
    pk = O.packed_weights(p, tiled=False)
    assert pk["wq"].shape == (32 * 128,) and pk["rq"].shape == (32 * 64,)
    rq = O.unpack_int4(pk["rq"].reshape(32, 64))
    assert not rq[:, 16:].any()
    np.testing.assert_array_equal(rq[:, :16], p["rq"].T)
    tiled = O.packed_weights(p)
    np.testing.assert_array_equal(O.untile_rows(tiled["wq"], 32, 128), pk["wq"].reshape(32, 128))
    np.testing.assert_array_equal(O.untile_rows(tiled["rq"], 32, 64), pk["rq"].reshape(32, 64))


def test_weight_tile_positions():
    """Layout version 3: 1024-byte tiles of 16 rows x 64 bytes, row blocks
    outermost, then 64-byte chunks of K, rows in order inside a tile.  Spot
    positions worked out by hand for a 32 x 128-byte matrix whose byte
    (n, b) holds a distinct value."""
    rows = np.zeros((32, 128), np.uint8)
    val = {}
    for n, b, v in ((0, 0, 1), (0, 63, 2), (0, 64, 3), (1, 0, 4), (15, 127, 5), (16, 0, 6), (17, 65, 7),
                    (31, 127, 8)):
        rows[n, b] = v
        val[v] = (n, b)
    flat = O.tile_rows(rows)
    assert flat.size == 4096
    # tile 0 = rows 0-15, bytes 0-63; tile 1 = rows 0-15, bytes 64-127;
    # tile 2 = rows 16-31, bytes 0-63; tile 3 = rows 16-31, bytes 64-127
    expect = {0: 1, 63: 2, 1024: 3, 64: 4, 1024 + 15 * 64 + 63: 5, 2048: 6, 3072 + 64 + 1: 7, 4095: 8}
    for pos, v in expect.items():
        assert flat[pos] == v, (pos, v, val[v])
    assert np.count_nonzero(flat) == len(expect)
    np.testing.assert_array_equal(O.untile_rows(flat, 32, 128), rows)


def test_mx_scale_group_positions():
    """Layout version 4, MX E8M0 bytes: groups of four K steps (16 bytes of a
    row), zero-padded to whole groups; blocks of 16 rows outermost, then the
    groups, the 16 rows of a block inside a group.  Spot positions worked out
    by hand for a 32-row matrix of 5 K steps (20 bytes a row: two groups, the
    second holding 4 bytes and 12 of padding) whose byte (n, b) is distinct."""
    rows = np.zeros((32, 20), np.uint8)
    for n, b, v in ((0, 0, 1), (0, 15, 2), (0, 16, 3), (1, 0, 4), (15, 19, 5), (16, 0, 6), (17, 17, 7),
                    (31, 19, 8)):
        rows[n, b] = v
    flat = O.tile_scale_rows(rows)
    assert flat.size == 32 * 32
    # block 0: group 0 at 0 (row j at 16 j), group 1 at 256; block 1: group 0
    # at 512, group 1 at 768
    expect = {0: 1, 15: 2, 256: 3, 16: 4, 256 + 15 * 16 + 3: 5, 512: 6, 768 + 16 + 1: 7, 768 + 15 * 16 + 3: 8}
    for pos, v in expect.items():
        assert flat[pos] == v, (pos, v)
    assert np.count_nonzero(flat) == len(expect)
    np.testing.assert_array_equal(O.untile_scale_rows(flat, 32, 20), rows)


def test_mx_packed_weights_are_tiled_codes_and_grouped_scales():
    """MX What_q / Q(R) take the INT4 tile order of their row-major nibbles;
    their E8M0 bytes take the 16-row groups; both round-trip."""
    c = WL.random_case(31, 8, 640, 48, 96, "mxfp4", n_out=3, factor=40.0, n_cal=16)
    p = O.prepare(c.W, c.X_cal, 96, "mxfp4")
    flat, tiled = O.packed_weights(p, tiled=False), O.packed_weights(p)
    np.testing.assert_array_equal(O.untile_rows(tiled["wq"], 48, 320), flat["wq"].reshape(48, 320))
    np.testing.assert_array_equal(O.untile_rows(tiled["rq"], 48, 64), flat["rq"].reshape(48, 64))
    np.testing.assert_array_equal(O.untile_scale_rows(tiled["wscale"], 48, 20), flat["wscale"].reshape(48, 20))
    np.testing.assert_array_equal(O.untile_scale_rows(tiled["rscale"], 48, 4), flat["rscale"].reshape(48, 4))
    assert tiled["wscale"].size == 48 * 32 and tiled["rscale"].size == 48 * 16
    # the row-major E8M0 bytes are the blocks' scales, channel by channel
    np.testing.assert_array_equal(flat["wscale"].reshape(48, 20), p["we"].T)


def test_int4_offset_layout_bytes_and_round_trip():
    codes = np.array([[3, -2, -7, 7, 0, -1]], np.int8)
    # activations: even k two's complement in the high nibble, odd k + 8 low
    assert O.pack_int4_act(codes).tolist() == [[0x36, 0x9F, 0x07]]
    # weights: even k + 8 in the low nibble, odd k two's complement high
    assert O.pack_int4_weight(codes).tolist() == [[0xEB, 0x71, 0xF8]]
    rng = np.random.default_rng(0)
    c = rng.integers(-7, 8, (5, 64)).astype(np.int8)
    np.testing.assert_array_equal(O.unpack_int4_act(O.pack_int4_act(c)), c)
    np.testing.assert_array_equal(O.unpack_int4_weight(O.pack_int4_weight(c)), c)


def test_int4_offset_layout_products_recover_exact_accumulators():
    """The byte-level products the kernels form -- (act & 0xF0) * (wgt & 0x0F)
    + (act & 0x0F) * (wgt & 0xF0) as int8 -- equal 16 * x.w plus 128 times
    (the even-k activation code sum + the odd-k weight code sum)."""
    rng = np.random.default_rng(1)
    x = rng.integers(-7, 8, (6, 256)).astype(np.int8)
    w = rng.integers(-7, 8, (9, 256)).astype(np.int8)          # [out][K]
    a = O.pack_int4_act(x).astype(np.int64)
    b = O.pack_int4_weight(w).astype(np.int64)
    a_hi = np.where((a & 0xF0) >= 128, (a & 0xF0) - 256, a & 0xF0)
    b_hi = np.where((b & 0xF0) >= 128, (b & 0xF0) - 256, b & 0xF0)
    acc = a_hi @ (b & 0x0F).T + (a & 0x0F) @ b_hi.T
    sx = O.act_code_sums(x)[:, -1].astype(np.int64)
    sw = w.astype(np.int64)[:, 1::2].sum(axis=1)
    exact = x.astype(np.int64) @ w.astype(np.int64).T
    np.testing.assert_array_equal(acc, 16 * exact + 128 * (sx[:, None] + sw[None, :]))


def test_act_code_sums_are_running_chunk_sums():
    x = np.zeros((2, 384), np.int8)
    x[0, 0] = 3          # even k, chunk 0
    x[0, 1] = 7          # odd k: not counted
    x[0, 130] = -2       # even k, chunk 1
    x[1, 382] = 5        # even k, chunk 2
    assert O.act_code_sums(x).tolist() == [[3, 1, 1], [0, 0, 5]]


@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
def test_prepare_on_sampled_columns_equals_full_prepare(fmt):
    c = WL.random_case(21, 4, 256, 96, 64, fmt, n_out=3, factor=40.0, n_cal=16)
    full = O.prepare(c.W, c.X_cal, 64, fmt)
    cols = np.array([0, 5, 17, 95])
    part = O.prepare(c.W, c.X_cal, 64, fmt, cols=cols)
    np.testing.assert_array_equal(part["perm"], full["perm"])
    for k in ("W_hat", "wq", "D", "R", "rq"):
        np.testing.assert_array_equal(part[k], full[k][:, cols])
    for k in (("sw", "sR") if fmt == "int4" else ("we", "re")):
        np.testing.assert_array_equal(part[k], full[k][..., cols])


# ---------------------------------------------------------------- producers of X

def test_exp32_against_the_exponential():
    """exp32 is the exponential to within 2 ulp of fp32 over its whole range,
    exact at 0, +inf above 88.5 and 0 below -87 (mathematical closed form)."""
    x = np.concatenate([np.linspace(-87.0, 88.5, 400001), [0.0, 1.0, -1.0, 0.5, 1e-8, -1e-8]]).astype(np.float32)
    e = O.exp32(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    ulps = np.abs(e - ref) / np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert ulps.max() <= 2.0, ulps.max()
    assert O.exp32(np.array([0.0], np.float32))[0] == 1.0
    lim = O.exp32(np.array([88.6, 1000.0, -87.5, -1000.0], np.float32))
    assert np.isinf(lim[0]) and np.isinf(lim[1]) and lim[2] == 0.0 and lim[3] == 0.0


def test_swiglu_identities():
    """silu(0) = 0; silu(g) - silu(-g) = g (sigma(g) + sigma(-g) = 1) to a few
    ulp; silu(g) -> g for large g and -> -0 for very negative g; U scales the
    result; one hand value: silu(1) = 1 / (1 + e^-1) = 0.7310585786..."""
    g = np.linspace(-30, 30, 6001).astype(np.float32)
    one = np.ones_like(g)
    d = O.swiglu(g, one).astype(np.float64) - O.swiglu(-g, one).astype(np.float64)
    assert np.max(np.abs(d - g) / np.maximum(np.abs(g), 1.0)) < 4e-7
    v = O.swiglu(np.array([0.0, 1.0, 100.0, -100.0], np.float32), np.ones(4, np.float32))
    assert v[0] == 0.0 and abs(v[1] - 0.7310585786300049) < 1e-7 and v[2] == 100.0 and v[3] == 0.0
    u = np.float32(3.0)
    np.testing.assert_array_equal(O.swiglu(g, one * u), (O.swiglu(g, one) * u).astype(np.float32))


def test_swiglu_pairs_give_the_unfused_chain():
    """The paired gate|up layout is a column permutation (codes and scales
    per column unchanged), and SwiGLU on a paired output equals the unfused
    chain -- SwiGLU of the separate gate and up outputs, then the next
    layer's flattening (gather by perm, divide by s) -- bit for bit."""
    rng = np.random.default_rng(12)
    d_in, d = 64, 48
    Wg = (rng.standard_normal((d_in, d)) * 0.1).astype(np.float32)
    Wu = (rng.standard_normal((d_in, d)) * 0.1).astype(np.float32)
    perm = rng.permutation(d)
    s = rng.uniform(0.3, 3.0, d).astype(np.float32)
    W = O.swiglu_pairs(Wg, Wu, perm)
    np.testing.assert_array_equal(W[:, 0::2], Wg[:, perm])
    np.testing.assert_array_equal(W[:, 1::2], Wu[:, perm])
    Xc = rng.standard_normal((32, d_in)).astype(np.float32)
    pg = O.prepare(np.concatenate([Wg, Wu], axis=1), Xc, 16, "int4")
    pp = O.prepare(W, Xc, 16, "int4")
    cols = np.empty(2 * d, int)
    cols[0::2], cols[1::2] = perm, d + perm
    np.testing.assert_array_equal(pp["wq"], pg["wq"][:, cols])
    np.testing.assert_array_equal(pp["sw"], pg["sw"][cols])
    X = rng.standard_normal((20, d_in)).astype(np.float32)
    G = (X.astype(np.float64) @ Wg.astype(np.float64)).astype(np.float32)
    U = (X.astype(np.float64) @ Wu.astype(np.float64)).astype(np.float32)
    Y = np.empty((20, 2 * d), np.float32)
    Y[:, 0::2], Y[:, 1::2] = G[:, perm], U[:, perm]
    np.testing.assert_array_equal(O.swiglu_paired(Y, s[perm]), O.flatten_acts(O.swiglu(G, U), s, perm))


def test_rmsnorm_against_definition():
    """RMSNorm matches the fp64 evaluation of h / sqrt(mean(h^2) + eps) * gamma
    within a few fp32 ulp; a constant row c gives c / sqrt(c^2 + eps) * gamma;
    with eps = 0 the output does not change when h is scaled by a power of 2
    (every step scales exactly)."""
    rng = np.random.default_rng(7)
    h = (rng.standard_normal((6, 512)) * rng.uniform(0.01, 50, (6, 1))).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, 512).astype(np.float32)
    eps = 1e-5
    got = O.rmsnorm(h, gamma, eps).astype(np.float64)
    hd = h.astype(np.float64)
    ref = hd / np.sqrt((hd ** 2).mean(axis=1, keepdims=True) + eps) * gamma
    assert np.max(np.abs(got - ref) / np.abs(ref).max()) < 3e-7
    c = np.full((1, 512), 3.0, np.float32)
    np.testing.assert_allclose(O.rmsnorm(c, gamma, eps)[0], 3.0 / np.sqrt(9.0 + eps) * gamma, rtol=3e-7)
    np.testing.assert_array_equal(O.rmsnorm(h * np.float32(8.0), gamma, 0.0), O.rmsnorm(h, gamma, 0.0))


# ---------------------------------------------------------------- MX W4A8 (E4M3 activations)

def test_e4m3_values_and_codes_hand_table():
    """OCP FP8 E4M3 (bias 7, subnormals m/8 * 2^-6, max 0x7E = 448): values of
    hand-picked codes, and rounding of hand-picked inputs, ties to the even
    code, saturation at 448, sign from the input."""
    val = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 / 8 * 2.0 ** -6, 0x08: 2.0 ** -6, 0x38: 1.0, 0x39: 1.125,
           0x3C: 1.5, 0x40: 2.0, 0x77: 240.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in val.items():
        assert O.e4m3_value(np.array([c], np.uint8))[0] == v, hex(c)
    cases = {1.0625: 0x38, 1.1875: 0x3A, 1.07: 0x39, 500.0: 0x7E, 1e6: 0x7E, 464.0: 0x7E,
             2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02, 2.0 ** -6 * 1.0625: 0x08, 240.0: 0x77, 248.0: 0x78,
             -1.0: 0xB8, -0.0: 0x80}
    for v, c in cases.items():
        assert O.e4m3_code(np.array([v]))[0] == c, (v, hex(c), hex(O.e4m3_code(np.array([v]))[0]))


def test_e4m3_round_trip_and_closed_form():
    """Every finite code decodes and re-encodes to itself; random inputs match
    the closed form code = 8 (e + 7) + rint((|v| 2^-e - 1) 8) for normal |v|
    (e = floor(log2 |v|), rint ties to even) and rint(|v| 2^9) below 2^-6."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    np.testing.assert_array_equal(O.e4m3_code(O.e4m3_value(codes)), codes)
    rng = np.random.default_rng(3)
    v = np.abs(rng.standard_normal(20000)) * np.exp2(rng.uniform(-12, 9, 20000))
    v = np.concatenate([v, np.arange(0, 512) / 512.0 * 2.0 ** -6])
    _, e = np.frexp(v)
    e = e - 1
    normal = np.rint((v / np.exp2(e) - 1.0) * 8.0) + 8 * (e + 7)
    sub = np.rint(v * 2.0 ** 9)
    want = np.minimum(np.where(v < 2.0 ** -6, sub, normal), 126).astype(np.uint8)
    np.testing.assert_array_equal(O.e4m3_code(v), want)


def test_mx_w4a8_scale_and_block_bound():
    """Shared exponent floor(log2 amax) - 8: a block whose amax is 448 gets
    E8M0 127 and is represented exactly; every element lands within half an
    E4M3 step of its scaled value (or at 448 when it saturates)."""
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((3, 128)) * 3).astype(np.float32)
    x[0, :32] = 0.0
    x[0, 0] = 448.0
    q, e = O.quant_act(x, O.MXW4A8)
    assert e[0, 0] == 127 and O.e4m3_value(q[0, :1])[0] == 448.0
    deq = O.mx_dequant(q, e, axis=1, elem="e4m3")
    scale = np.repeat(np.ldexp(1.0, e.astype(np.int64) - 127), 32, axis=1)
    v = x / scale
    step = np.where(np.abs(v) < 2.0 ** -6, 2.0 ** -9, np.exp2(np.floor(np.log2(np.maximum(np.abs(v), 1e-30)))) / 8)
    err = np.abs(deq / scale - v)
    assert np.all((err <= step / 2 + 1e-12) | (np.abs(v) > 448))


def test_mx_w4a8_linear_blockwise():
    """The MX W4A8 layer equals the block-by-block sum of E4M3 x E2M1 products
    times both block scales (brute force on a tiny case), plus the residual."""
    c = WL.random_case(23, 3, 128, 16, 32, "mxfp4", n_out=2, factor=30.0, n_cal=8)
    p = O.prepare(c.W, c.X_cal, 32, O.MXW4A8)
    Xh = O.flatten_acts(c.X, p["s"], p["perm"])
    xq, xe = O.quant_act(Xh, O.MXW4A8)
    Y = O.linear_mx(xq, xe, p)
    want = np.zeros((3, 16))
    for m in range(3):
        for o in range(16):
            acc = 0.0
            for b in range(4):
                for k in range(32 * b, 32 * b + 32):
                    acc += (O.e4m3_value(xq[m, k]) * 2.0 ** (int(xe[m, b]) - 127)
                            * O.e2m1_value(p["wq"][k, o]) * 2.0 ** (int(p["we"][b, o]) - 127))
            for k in range(32):
                acc += (O.e4m3_value(xq[m, k]) * 2.0 ** (int(xe[m, k // 32]) - 127)
                        * O.e2m1_value(p["rq"][k, o]) * 2.0 ** (int(p["re"][k // 32, o]) - 127))
            want[m, o] = acc
    np.testing.assert_allclose(Y, want, rtol=0, atol=1e-12 * np.abs(want).max())
    np.testing.assert_allclose(O.linear_mx_blocks(xq, xe, p), want, rtol=0, atol=1e-12 * np.abs(want).max())


# ---------------------------------------------------------------- L2QER comparator

def _l2qer_case(seed=11, M=12, d_in=256, d_out=48, k=32):
    c = WL.random_case(seed, M, d_in, d_out, 0, "int4", n_out=3, factor=30.0, n_cal=16)
    p = O.prepare(c.W, c.X_cal, 0, "int4")
    X = O.flatten_acts(c.X, p["s"], p["perm"])
    xq, sx = O.quant_act(X, "int4")
    return c, p, X, xq, sx, k


def test_weight_error_is_bounded_by_half_a_step_and_zero_on_the_grid():
    """Round to nearest leaves at most half a quantization step per element;
    a column whose values are exact multiples of its step has no error."""
    _, p, _, _, _, _ = _l2qer_case()
    E = O.weight_error(p)
    step = p["sw"].astype(np.float64)
    assert np.all(np.abs(E) <= step[None, :] * 0.5 * (1 + 1e-6) + 1e-12)
    assert np.abs(E).max() > 0.1 * step.max()            # not trivially zero
    W_hat = np.array([[1.75, 0.5], [-0.75, 0.3], [0.5, -0.05], [0.0, 0.07]], np.float32)
    wq, sw = O.sym_quant(W_hat, 4, axis=0)
    E2 = O.weight_error({"fmt": "int4", "W_hat": W_hat, "wq": wq, "sw": sw})
    assert sw[0] == np.float32(0.25)                     # 1.75 / 7, exact
    assert np.all(E2[:, 0] == 0)                         # 7, -3, 2, 0 steps exactly
    assert np.any(E2[:, 1] != 0)


def test_l2qer_factors_eckart_young_and_balanced_split():
    """The rank-k factors leave exactly the energy of the discarded singular
    values (eigenvalues of E^T E from an independent routine), and the split
    gives both factors sqrt(sigma_i) norms."""
    _, p, _, _, _, k = _l2qer_case()
    E = O.weight_error(p).astype(np.float64)
    L1, L2 = O.l2qer_factors(E, k)
    ev = np.sort(np.linalg.eigvalsh(E.T @ E))[::-1]       # sigma^2, descending
    resid = np.linalg.norm(E - L1.astype(np.float64) @ L2.astype(np.float64)) ** 2
    np.testing.assert_allclose(resid, ev[k:].sum(), rtol=1e-4)
    n1 = np.linalg.norm(L1.astype(np.float64), axis=0)
    n2 = np.linalg.norm(L2.astype(np.float64), axis=1)
    np.testing.assert_allclose(n1, n2, rtol=1e-5)
    np.testing.assert_allclose(n1 ** 4, ev[:k], rtol=1e-4)
    full = min(E.shape)
    A, B = O.l2qer_factors(E, full)
    np.testing.assert_allclose(A.astype(np.float64) @ B.astype(np.float64), E, atol=1e-6 * np.abs(E).max())


def test_l2qer_intermediate_brute_force():
    """T by explicit loops over a tiny case: the integer product, then the
    two fp32 products in the stated order."""
    rng = np.random.default_rng(3)
    xq = rng.integers(-7, 8, (3, 8)).astype(np.int8)
    l1q = rng.integers(-7, 8, (8, 4)).astype(np.int8)
    sx = rng.uniform(0.01, 1, 3).astype(np.float32)
    sl1 = rng.uniform(0.01, 1, 4).astype(np.float32)
    T = O.l2qer_intermediate(xq, sx, {"l1q": l1q, "sl1": sl1})
    for m in range(3):
        for j in range(4):
            a = 0
            for kk in range(8):
                a += int(xq[m, kk]) * int(l1q[kk, j])
            want = np.float32(sx[m]) * np.float32(np.float32(sl1[j]) * np.float32(a))
            assert T[m, j] == want


def test_l2qer_reconstructs_the_weight_error():
    """The comparator exists to cancel quantization error: its output is much
    closer to X-hat . W-hat than the main path alone (a sign error, a
    transposed factor or a dropped scale all break this), and with an error
    that vanishes it is the main path exactly."""
    _, p, X, xq, sx, k = _l2qer_case(M=32, d_out=64)
    ref = X.astype(np.float64) @ p["W_hat"].astype(np.float64)
    main = O.linear_int(xq, sx, p)[0]
    fac = O.l2qer_prepare(*O.l2qer_factors(O.weight_error(p), k))
    o = O.l2qer_linear(xq, sx, p, fac)
    e_main, e_l2 = np.abs(main - ref).mean(), np.abs(o["Y"] - ref).mean()
    assert e_l2 < 0.85 * e_main, (e_l2, e_main)
    zero = O.l2qer_prepare(np.zeros((p["W_hat"].shape[0], 8), np.float32), np.zeros((8, 64), np.float32))
    np.testing.assert_array_equal(O.l2qer_linear(xq, sx, p, zero)["Y"], main)


def test_packed_l2qer_round_trips():
    _, p, _, _, _, k = _l2qer_case()
    fac = O.l2qer_prepare(*O.l2qer_factors(O.weight_error(p), k))
    pk = O.packed_l2qer(fac)
    d_in, d_out, kp = p["W_hat"].shape[0], p["W_hat"].shape[1], O.r_padded(k)
    l1 = O.unpack_int4_weight(O.untile_rows(pk["l1q"], kp, d_in // 2)).T
    np.testing.assert_array_equal(l1[:, :k], fac["l1q"])
    assert np.all(l1[:, k:] == 0)
    l2 = O.unpack_int4_weight(O.untile_rows(pk["l2q"], d_out, kp // 2)).T
    np.testing.assert_array_equal(l2[:k], fac["l2q"])
    s1 = pk["l1scale"][: 4 * kp].view(np.float32)
    np.testing.assert_array_equal(s1[:k], fac["sl1"])
    assert np.all(s1[k:] == 0)


def _l2qer_mx_case(seed=17, M=12, d_in=256, d_out=48, k=32):
    c = WL.random_case(seed, M, d_in, d_out, 0, "mxfp4", n_out=3, factor=30.0, n_cal=16)
    p = O.prepare(c.W, c.X_cal, 0, "mxfp4")
    X = O.flatten_acts(c.X, p["s"], p["perm"])
    xq, xe = O.quant_act(X, "mxfp4")
    return c, p, X, xq, xe, k


def test_mx_weight_error_bounds_and_zero_on_the_grid():
    """MX round to nearest: |E| is at most half the widest grid step of its
    block (2 x 2^e, between 4 and 6) -- or 2 x 2^e where a value above 6
    saturates -- and a block of exact grid values has no error."""
    _, p, _, _, _, _ = _l2qer_mx_case()
    E = O.weight_error(p)
    scale = np.repeat(np.ldexp(1.0, p["we"].astype(np.int64) - 127), 32, axis=0)
    assert np.all(np.abs(E) <= 2.0 * scale + 1e-12)
    assert np.abs(E).max() > 0.05 * scale.max()
    W_hat = np.zeros((32, 2), np.float32)
    W_hat[:8, 0] = [6, 4, -3, 2, 1.5, -1, 0.5, 0]          # on the grid at scale 2^0
    W_hat[:8, 1] = [6, 4, -3, 2, 1.5, -1, 0.5, 0.3]
    wq, we = O.mx_quant(W_hat, axis=0)
    E2 = O.weight_error({"fmt": "mxfp4", "W_hat": W_hat, "wq": wq, "we": we})
    assert np.all(E2[:, 0] == 0) and E2[7, 1] != 0


def test_l2qer_mx_intermediate_is_the_exact_block_sum_rounded_once():
    """T by exact rational arithmetic on a tiny case: every block term and
    their sum exactly (Fractions), then one rounding to fp32."""
    from fractions import Fraction
    rng = np.random.default_rng(5)
    xq = rng.integers(0, 16, (3, 64)).astype(np.uint8)
    l1q = rng.integers(0, 16, (64, 4)).astype(np.uint8)
    xe = rng.integers(120, 135, (3, 2)).astype(np.uint8)
    l1e = rng.integers(110, 130, (2, 4)).astype(np.uint8)
    T = O.l2qer_intermediate_mx(xq, xe, {"l1q": l1q, "l1e": l1e})
    for m in range(3):
        for j in range(4):
            acc = Fraction(0)
            for kk in range(64):
                b = kk // 32
                acc += (Fraction(O.e2m1_value(xq[m, kk]).item()) * Fraction(O.e2m1_value(l1q[kk, j]).item())
                        * Fraction(2) ** (int(xe[m, b]) + int(l1e[b, j]) - 254))
            assert Fraction(float(acc)) == acc                     # the exact sum is an fp64 value
            assert T[m, j] == np.float32(float(acc))


def test_l2qer_mx_reconstructs_the_weight_error():
    """In MXFP4 too the comparator's output is much closer to X-hat . W-hat
    than the main path alone, and zero factors leave the main path."""
    c, p, X, xq, xe, k = _l2qer_mx_case(M=32, d_out=64)
    ref = X.astype(np.float64) @ p["W_hat"].astype(np.float64)
    main = O.linear_mx(xq, xe, p)
    fac = O.l2qer_prepare_mx(*O.l2qer_factors(O.weight_error(p), k))
    o = O.l2qer_linear_mx(xq, xe, p, fac)
    e_main, e_l2 = np.abs(main - ref).mean(), np.abs(o["Y"] - ref).mean()
    assert e_l2 < 0.9 * e_main, (e_l2, e_main)
    zero = O.l2qer_prepare_mx(np.zeros((p["W_hat"].shape[0], 32), np.float32), np.zeros((32, 64), np.float32))
    np.testing.assert_array_equal(O.l2qer_linear_mx(xq, xe, p, zero)["Y"], main)


def test_packed_l2qer_mx_round_trips():
    _, p, _, _, _, k = _l2qer_mx_case()
    fac = O.l2qer_prepare_mx(*O.l2qer_factors(O.weight_error(p), k))
    pk = O.packed_l2qer(fac)
    d_in, d_out, kp = p["W_hat"].shape[0], p["W_hat"].shape[1], O.r_padded(k)
    l1 = O.untile_rows(pk["l1q"], kp, d_in // 2)
    np.testing.assert_array_equal(l1[:k], O.pack_nibbles(fac["l1q"].T))
    assert np.all(l1[k:] == 0)
    e1 = O.untile_scale_rows(pk["l1scale"], kp, d_in // 32)
    np.testing.assert_array_equal(e1[:k], fac["l1e"].T)
    assert np.all(e1[k:] == 127)
    l2 = O.untile_rows(pk["l2q"], d_out, kp // 2)
    np.testing.assert_array_equal(l2[:, : k // 2], O.pack_nibbles(fac["l2q"].T))
    e2 = O.untile_scale_rows(pk["l2scale"], d_out, kp // 32)
    np.testing.assert_array_equal(e2[:, : k // 32], fac["l2e"].T)
    assert np.all(e2[:, k // 32:] == 127)


# ---------------------------------------------------------------- GPTQ

def test_gptq_with_a_diagonal_hessian_is_round_to_nearest():
    """Channels that never co-occur give a diagonal Hessian, hence a diagonal
    U: no error propagates and GPTQ is the plain quantizer."""
    rng = np.random.default_rng(8)
    n, d_out = 12, 10
    W = rng.standard_normal((n, d_out)).astype(np.float32)
    Xc = np.diag(rng.uniform(0.5, 3.0, n)).astype(np.float32)       # one channel per row
    _, sw = O.sym_quant(W, 4, axis=0)
    want, _ = O.sym_quant(W, 4, axis=0)
    np.testing.assert_array_equal(O.gptq_codes(W, Xc, sw), want)


def test_gptq_two_rows_closed_form():
    """Two channels, one output: the 2 x 2 inverse and its Cholesky factor by
    hand, then quantize row 0, push its scaled error into row 1, quantize."""
    Xc = np.array([[2.0, 1.5], [0.0, np.sqrt(4.0 - 2.25)]], np.float32)
    XtX = Xc.astype(np.float64).T @ Xc.astype(np.float64)
    a, b, c = XtX[0, 0], XtX[0, 1], XtX[1, 1]
    damp = 0.01 * (2 * a + 2 * c) / 2
    h00, h01, h11 = 2 * a + damp, 2 * b, 2 * c + damp
    det = h00 * h11 - h01 * h01
    i00, i01, i11 = h11 / det, -h01 / det, h00 / det
    u00 = math.sqrt(i00)
    u01 = i01 / u00
    W = np.array([[1.0], [0.1]], np.float32)
    sw = np.array([0.3], np.float32)                                # codes in [-7, 7]
    q0 = float(np.clip(np.rint(np.float32(1.0) / np.float32(0.3)), -7, 7))
    d0 = float(np.float32(q0) * np.float32(0.3))
    w1 = float(np.float32(0.1)) - u01 * (1.0 - d0) / u00           # 0.1 + (h01 / h11) * 0.1
    q1 = float(np.clip(np.rint(np.float32(w1) / np.float32(0.3)), -7, 7))
    got = O.gptq_codes(W, Xc, sw)
    assert (q0, q1) == (3.0, 1.0)
    assert got[0, 0] == q0 and got[1, 0] == q1
    assert q1 != float(np.rint(np.float32(0.1) / np.float32(0.3)))    # the update mattered


def test_gptq_lowers_the_calibration_error_and_keeps_the_salient_rows():
    """GPTQ's purpose: a smaller output error on the calibration activations
    than round to nearest (a sign or index error in the update breaks it),
    for the non-salient rows of What_q and for Q(R) against R; by the
    reading taken here the salient rows, their scales, D and R do not
    change."""
    c = WL.random_case(3, 64, 512, 96, 64, "int4", n_out=6, factor=40.0, n_cal=128)
    pr = O.prepare(c.W, c.X_cal, 64, "int4")
    pg = O.prepare_gptq(c.W, c.X_cal, 64, "int4")
    Xh = O.flatten_acts(c.X_cal, pr["s"], pr["perm"]).astype(np.float64)
    err, err_r = {}, {}
    for name, p in (("rtn", pr), ("gptq", pg)):
        D = p["wq"].astype(np.float64) * p["sw"].astype(np.float64)[None, :]
        err[name] = np.linalg.norm(Xh[:, 64:] @ D[64:] - Xh[:, 64:] @ p["W_hat"][64:].astype(np.float64))
        Rd = p["rq"].astype(np.float64) * p["sR"].astype(np.float64)[None, :]
        err_r[name] = np.linalg.norm(Xh[:, :64] @ (Rd - p["R"].astype(np.float64)))
    assert err["gptq"] < 0.8 * err["rtn"], err
    assert err_r["gptq"] < 0.95 * err_r["rtn"], err_r
    np.testing.assert_array_equal(pg["wq"][:64], pr["wq"][:64])
    for k in ("sw", "R", "sR", "D"):
        np.testing.assert_array_equal(pg[k], pr[k])
    assert np.mean(pg["wq"] != pr["wq"]) > 0.05 and np.mean(pg["rq"] != pr["rq"]) > 0.02


def _pair_hessian_factor(n, i, j):
    """Calibration rows giving channels i and j (adjacent) the 2 x 2 block
    2 [[4, 3], [3, 4]] and every other channel 2; returns (Xc, u_ii, u_ij)
    with the block's inverse and its Cholesky factor worked by hand."""
    Xc = np.zeros((n, n), np.float32)
    Xc[0, i], Xc[0, j] = 2.0, 1.5
    Xc[1, j] = np.sqrt(np.float32(4.0 - 2.25))
    rows = [k for k in range(n) if k not in (i, j)]
    for t, k in enumerate(rows):
        Xc[2 + t, k] = 1.0
    XtX = Xc.astype(np.float64).T @ Xc.astype(np.float64)
    damp = 0.01 * np.mean(2.0 * np.diag(XtX))
    h00, h01, h11 = 2 * XtX[i, i] + damp, 2 * XtX[i, j], 2 * XtX[j, j] + damp
    det = h00 * h11 - h01 * h01
    u00 = math.sqrt(h11 / det)
    return Xc, u00, (-h01 / det) / u00


def e2m1_nearest(v):
    """Nearest E2M1 magnitude by brute force over the grid, ties to the even
    code (grid index), saturating at 6; sign kept."""
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    a = abs(v)
    best = min(range(8), key=lambda k: (abs(a - grid[k]), k % 2))
    return math.copysign(grid[best], v)


def test_gptq_mx_with_a_diagonal_hessian_is_round_to_nearest():
    """A diagonal Hessian propagates nothing: MX GPTQ gives mx_quant's codes
    and E8M0 bytes."""
    rng = np.random.default_rng(18)
    n, d_out = 64, 10
    W = (rng.standard_normal((n, d_out)) * rng.uniform(0.01, 3.0, (n, 1))).astype(np.float32)
    Xc = np.diag(rng.uniform(0.5, 3.0, n)).astype(np.float32)
    codes, e8 = O.gptq_codes_mx(W, Xc)
    want_c, want_e = O.mx_quant(W, axis=0)
    np.testing.assert_array_equal(codes, want_c)
    np.testing.assert_array_equal(e8, want_e)


def test_gptq_mx_two_rows_in_a_group_closed_form():
    """One 32-row group, channels 0 and 1 correlated: the group scale comes
    from the rows as they start (max 0.9 -> 2^-3), row 0 saturates at 6 x
    2^-3, its error moves row 1 by (h01 / h11) x 0.15 (0.1 -> 0.212), and
    row 1's code is the nearest E2M1 of the moved value over the scale
    (1.70 -> 1.5, not the 1.0 of RTN)."""
    n = 32
    Xc, u00, u01 = _pair_hessian_factor(n, 0, 1)
    W = np.full((n, 1), 0.01, np.float32)
    W[0, 0], W[1, 0] = 0.9, 0.1
    codes, e8 = O.gptq_codes_mx(W, Xc)
    assert int(e8[0, 0]) == 127 - 3
    scale = 2.0 ** -3
    d0 = 6.0 * scale
    w1 = float(np.float32(0.1)) - u01 * (float(np.float32(0.9)) - d0) / u00
    q1 = e2m1_nearest(float(np.float32(w1)) / scale)
    assert O.e2m1_value(codes[0, 0]) == 6.0 and O.e2m1_value(codes[1, 0]) == q1
    assert q1 == 1.5 and e2m1_nearest(float(np.float32(0.1)) / scale) == 1.0   # the update mattered
    assert np.all(O.e2m1_value(codes[2:, 0]) == 0.0)                             # 0.08 rounds to 0


def test_gptq_mx_group_scale_follows_the_updated_rows():
    """Channels 31 and 32 correlated across the group boundary: row 31's
    error moves row 32 before group 1 starts, and group 1's E8M0 is taken
    from the moved value (0.45 + 0.15 h01/h11 ~ 0.56: exponent -1 - 2), not
    from the original rows (0.45: -2 - 2) as round to nearest would."""
    n = 64
    Xc, u00, u01 = _pair_hessian_factor(n, 31, 32)
    W = np.full((n, 1), 0.01, np.float32)
    W[31, 0], W[0, 0], W[32, 0] = 0.9, 0.9, 0.45
    codes, e8 = O.gptq_codes_mx(W, Xc)
    w32 = float(np.float32(0.45)) - u01 * (float(np.float32(0.9)) - 0.75) / u00
    assert 0.5 <= w32 < 1.0
    assert int(e8[0, 0]) == 127 - 3 and int(e8[1, 0]) == 127 - 3
    _, rtn_e = O.mx_quant(W, axis=0)
    assert int(rtn_e[1, 0]) == 127 - 4
    assert O.e2m1_value(codes[32, 0]) == e2m1_nearest(float(np.float32(w32)) / 2.0 ** -3)


def test_gptq_mx_lowers_the_calibration_error_and_keeps_the_salient_rows():
    """On activations that share a latent factor (GPTQ's use case) MX GPTQ
    leaves a smaller calibration output error than round to nearest, in the
    non-salient rows and in Q(R) against R; the salient rows, their E8M0, D
    and R do not change."""
    c = WL.correlated_case(WL.random_case(5, 64, 512, 96, 64, "mxfp4", n_out=6, factor=40.0, n_cal=32),
                           n_cal=1024, rank=32, noise=0.3, factor=50, seed=2001)
    pr = O.prepare(c.W, c.X_cal, 64, "mxfp4")
    pg = O.prepare_gptq(c.W, c.X_cal, 64, "mxfp4")
    Xh = O.flatten_acts(c.X_cal, pr["s"], pr["perm"]).astype(np.float64)
    err, err_r = {}, {}
    for name, p in (("rtn", pr), ("gptq", pg)):
        D = O.mx_dequant(p["wq"], p["we"], axis=0)
        err[name] = np.linalg.norm(Xh[:, 64:] @ (D[64:] - p["W_hat"][64:].astype(np.float64)))
        Rd = O.mx_dequant(p["rq"], p["re"], axis=0)
        err_r[name] = np.linalg.norm(Xh[:, :64] @ (Rd - p["R"].astype(np.float64)))
    assert err["gptq"] < 0.9 * err["rtn"], err
    assert err_r["gptq"] < 0.95 * err_r["rtn"], err_r
    np.testing.assert_array_equal(pg["wq"][:64], pr["wq"][:64])
    np.testing.assert_array_equal(pg["we"][:2], pr["we"][:2])
    for k in ("R", "D"):
        np.testing.assert_array_equal(pg[k], pr[k])


def test_gptq_dead_channel_stays_finite():
    c = WL.random_case(4, 32, 256, 32, 32, "int4", n_out=3, factor=40.0, n_cal=64)
    c.X_cal[:, 100:110] = 0.0
    p = O.prepare_gptq(c.W, c.X_cal, 32, "int4")
    assert np.all(np.abs(p["wq"]) <= 7)


def test_gptq_sampled_columns_equal_the_full_run():
    """Output channels are independent under GPTQ (shared Hessian, per-column
    updates and, for MX, per-column group scales): the sampled form equals
    the full form on those columns."""
    c = WL.random_case(6, 16, 256, 64, 32, "int4", n_out=3, factor=40.0, n_cal=64)
    full = O.prepare_gptq(c.W, c.X_cal, 32, "int4")
    cols = np.array([0, 5, 17, 63])
    part = O.prepare_gptq(c.W, c.X_cal, 32, "int4", cols=cols)
    np.testing.assert_array_equal(part["wq"], full["wq"][:, cols])
    fm = O.prepare_gptq(c.W, c.X_cal, 32, "mxfp4")
    pm = O.prepare_gptq(c.W, c.X_cal, 32, "mxfp4", cols=cols)
    np.testing.assert_array_equal(pm["wq"], fm["wq"][:, cols])
    np.testing.assert_array_equal(pm["we"], fm["we"][:, cols])
