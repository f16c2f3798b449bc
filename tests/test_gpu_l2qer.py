"""GPU parity of the L2QER comparator through the C ABI against the oracle.

Bar: the intermediate T (fp32) and its quantization (codes, scales, code
sums) bit-exact; Y within max|dY| <= 1e-5 * max|Y|; the whole-layer entry
point equal to the two-step one bit for bit.  The factors are inputs: both
sides quantize the same fp32 L1, L2 (a truncated SVD of the weight error at
test sizes; at the attention-projection size a randomized range finder of
the same rank, since any factors serve a parity check)."""
import numpy as np
import pytest

from oracle import serq_oracle as O
from rank_error_compensated_amd import binding as B
from rank_error_compensated_amd import workloads as WL

pytestmark = pytest.mark.gpu
TOL = 1e-5


def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    B.lib()
    return torch


def dev(a):
    torch = torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t):
    return t.cpu().numpy()


def _range_factors(E, k, seed=0):
    """Rank-k factors of E by a randomized range finder (two power steps)."""
    rng = np.random.default_rng(seed)
    E64 = E.astype(np.float64)
    Q, _ = np.linalg.qr(E64 @ rng.standard_normal((E.shape[1], k)))
    for _ in range(2):
        Q, _ = np.linalg.qr(E64 @ (E64.T @ Q))
    B_ = Q.T @ E64                                   # k x d_out
    U, S, Vt = np.linalg.svd(B_, full_matrices=False)
    h = np.sqrt(S)
    return ((Q @ U) * h).astype(np.float32), (h[:, None] * Vt).astype(np.float32)


def run_case(c, k, bf16=False, factors=None, rows=None, cols=None):
    torch = torch_cuda()
    M, d_in, d_out = c.M, c.d_in, c.d_out
    L = B.serq_query_layout(d_in, d_out, 0, "int4")
    lp = B.serq_prepare_weights(L, c.W, c.X_cal)
    p = O.prepare(c.W, c.X_cal, 0, "int4", cols=cols)
    E = B.serq_weight_error(L, c.W, c.X_cal)
    L1, L2 = (factors or O.l2qer_factors)(E, k)
    fl = B.serq_l2qer_prepare(L, L1, L2)
    fo = O.l2qer_prepare(L1, L2 if cols is None else L2[:, cols])
    kp = O.r_padded(k)

    X_hat = O.flatten_acts(c.X, lp["s"], lp["perm"])
    Xd = dev(X_hat)
    if bf16:
        Xd = Xd.to(torch.bfloat16)
        X_hat = Xd.float().cpu().numpy()
    xq_o, sx_o = O.quant_act(X_hat, "int4")
    nq, ns = B.serq_act_bytes(M, d_in, "int4")
    xq = torch.empty(nq, dtype=torch.uint8, device="cuda")
    xs = torch.empty(ns, dtype=torch.uint8, device="cuda")
    B.serq_quant_act(Xd, "int4", xq, xs)
    d = {n: dev(lp[n]) for n in ("wq", "wscale")}
    f = {n: dev(fl[n]) for n in ("l1q", "l1scale", "l2q", "l2scale")}

    # the intermediate and its on-the-fly quantization: bit-exact
    T = torch.full((M, kp), np.nan, dtype=torch.float32, device="cuda")
    tq = torch.empty(M * kp // 2, dtype=torch.uint8, device="cuda")
    ts = torch.empty(M * 4 + M * (kp // 128) * 4, dtype=torch.uint8, device="cuda")
    ws = torch.empty(B.serq_l2qer_workspace_bytes(L, M, k), dtype=torch.uint8, device="cuda")
    B.serq_l2qer_intermediate(L, k, xq, xs, M, f["l1q"], f["l1scale"], T, tq, ts)
    torch.cuda.synchronize()
    T_o = np.zeros((M, kp), np.float32)
    T_o[:, :k] = O.l2qer_intermediate(xq_o, sx_o, fo)
    np.testing.assert_array_equal(host(T), T_o)
    want_q, want_s = O.packed_acts(*O.quant_act(T_o, "int4"), "int4")
    np.testing.assert_array_equal(host(tq).reshape(M, -1), want_q.reshape(M, -1))
    np.testing.assert_array_equal(host(ts), want_s)

    # the layer output
    Y = torch.full((M, d_out), np.nan, dtype=torch.float32, device="cuda")
    B.serq_l2qer_linear_q(L, k, xq, xs, M, d["wq"], d["wscale"], tq, ts, f["l2q"], f["l2scale"], Y)
    torch.cuda.synchronize()
    rsel = np.arange(M) if rows is None else rows
    csel = slice(None) if cols is None else cols
    Yo = O.l2qer_linear(xq_o[rsel], sx_o[rsel], p, fo)["Y"]
    Yg = host(Y)[rsel][:, csel]
    assert np.all(np.isfinite(Yg))
    err, scale = np.abs(Yg - Yo).max(), np.abs(Yo).max()
    assert err <= TOL * scale, (err, scale)

    # the whole layer in one call: the same bytes
    Y2 = torch.full((M, d_out), np.nan, dtype=torch.float32, device="cuda")
    B.serq_l2qer_linear(L, k, Xd, d["wq"], d["wscale"], f["l1q"], f["l1scale"], f["l2q"], f["l2scale"], Y2, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(Y2), host(Y))
    return err / scale


SHAPES = [  # M, d_in, d_out, k -- ragged M, k below / at / between the 128 pads, K split remainders
    (129, 256, 48, 16), (200, 512, 144, 128), (300, 1024, 272, 200), (257, 768, 320, 256), (384, 1280, 128, 100),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_l2qer_small_shapes(shape):
    M, d_in, d_out, k = shape
    c = WL.random_case(sum(shape), M, d_in, d_out, 0, "int4", n_out=4, factor=50.0, n_cal=64)
    run_case(c, k)


def test_l2qer_bf16_input():
    c = WL.random_case(7, 260, 512, 96, 0, "int4", n_out=4, factor=50.0, n_cal=32)
    run_case(c, 64, bf16=True)


def test_l2qer_rejects_small_batches():
    torch = torch_cuda()
    L = B.serq_query_layout(256, 48, 0, "int4")
    with pytest.raises(B.SerqError) as e:
        B.serq_l2qer_linear_q(L, 16, *(torch.empty(1024, dtype=torch.uint8, device="cuda"),) * 2, 64,
                              *(torch.empty(1024, dtype=torch.uint8, device="cuda"),) * 6,
                              torch.empty(64 * 48, dtype=torch.float32, device="cuda"))
    assert e.value.status == B.SERQ_ERR_UNSUPPORTED


@pytest.mark.slow
def test_l2qer_attention_projection():
    c = WL.attn_proj_int4()[0]
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, c.M - 1], rng.choice(c.M, 64, replace=False)]))
    cols = np.unique(np.concatenate([[0, c.d_out - 1], rng.choice(c.d_out, 256, replace=False)]))
    run_case(c, 128, factors=_range_factors, rows=rows, cols=cols)


# --------------------------------------------------------------------------
# MXFP4 layers: MX-quantized factors, T the exact block sum rounded once to
# fp32 (bit-exact), Q(T) by the per-token MXFP4 quantizer (bit-exact codes and
# E8M0 bytes), Y within the MXFP4 layer's bound, max|dY| <= 1e-4 * max|Y|.
# --------------------------------------------------------------------------
TOL_MX = 1e-4


def run_case_mx(c, k, bf16=False, rows=None):
    torch = torch_cuda()
    M, d_in, d_out = c.M, c.d_in, c.d_out
    L = B.serq_query_layout(d_in, d_out, 0, "mxfp4")
    lp = B.serq_prepare_weights(L, c.W, c.X_cal)
    p = O.prepare(c.W, c.X_cal, 0, "mxfp4")
    E = B.serq_weight_error(L, c.W, c.X_cal)
    L1, L2 = O.l2qer_factors(E, k)
    fl = B.serq_l2qer_prepare(L, L1, L2)
    fo = O.l2qer_prepare_mx(L1, L2)
    kp = O.r_padded(k)

    X_hat = O.flatten_acts(c.X, lp["s"], lp["perm"])
    Xd = dev(X_hat)
    if bf16:
        Xd = Xd.to(torch.bfloat16)
        X_hat = Xd.float().cpu().numpy()
    xq_o, xe_o = O.quant_act(X_hat, "mxfp4")
    nq, ns = B.serq_act_bytes(M, d_in, "mxfp4")
    xq = torch.empty(nq, dtype=torch.uint8, device="cuda")
    xs = torch.empty(ns, dtype=torch.uint8, device="cuda")
    B.serq_quant_act(Xd, "mxfp4", xq, xs)
    d = {n: dev(lp[n]) for n in ("wq", "wscale")}
    f = {n: dev(fl[n]) for n in ("l1q", "l1scale", "l2q", "l2scale")}

    T = torch.full((M, kp), np.nan, dtype=torch.float32, device="cuda")
    tq = torch.empty(M * kp // 2, dtype=torch.uint8, device="cuda")
    te = torch.empty(M * kp // 32, dtype=torch.uint8, device="cuda")
    B.serq_l2qer_intermediate(L, k, xq, xs, M, f["l1q"], f["l1scale"], T, tq, te)
    torch.cuda.synchronize()
    T_o = np.zeros((M, kp), np.float32)
    T_o[:, :k] = O.l2qer_intermediate_mx(xq_o, xe_o, fo)
    np.testing.assert_array_equal(host(T), T_o)
    want_q, want_e = O.packed_acts(*O.quant_act(T_o, "mxfp4"), "mxfp4")
    np.testing.assert_array_equal(host(tq).reshape(M, -1), want_q.reshape(M, -1))
    np.testing.assert_array_equal(host(te).reshape(M, -1), want_e.reshape(M, -1))

    Y = torch.full((M, d_out), np.nan, dtype=torch.float32, device="cuda")
    B.serq_l2qer_linear_q(L, k, xq, xs, M, d["wq"], d["wscale"], tq, te, f["l2q"], f["l2scale"], Y)
    torch.cuda.synchronize()
    rsel = np.arange(M) if rows is None else rows
    Yo = O.l2qer_linear_mx(xq_o[rsel], xe_o[rsel], p, fo)["Y"]
    Yg = host(Y)[rsel]
    assert np.all(np.isfinite(Yg))
    err, scale = np.abs(Yg - Yo).max(), np.abs(Yo).max()
    assert err <= TOL_MX * scale, (err, scale)

    ws = torch.empty(B.serq_l2qer_workspace_bytes(L, M, k), dtype=torch.uint8, device="cuda")
    Y2 = torch.full((M, d_out), np.nan, dtype=torch.float32, device="cuda")
    B.serq_l2qer_linear(L, k, Xd, d["wq"], d["wscale"], f["l1q"], f["l1scale"], f["l2q"], f["l2scale"], Y2, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(Y2), host(Y))
    return err / scale


SHAPES_MX = [  # M, d_in, d_out, k -- the smallest batch, ragged M and d_out, k below the 128 pad, several K groups
    (17, 512, 48, 32), (200, 1024, 272, 96), (300, 1536, 448, 128), (513, 2560, 208, 64),
]


@pytest.mark.parametrize("shape", SHAPES_MX, ids=lambda s: "x".join(map(str, s)))
def test_l2qer_mx_small_shapes(shape):
    M, d_in, d_out, k = shape
    c = WL.random_case(sum(shape) + 1, M, d_in, d_out, 0, "mxfp4", n_out=4, factor=50.0, n_cal=64)
    run_case_mx(c, k)


def test_l2qer_mx_bf16_input():
    c = WL.random_case(8, 100, 512, 96, 0, "mxfp4", n_out=4, factor=50.0, n_cal=32)
    run_case_mx(c, 64, bf16=True)


def test_l2qer_mx_rejects_decode_batches_and_bad_k():
    torch = torch_cuda()
    L = B.serq_query_layout(512, 48, 0, "mxfp4")
    bufs = [torch.empty(4096, dtype=torch.uint8, device="cuda") for _ in range(8)]
    Y = torch.empty(16 * 48, dtype=torch.float32, device="cuda")
    with pytest.raises(B.SerqError) as e:
        B.serq_l2qer_linear_q(L, 32, bufs[0], bufs[1], 16, *bufs[2:8], Y)
    assert e.value.status == B.SERQ_ERR_UNSUPPORTED
    with pytest.raises(B.SerqError) as e:
        B.serq_l2qer_linear_q(L, 48, bufs[0], bufs[1], 64, *bufs[2:8], Y)
    assert e.value.status == B.SERQ_ERR_SHAPE


@pytest.mark.slow
def test_l2qer_mx_many_tiles():
    """16 x 16 tiles of 256 x 224 (the 224-channel form fills the CUs in one
    round), sampled rows."""
    c = WL.random_case(9, 4096, 512, 3584, 0, "mxfp4", n_out=6, factor=50.0, n_cal=128)
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[0, c.M - 1], rng.choice(c.M, 96, replace=False)]))
    run_case_mx(c, 128, rows=rows)


@pytest.mark.slow
def test_l2qer_mx_two_rounds_of_tiles():
    """More tiles than CUs (16 x 24 tiles of 256 x 192 on a 256-CU device),
    sampled rows."""
    c = WL.random_case(10, 4096, 512, 4480, 0, "mxfp4", n_out=6, factor=50.0, n_cal=128)
    rng = np.random.default_rng(10)
    rows = np.unique(np.concatenate([[0, c.M - 1], rng.choice(c.M, 96, replace=False)]))
    run_case_mx(c, 96, rows=rows)
