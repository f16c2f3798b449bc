"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: quantized activation codes and scales, and the int32 accumulators
A_main / A_res, bit-exact; Y within max|dY| <= 1e-5 * max|Y| (INT4, W4A8) or
1e-4 * max|Y| (MXFP4).  Full-size workloads compare a seeded sample of rows
(plus the first and last) that the oracle evaluates one by one.
"""
import functools

import numpy as np
import pytest

from oracle import serq_oracle as O
from rank_error_compensated_amd import binding as B
from rank_error_compensated_amd import workloads as WL

pytestmark = pytest.mark.gpu

TOL = {"int4": 1e-5, "w4a8": 1e-5, "mxfp4": 1e-4, "mxw4a8": 1e-4}
ALL_FMTS = ["int4", "w4a8", "mxfp4", "mxw4a8"]
MX = ("mxfp4", "mxw4a8")


def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    B.lib()          # fail loudly when the library is not built
    return torch


def dev(a):
    torch = torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t):
    return t.cpu().numpy()


@functools.lru_cache(maxsize=None)
def workload(name):
    return {"tiny": WL.tiny_int4, "attn": WL.attn_proj_int4, "mlp": WL.llama3_mlp_int4,
            "mx": WL.llama3_layer_mxfp4,
            "mx8": lambda: WL.llama3_layer_mxfp4(fmt="mxw4a8")}[name]()


def sample_rows(M, n=96, seed=0):
    if M <= n:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, M - 1], rng.choice(M, n, replace=False)]))


def sample_cols(N, n=256, seed=1):
    if N <= n:
        return None
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, N - 1], rng.choice(N, n, replace=False)]))


def prepared(c, fmt, cols=None, gptq=False):
    """Oracle prep (on the sampled output channels), library prep (full; its
    buffers checked equal to the oracle's on those channels).  With gptq the
    non-salient rows come from GPTQ on both sides."""
    if gptq:
        p = O.prepare_gptq(c.W, c.X_cal, c.r, fmt, cols=cols)
    else:
        p = O.prepare(c.W, c.X_cal, c.r, fmt, cols=cols)
    want = O.packed_weights(p, tiled=cols is None)
    L = B.serq_query_layout(c.d_in, c.d_out, c.r, fmt)
    got = B.serq_prepare_weights(L, c.W, c.X_cal, gptq_damp=0.01 if gptq else None)
    for k in ("perm", "s"):
        np.testing.assert_array_equal(got[k], want[k], err_msg=k)
    for k in ("wq", "rq"):
        if cols is None:
            np.testing.assert_array_equal(got[k], want[k], err_msg=k)
        else:   # the sampled channels' rows, back in row-major order
            rb = (c.d_in if k == "wq" else L.r_pad) // 2
            rows = O.untile_rows(got[k], c.d_out, rb)
            np.testing.assert_array_equal(rows[cols].reshape(-1), want[k], err_msg=k)
    if cols is None:
        for k in ("wscale", "rscale"):
            np.testing.assert_array_equal(got[k], want[k], err_msg=k)
    else:   # scale buffers hold per-channel arrays (INT) or grouped E8M0 bytes (MX)
        for k in ("wscale", "rscale"):
            g_, w_ = got[k], want[k]
            if fmt in MX:
                nb = (c.d_in if k == "wscale" else L.r_pad) // 32
                g_ = O.untile_scale_rows(g_, c.d_out, nb)[cols].reshape(-1) if nb else g_
            else:
                parts = g_.size // (4 * c.d_out)
                g_ = np.concatenate([g_.view(np.int32).reshape(parts, c.d_out)[j][cols].view(np.uint8)
                                     for j in range(parts)])
            np.testing.assert_array_equal(g_, w_, err_msg=k)
    return p, L, got


def check_layer(c, fmt=None, rows=None, bf16=False, X_hat=None, cols=None, gptq=False):
    """Runs quant_act, linear_q (with accumulators) and linear on the GPU and
    compares each with the oracle (on sampled rows / output channels)."""
    torch = torch_cuda()
    fmt = fmt or c.fmt
    p, L, lp = prepared(c, fmt, cols, gptq)
    csel = slice(None) if cols is None else cols
    if X_hat is None:
        X_hat = O.flatten_acts(c.X, p["s"], p["perm"])
        np.testing.assert_array_equal(B.serq_flatten_act(c.X, lp["perm"], lp["s"]), X_hat)
    Xd = dev(X_hat)
    if bf16:
        Xd = Xd.to(torch.bfloat16)
        X_hat = Xd.float().cpu().numpy()          # the exact fp32 values of the bf16 input
    M = X_hat.shape[0]
    rows = np.arange(M) if rows is None else rows

    # oracle on the sampled rows
    xq_o, xs_o = O.quant_act(X_hat, fmt)
    wd = {k: dev(lp[k]) if lp[k].size else None for k in ("wq", "wscale", "rq", "rscale")}

    # quant_act: codes and scales bit-exact on every row
    nq, ns = B.serq_act_bytes(M, c.d_in, fmt)
    xq = torch.empty(nq, dtype=torch.uint8, device="cuda")
    xs = torch.empty(ns, dtype=torch.uint8, device="cuda")
    B.serq_quant_act(Xd, fmt, xq, xs)
    torch.cuda.synchronize()
    want_q, want_s = O.packed_acts(xq_o, xs_o, fmt)
    np.testing.assert_array_equal(host(xq).reshape(M, -1), want_q.reshape(M, -1))
    np.testing.assert_array_equal(host(xs), want_s)

    # linear_q: accumulators bit-exact, Y within tolerance
    Y = torch.full((M, c.d_out), np.nan, dtype=torch.float32, device="cuda")
    mx = fmt in MX
    am = None if mx else torch.empty((M, c.d_out), dtype=torch.int32, device="cuda")
    ar = None if mx else torch.empty((M, c.d_out), dtype=torch.int32, device="cuda")
    B.serq_linear_q(L, xq, xs, M, wd["wq"], wd["wscale"], wd["rq"], wd["rscale"], Y, am, ar)
    torch.cuda.synchronize()
    Yg = host(Y)[rows][:, csel]
    if mx:
        Yo = O.linear_mx(xq_o[rows], xs_o[rows], p)
    else:
        Yo, Am, Ar = O.linear_int(xq_o[rows], xs_o[rows], p)
        np.testing.assert_array_equal(host(am)[rows][:, csel], Am)
        np.testing.assert_array_equal(host(ar)[rows][:, csel], Ar)
    scale = np.abs(Yo).max()
    err = np.abs(Yg - Yo).max()
    assert np.all(np.isfinite(Yg))
    assert err <= TOL[fmt] * scale, (err, scale)

    # the whole layer: quantization fused with the product, same result
    Y2 = torch.full((M, c.d_out), np.nan, dtype=torch.float32, device="cuda")
    ws = torch.empty(B.serq_linear_workspace_bytes(L, M), dtype=torch.uint8, device="cuda")
    B.serq_linear(L, Xd, wd["wq"], wd["wscale"], wd["rq"], wd["rscale"], Y2, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(Y2), host(Y))
    return err / scale


# ---------------------------------------------------------------- quantizer

@pytest.mark.parametrize("fmt", ALL_FMTS)
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("M,d_in", [(1, 128), (7, 256), (33, 4096), (5, 14336), (3, 16512), (2, 24576),
                                    (300, 4096), (260, 14336)])
def test_quant_act_bit_exact(fmt, bf16, M, d_in):
    """Codes, scales (and INT4 code sums) bit-exact against the oracle, for a
    few tokens (1024-thread workgroups) and for more tokens than compute units
    (256-thread workgroups)."""
    torch = torch_cuda()
    rng = np.random.default_rng(M * 1000 + d_in)
    X = (rng.standard_normal((M, d_in)) * rng.uniform(0.1, 20, (M, 1))).astype(np.float32)
    X[0, :2] = [94.89062, 20.333702]          # the divide-versus-reciprocal vector
    X[0, 2:9] = [7.0, -3.5, 2.5, 0.5, -0.5, 1.5, 0.0]
    if M > 2:
        X[2] = 0.0                            # an all-zero token
    if M > 3:
        X[3, 32:64] = 0.0                     # an all-zero MX block
    Xd = dev(X)
    if bf16:
        Xd = Xd.to(torch.bfloat16)
        X = Xd.float().cpu().numpy()
    nq, ns = B.serq_act_bytes(M, d_in, fmt)
    xq = torch.empty(nq, dtype=torch.uint8, device="cuda")
    xs = torch.empty(ns, dtype=torch.uint8, device="cuda")
    B.serq_quant_act(Xd, fmt, xq, xs)
    torch.cuda.synchronize()
    q, s = O.quant_act(X, fmt)
    want_q, want_s = O.packed_acts(q, s, fmt)
    np.testing.assert_array_equal(host(xq).reshape(M, -1), want_q.reshape(M, -1))
    np.testing.assert_array_equal(host(xs), want_s)


# ---------------------------------------------------------------- layer, small shapes

SHAPES = [  # M, d_in, d_out, r  -- ragged M and N tails, r = 0, r = d_in, decode and prefill paths
    (1, 128, 16, 0), (3, 128, 48, 32), (16, 256, 128, 16), (16, 256, 144, 256), (17, 384, 144, 128),
    (130, 256, 272, 256), (257, 512, 400, 96), (64, 1024, 256, 384), (200, 768, 1040, 0),
    (384, 1280, 272, 128),
]


@pytest.mark.parametrize("fmt", ALL_FMTS)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_layer_small_shapes(fmt, shape):
    M, d_in, d_out, r = shape
    if fmt in MX and r % 32:
        r = (r + 31) // 32 * 32
    c = WL.random_case(hash(shape) % 10000, M, d_in, d_out, r, fmt, n_out=4, factor=50.0, n_cal=64)
    check_layer(c)


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_layer_many_token_tiles(fmt):
    """5000 tokens: 20 token tiles of the large-tile kernels (the last one
    ragged) under the XCD-grouped tile order, on sampled tokens including
    the first and last."""
    c = WL.random_case(5000 + len(fmt), 5000, 512, 1024, 128, fmt, n_out=4, factor=50.0, n_cal=64)
    check_layer(c, rows=np.unique(np.concatenate([sample_rows(5000, 96), np.arange(4990, 5000)])))


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_layer_bf16_input(fmt):
    c = WL.random_case(77, 40, 512, 160, 64, fmt, n_out=4, factor=50.0, n_cal=32)
    check_layer(c, bf16=True)


@pytest.mark.parametrize("fmt", ALL_FMTS)
@pytest.mark.parametrize("shape", [(130, 256, 48, 0), (257, 512, 144, 64), (16, 384, 272, 128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_layer_gptq_prepared(fmt, shape):
    """GPTQ-prepared weights through the same kernels (prefill and decode)."""
    M, d_in, d_out, r = shape
    c = WL.random_case(sum(shape), M, d_in, d_out, r, fmt, n_out=4, factor=50.0, n_cal=96)
    check_layer(c, gptq=True)


@pytest.mark.slow
def test_workload_attention_projection_gptq():
    c = workload("attn")[0]
    check_layer(c, rows=sample_rows(c.M, 48), cols=sample_cols(c.d_out, 256), gptq=True)


@pytest.mark.slow
@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
def test_workload_down_projection_gptq(fmt):
    """The LLaMA-3-8B down projection (14336 -> 4096, r = 128: 14208
    non-salient rows GPTQ'd against their Hessian, Q(R) against the salient
    channels') prepared by the library in full and by the oracle on sampled
    output channels: bytes equal, then the layer on the GPU against the
    oracle on sampled tokens and channels."""
    c = {x.name: x for x in workload("mlp")}["down"]
    check_layer(c, fmt=fmt, rows=sample_rows(c.M, 32), cols=sample_cols(c.d_out, 96), gptq=True)


def test_layer_degenerate_inputs():
    """Zero tokens, a zero weight column and tied saliency scores."""
    c = WL.random_case(78, 24, 256, 64, 32, "int4", n_out=3, factor=40.0, n_cal=16)
    c.X[5] = 0.0
    c.W[:, 7] = 0.0
    c.W[12] = c.W[13]
    c.X_cal[:, 12] = c.X_cal[:, 13]
    for fmt in ALL_FMTS:
        check_layer(c, fmt)


def test_determinism_and_no_out_of_bounds_writes():
    torch = torch_cuda()
    c = WL.random_case(79, 150, 512, 272, 128, "int4", n_out=4, factor=50.0, n_cal=32)
    for fmt in ("int4", "mxfp4", "mxw4a8"):
        p, L, lp = prepared(c, fmt)
        Xh = O.flatten_acts(c.X, p["s"], p["perm"])
        wd = {k: dev(lp[k]) for k in ("wq", "wscale", "rq", "rscale")}
        M, N = Xh.shape[0], c.d_out
        pad = 4096
        outs = []
        for _ in range(2):
            buf = torch.full((M * N + 2 * pad,), 12345.0, dtype=torch.float32, device="cuda")
            Y = buf[pad:pad + M * N].view(M, N)
            ws = torch.empty(B.serq_linear_workspace_bytes(L, M), dtype=torch.uint8, device="cuda")
            B.serq_linear(L, dev(Xh), wd["wq"], wd["wscale"], wd["rq"], wd["rscale"], Y, ws)
            torch.cuda.synchronize()
            b = host(buf)
            assert np.all(b[:pad] == 12345.0) and np.all(b[pad + M * N:] == 12345.0)
            outs.append(b[pad:pad + M * N].copy())
        np.testing.assert_array_equal(outs[0], outs[1])


# ---------------------------------------------------------------- the five workloads

def test_workload_tiny_int4():
    check_layer(workload("tiny")[0])


@pytest.mark.slow
def test_workload_attention_projection_int4():
    """2048 tokens, 4096 -> 4096, r = 128: every accumulator of every row."""
    check_layer(workload("attn")[0])


@pytest.mark.slow
@pytest.mark.parametrize("layer", ["gate", "up", "down"])
def test_workload_llama3_mlp_int4(layer):
    c = {x.name: x for x in workload("mlp")}[layer]
    check_layer(c, rows=sample_rows(c.M), cols=sample_cols(c.d_out, 1024))


@pytest.mark.slow
def test_workload_llama3_mlp_fused_gate_up():
    g, u, _ = workload("mlp")
    check_layer(WL.concat_shared([g, u], "gate_up"), rows=sample_rows(g.M, 48), cols=sample_cols(2 * g.d_out, 1024))


@pytest.mark.slow
@pytest.mark.parametrize("wl", ["mx", "mx8"])
@pytest.mark.parametrize("layer", ["q", "k", "v", "o", "gate", "up", "down"])
def test_workload_llama3_layer_mx(wl, layer):
    c = {x.name: x for x in workload(wl)}[layer]
    check_layer(c, rows=sample_rows(c.M, 64), cols=sample_cols(c.d_out))


@pytest.mark.parametrize("fmt", ["mxw4a8", "mxfp4"])
@pytest.mark.parametrize("shape", [(1000, 256, 32768, 64), (600, 384, 65552, 128), (300, 256, 73728, 96)],
                         ids=lambda s: "x".join(map(str, s)))
def test_mx_wide_tiles(fmt, shape):
    """Shapes outside the LDS-direct domain (d_in not a multiple of 512)
    with many channel tiles take the general MX kernels: ragged token tiles,
    a partial last channel tile, r < 128."""
    M, d_in, d_out, r = shape
    c = WL.random_case(sum(shape), M, d_in, d_out, r, fmt, n_out=4, factor=50.0, n_cal=32)
    cols = np.unique(np.concatenate([sample_cols(d_out, 192), np.arange(d_out - 40, d_out)]))
    check_layer(c, rows=sample_rows(M, 48), cols=cols)


@pytest.mark.parametrize("fmt", ["mxfp4", "mxw4a8"])
@pytest.mark.parametrize("shape", [(1000, 512, 32768, 64), (600, 1024, 65552, 128), (300, 512, 73728, 0),
                                   (257, 2048, 28672, 128)], ids=lambda s: "x".join(map(str, s)))
def test_mx_wide_lds_direct(fmt, shape):
    """MX shapes with d_in % 512 == 0 and r <= 128 take the LDS-direct
    kernels: ragged token tiles, partial last channel tiles, the tile widths
    256, 224 and 192 (MX W4A8 up to 224), r = 64 (padded to 128), 128 and 0
    (no Q(R) tile), and d_in of one, two and four groups of four K steps."""
    M, d_in, d_out, r = shape
    c = WL.random_case(sum(shape) + 7, M, d_in, d_out, r, fmt, n_out=4, factor=50.0, n_cal=32)
    cols = np.unique(np.concatenate([sample_cols(d_out, 192), np.arange(d_out - 40, d_out)]))
    check_layer(c, rows=np.unique(np.concatenate([sample_rows(M, 48), np.arange(max(0, M - 8), M)])), cols=cols)


@pytest.mark.parametrize("fmt", ["mxfp4", "mxw4a8"])
@pytest.mark.parametrize("shape", [(129, 512, 4096, 128), (300, 1536, 1008, 0), (2048, 1024, 640, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_mx_narrow_lds_direct(fmt, shape):
    """MX shapes whose rounds favour 128-channel tiles (d_in % 512 == 0, r <=
    128, M > 128) take the LDS-direct kernels at 128 channels (eight waves
    for MXFP4): one partial token tile, a partial last channel tile (1008 =
    7 x 128 + 112), d_in of three four-step groups, r = 0, 64 and 128."""
    M, d_in, d_out, r = shape
    c = WL.random_case(sum(shape) + 11, M, d_in, d_out, r, fmt, n_out=4, factor=50.0, n_cal=32)
    cols = np.unique(np.concatenate([sample_cols(d_out, 192) if d_out > 256 else np.arange(d_out),
                                     np.arange(d_out - 24, d_out)]))
    check_layer(c, rows=np.unique(np.concatenate([sample_rows(M, 48), np.arange(max(0, M - 8), M)])), cols=cols)


@pytest.mark.parametrize("fmt", ["mxfp4", "mxw4a8"])
@pytest.mark.parametrize("shape", [(1, 512, 4096, 128), (5, 1024, 640, 0), (16, 512, 16384, 256), (16, 1536, 1024, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_mx_decode(fmt, shape):
    """MX layers with at most 16 tokens take the MX decode kernel: one token,
    a ragged token count, a full 16; sixteen waves splitting K where the
    16-channel blocks are few (640, 1024 and 4096 channels) and four where
    they fill the CUs (16384); r = 0, 64, 128 and 256 (two Q(R) steps)."""
    M, d_in, d_out, r = shape
    c = WL.random_case(sum(shape) + 13, M, d_in, d_out, r, fmt, n_out=4, factor=50.0, n_cal=32)
    check_layer(c, cols=sample_cols(d_out, 512))


@pytest.mark.slow
@pytest.mark.parametrize("wl", ["mx", "mx8"])
def test_workload_llama3_layer_mx_fused_gate_up(wl):
    cs = {x.name: x for x in workload(wl)}
    c = WL.concat_shared([cs["gate"], cs["up"]], "gate_up")
    check_layer(c, rows=sample_rows(c.M, 48), cols=sample_cols(c.d_out, 512))


@pytest.mark.parametrize("fmt", ["mxfp4", "mxw4a8"])
@pytest.mark.parametrize("shape", [(16, 4096, 16384, 256), (16, 14336, 1024, 256), (9, 8192, 4112, 128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_mx_decode_long_k(fmt, shape):
    """MX decode shapes whose K sequence (main then Q(R) steps) is longer than
    one pass of every wave's in-flight steps: 34 steps on four-wave
    workgroups (16384 channels), 114 and 65 steps on sixteen-wave ones; the
    last 16-channel block is among the sampled channels."""
    M, d_in, d_out, r = shape
    c = WL.random_case(sum(shape) + 17, M, d_in, d_out, r, fmt, n_out=4, factor=50.0, n_cal=32)
    cols = np.unique(np.concatenate([sample_cols(d_out, 384), np.arange(d_out - 32, d_out)]))
    check_layer(c, cols=cols)


@pytest.mark.parametrize("shape", [(300, 4096, 272, 384), (300, 640, 272, 128), (257, 1024, 400, 512)],
                         ids=lambda s: "x".join(map(str, s)))
def test_int4_general_kernel_many_token_tiles(shape):
    """INT4 prefill shapes outside the large-tile kernel's domain (r_pad above
    256, or d_in not a multiple of 256) run the general 128 x 128 kernel over
    several token tiles, the last one ragged: every accumulator of every
    row."""
    M, d_in, d_out, r = shape
    c = WL.random_case(sum(shape) + 19, M, d_in, d_out, r, "int4", n_out=4, factor=50.0, n_cal=32)
    check_layer(c)


@pytest.mark.slow
@pytest.mark.parametrize("fmt", ["int4", "w4a8", "mxfp4", "mxw4a8"])
@pytest.mark.parametrize("M", [1, 8, 16])
def test_workload_decode(fmt, M):
    """The decode workload's two layers (gate|up 4096 -> 28672, down 14336 ->
    4096, r = 256) in every format: sampled output channels including the
    first and last."""
    for c in WL.decode_llama3(fmt, M):
        check_layer(c, cols=np.unique(np.concatenate([sample_cols(c.d_out, 2048),
                                                      np.arange(c.d_out - 16, c.d_out)])))


@pytest.mark.parametrize("fmt", ["int4", "w4a8"])
@pytest.mark.parametrize("shape", [(5, 512, 16400, 128), (16, 384, 16432, 256), (1, 256, 16448, 0)],
                         ids=lambda s: "x".join(map(str, s)))
def test_decode_wide_ragged(fmt, shape):
    """Decode layers wide enough for four column blocks per workgroup
    (d_out >= 16384) whose last workgroup holds fewer than four real blocks:
    1, 3 and 0 blocks past a multiple of four, with the INT4 form's waves in
    pairs and W4A8's all on K; every output channel of the last workgroups
    is checked."""
    M, d_in, d_out, r = shape
    c = WL.random_case(sum(shape), M, d_in, d_out, r, fmt, n_out=4, factor=50.0, n_cal=32)
    cols = np.unique(np.concatenate([sample_cols(d_out, 256), np.arange(d_out - 200, d_out)]))
    check_layer(c, cols=cols)


@pytest.mark.parametrize("fmt", ["int4", "w4a8"])
@pytest.mark.parametrize("shape", [(16, 14336, 1024, 256), (5, 2176, 272, 2048), (16, 1024, 256, 1024),
                                   (4, 4224, 16384, 256), (12, 2048, 16400, 256)],
                         ids=lambda s: "x".join(map(str, s)))
def test_decode_residual_half_steps(fmt, shape):
    """The decode kernels take Q(R) in half steps of 64 elements where that
    shortens the longest wave: one half each on four of sixteen waves (the
    down projection's split); 17 main steps over 16 waves with 32 halves;
    the wide form with two waves on K (INT4, 33 main steps) and four (W4A8,
    16 main steps); and whole residual steps where halves gain nothing (a
    residual as long as the main part)."""
    M, d_in, d_out, r = shape
    c = WL.random_case(sum(shape) + 7, M, d_in, d_out, r, fmt, n_out=4, factor=50.0, n_cal=32)
    cols = None if d_out <= 1024 else np.unique(np.concatenate([sample_cols(d_out, 512),
                                                                np.arange(d_out - 64, d_out)]))
    check_layer(c, cols=cols)


def test_graph_replays_match_eager():
    """serq_linear captured in a HIP graph: every replay (with eager work and
    synchronizations between replays) equals the eager result bit for bit."""
    torch = torch_cuda()
    for fmt, shape in (("int4", (300, 512, 272, 128)), ("int4", (16, 512, 2048, 256)),
                       ("w4a8", (200, 384, 144, 128)), ("mxfp4", (130, 512, 256, 64)),
                       ("mxw4a8", (300, 384, 272, 96))):
        M, d_in, d_out, r = shape
        c = WL.random_case(81, M, d_in, d_out, r, fmt, n_out=4, factor=50.0, n_cal=32)
        layer = B.PreparedLayer.prepare(c.W, c.X_cal, r, fmt, "cuda")
        X = dev(B.serq_flatten_act(c.X, layer.host["perm"], layer.host["s"]))
        Y = torch.empty((M, d_out), dtype=torch.float32, device="cuda")
        ws = layer.workspace(M)
        layer(X, Y, ws)
        torch.cuda.synchronize()
        eager = host(Y).copy()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layer(X, Y, ws)
        for _ in range(3):
            Y.fill_(float("nan"))
            _ = (X * 2.0).sum()          # unrelated eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            np.testing.assert_array_equal(host(Y), eager)


# ---------------------------------------------------------------- producers fused with quantization

def _producer_inputs(M, d, seed):
    rng = np.random.default_rng(seed)
    perm = rng.permutation(d).astype(np.int32)
    s = rng.uniform(0.2, 5.0, d).astype(np.float32)
    return rng, perm, s


def _check_codes(xq, xs, X, perm, s, fmt, M):
    q, sc = O.quant_act(O.flatten_acts(X, s, perm), fmt)
    want_q, want_s = O.packed_acts(q, sc, fmt)
    np.testing.assert_array_equal(host(xq).reshape(M, -1), want_q.reshape(M, -1))
    np.testing.assert_array_equal(host(xs), want_s)


@pytest.mark.parametrize("fmt", ALL_FMTS)
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("M,d", [(1, 128), (7, 4096), (33, 512), (3, 14336), (2, 16384), (300, 4096)])
def test_rmsnorm_quant_bit_exact(fmt, bf16, M, d):
    """serq_rmsnorm_quant = RMSNorm, flatten (perm, / s), quant_act: codes,
    scales and code sums bit-exact against the oracle's chain."""
    torch = torch_cuda()
    rng, perm, s = _producer_inputs(M, d, M * 7 + d)
    h = (rng.standard_normal((M, d)) * rng.uniform(0.05, 30, (M, 1))).astype(np.float32)
    h[:, rng.choice(d, max(1, d // 100), replace=False)] *= 50.0
    if M > 2:
        h[2] = 0.0                                        # r = 1 / sqrt(eps), X = 0
    gamma = rng.uniform(0.5, 1.5, d).astype(np.float32)
    eps = 1e-5
    Hd = dev(h)
    if bf16:
        Hd = Hd.to(torch.bfloat16)
        h = Hd.float().cpu().numpy()
    nq, ns = B.serq_act_bytes(M, d, fmt)
    xq = torch.empty(nq, dtype=torch.uint8, device="cuda")
    xs = torch.empty(ns, dtype=torch.uint8, device="cuda")
    B.serq_rmsnorm_quant(Hd, dev(gamma[perm]), eps, dev(perm), dev(s[perm]), fmt, xq, xs)
    torch.cuda.synchronize()
    _check_codes(xq, xs, O.rmsnorm(h, gamma, eps), perm, s, fmt, M)


@pytest.mark.parametrize("fmt", ALL_FMTS)
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("M,d", [(1, 128), (5, 14336), (17, 1024), (2, 16384), (272, 14336)])
def test_swiglu_quant_bit_exact(fmt, bf16, M, d):
    """serq_swiglu_quant = silu(gate) * up, flatten, quant_act: bit-exact
    against the oracle's chain, including gate values past the exponential's
    limits."""
    torch = torch_cuda()
    rng, perm, s = _producer_inputs(M, d, M * 11 + d)
    G = (rng.standard_normal((M, d)) * 3.0).astype(np.float32)
    U = (rng.standard_normal((M, d)) * rng.uniform(0.1, 10, (M, 1))).astype(np.float32)
    G[0, :6] = [0.0, 88.0, 89.0, -86.5, -87.5, -120.0]
    GU = np.concatenate([G, U], axis=1)
    GUd = dev(GU)
    if bf16:
        GUd = GUd.to(torch.bfloat16)
        GU = GUd.float().cpu().numpy()
    nq, ns = B.serq_act_bytes(M, d, fmt)
    xq = torch.empty(nq, dtype=torch.uint8, device="cuda")
    xs = torch.empty(ns, dtype=torch.uint8, device="cuda")
    B.serq_swiglu_quant(GUd, dev(perm), dev(s[perm]), fmt, xq, xs)
    torch.cuda.synchronize()
    _check_codes(xq, xs, O.swiglu(GU[:, :d], GU[:, d:]), perm, s, fmt, M)


@pytest.mark.parametrize("fmt", ["int4", "mxfp4", "mxw4a8"])
def test_fused_producers_give_the_unfused_layer_output(fmt):
    """The layer fed by the fused producer equals the layer fed the flattened
    producer output (serq_linear on X-hat), bit for bit: q|k|v behind RMSNorm
    and the down projection behind SwiGLU of the LLaMA-3-8B shapes (256
    tokens)."""
    torch = torch_cuda()
    rng = np.random.default_rng(5)
    M = 256
    for kind, d_in, d_out in (("rms", 4096, 1024), ("swiglu", 14336, 512)):
        c = WL.random_case(91, M, d_in, d_out, 128, fmt, n_out=max(1, d_in // 100), factor=50.0, n_cal=64)
        layer = B.PreparedLayer.prepare(c.W, c.X_cal, 128, fmt, "cuda")
        perm, s = layer.host["perm"], layer.host["s"]
        nq, ns = B.serq_act_bytes(M, d_in, fmt)
        xq = torch.empty(nq, dtype=torch.uint8, device="cuda")
        xs = torch.empty(ns, dtype=torch.uint8, device="cuda")
        if kind == "rms":
            h = rng.standard_normal((M, d_in)).astype(np.float32)
            gamma = rng.uniform(0.5, 1.5, d_in).astype(np.float32)
            B.serq_rmsnorm_quant(dev(h), dev(gamma[perm]), 1e-5, dev(perm), dev(s[perm]), fmt, xq, xs)
            X = O.rmsnorm(h, gamma, 1e-5)
        else:
            GU = (rng.standard_normal((M, 2 * d_in)) * 2.0).astype(np.float32)
            B.serq_swiglu_quant(dev(GU), dev(perm), dev(s[perm]), fmt, xq, xs)
            X = O.swiglu(GU[:, :d_in], GU[:, d_in:])
        d = layer.dev
        Y1 = torch.empty((M, d_out), dtype=torch.float32, device="cuda")
        B.serq_linear_q(layer.L, xq, xs, M, d["wq"], d["wscale"], d["rq"], d["rscale"], Y1)
        Y2 = layer(dev(B.serq_flatten_act(X, perm, s)))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(Y1), host(Y2))


@pytest.mark.parametrize("shape", [(300, 512, 384, 128), (257, 1024, 640, 64), (2048, 4096, 1024, 128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_swiglu_epilogue(shape):
    """serq_linear_swiglu on a gate|up layer in (gate, up) pairs: H equals the
    oracle's SwiGLU and flattening applied to the same layer's Y bit for bit,
    its quantized codes equal the unfused chain's (serq_swiglu_quant on Y),
    and H stays within the bound Y's tolerance implies of the oracle's
    end-to-end H (ragged token tiles, r below and at 128, 2048 tokens)."""
    torch = torch_cuda()
    M, d_in, d, r = shape
    c = WL.random_case(sum(shape) + 23, M, d_in, 2 * d, r, "int4", n_out=4, factor=50.0, n_cal=64)
    rng = np.random.default_rng(sum(shape))
    perm = rng.permutation(d).astype(np.int32)
    s = rng.uniform(0.3, 3.0, d).astype(np.float32)
    W = O.swiglu_pairs(c.W[:, :d], c.W[:, d:], perm)
    layer = B.PreparedLayer.prepare(W, c.X_cal, r, "int4", "cuda")
    Xh = B.serq_flatten_act(c.X, layer.host["perm"], layer.host["s"])
    X = dev(Xh)
    Y = torch.empty((M, 2 * d), dtype=torch.float32, device="cuda")
    layer(X, Y)
    H = torch.full((M, d), float("nan"), dtype=torch.float32, device="cuda")
    sd = dev(s[perm])
    dv = layer.dev
    B.serq_linear_swiglu(layer.L, X, dv["wq"], dv["wscale"], dv["rq"], dv["rscale"], sd, H, layer.workspace(M))
    torch.cuda.synchronize()
    Yh, Hh = host(Y), host(H)
    np.testing.assert_array_equal(Hh, O.swiglu_paired(Yh, s[perm]))
    # the unfused chain's codes: the fused producer on [gate | up] in saliency order
    nq, ns = B.serq_act_bytes(M, d, "int4")
    q1, s1, q2, s2 = (torch.empty(n, dtype=torch.uint8, device="cuda") for n in (nq, ns, nq, ns))
    B.serq_swiglu_quant(dev(np.concatenate([Yh[:, 0::2], Yh[:, 1::2]], axis=1)), None, sd, "int4", q1, s1)
    B.serq_quant_act(H, "int4", q2, s2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(q1), host(q2))
    np.testing.assert_array_equal(host(s1), host(s2))
    # end to end against the oracle: Y within 1e-5 max|Y|, then
    # |dH| <= (max|silu'| max|u| + max|silu(g)|) dY / min s  (max|silu'| < 1.1)
    p = O.prepare(W, c.X_cal, r, "int4")
    Yo = O.serq_linear(O.flatten_acts(c.X, p["s"], p["perm"]), p)["Y"]
    Ho = O.swiglu_paired(Yo, s[perm])
    dY = 1e-5 * np.abs(Yo).max()
    bound = (1.1 * np.abs(Yo[:, 1::2]).max() + np.abs(O.swiglu(Yo[:, 0::2], np.ones_like(Yo[:, 0::2]))).max()) \
        * dY / s.min() + 1e-6 * np.abs(Ho).max()
    assert np.abs(Hh - Ho).max() <= bound


@pytest.mark.parametrize("shape", [(300, 512, 384, 128), (257, 2048, 1024, 0), (2048, 4096, 7168, 128),
                                   (1024, 512, 16384, 64), (300, 512, 128, 32)], ids=lambda s: "x".join(map(str, s)))
def test_swiglu_quantizing_epilogue_mx(shape):
    """serq_linear_swiglu_q on an MXFP4 gate|up layer in (gate, up) pairs: the
    next layer's E2M1 codes and E8M0 bytes equal, bit for bit, the oracle's
    SwiGLU, flattening and MXFP4 quantization applied to the same layer's Y
    (serq_linear, whose LDS-direct kernel accumulates in the same order at
    these shapes).  On a 256-CU device the first two shapes take the
    128-channel tiles with eight waves, the next two the 256-channel ones
    (one and two rounds of workgroups), the last the narrowest layer (256
    columns, a 128-wide next layer); ragged token tiles, r = 0, 32, 64,
    128."""
    torch = torch_cuda()
    M, d_in, d, r = shape
    c = WL.random_case(sum(shape) + 29, M, d_in, 2 * d, r, "mxfp4", n_out=4, factor=50.0, n_cal=64)
    rng = np.random.default_rng(sum(shape) + 1)
    perm = rng.permutation(d).astype(np.int32)
    s = rng.uniform(0.3, 3.0, d).astype(np.float32)
    W = O.swiglu_pairs(c.W[:, :d], c.W[:, d:], perm)
    layer = B.PreparedLayer.prepare(W, c.X_cal, r, "mxfp4", "cuda")
    X = dev(B.serq_flatten_act(c.X, layer.host["perm"], layer.host["s"]))
    Y = torch.empty((M, 2 * d), dtype=torch.float32, device="cuda")
    layer(X, Y)
    nq, ns = B.serq_act_bytes(M, d, "mxfp4")
    xq = torch.full((nq,), 0xAB, dtype=torch.uint8, device="cuda")
    xe = torch.full((ns,), 0xCD, dtype=torch.uint8, device="cuda")
    dv = layer.dev
    B.serq_linear_swiglu_q(layer.L, X, dv["wq"], dv["wscale"], dv["rq"], dv["rscale"], dev(s[perm]), xq, xe,
                           layer.workspace(M))
    torch.cuda.synchronize()
    H = O.swiglu_paired(host(Y), s[perm])
    want_q, want_e = O.packed_acts(*O.quant_act(H, "mxfp4"), "mxfp4")
    np.testing.assert_array_equal(host(xq).reshape(M, -1), want_q.reshape(M, -1))
    np.testing.assert_array_equal(host(xe).reshape(M, -1), want_e.reshape(M, -1))


@pytest.mark.parametrize("fmt", ALL_FMTS)
@pytest.mark.parametrize("M,d", [(3, 14336), (9, 512), (264, 4096)])
def test_swiglu_quant_folded_permutation(fmt, M, d):
    """perm = NULL: gate and up arriving in saliency order give the same codes
    as the gather from original order."""
    torch = torch_cuda()
    rng, perm, s = _producer_inputs(M, d, M * 13 + d)
    GU = (rng.standard_normal((M, 2 * d)) * 3.0).astype(np.float32)
    folded = np.concatenate([GU[:, :d][:, perm], GU[:, d:][:, perm]], axis=1)
    nq, ns = B.serq_act_bytes(M, d, fmt)
    outs = []
    for src, pm in ((GU, dev(perm)), (folded, None)):
        xq = torch.empty(nq, dtype=torch.uint8, device="cuda")
        xs = torch.empty(ns, dtype=torch.uint8, device="cuda")
        B.serq_swiglu_quant(dev(src), pm, dev(s[perm]), fmt, xq, xs)
        torch.cuda.synchronize()
        outs.append((host(xq), host(xs)))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])
    _check_codes(torch.from_numpy(outs[1][0]), torch.from_numpy(outs[1][1]), O.swiglu(GU[:, :d], GU[:, d:]), perm, s,
                 fmt, M)
