"""CPU oracle for SERQ's quantized linear layer.

TEST INFRASTRUCTURE ONLY.  This is the slow, plainly written reference that the
HIP library is checked against.  Only the test suite, the package smoke check
and the bench's CPU-baseline leg may import or run it; the product path never
does, and nothing here is shared with the HIP path (no kernels, headers,
helpers, tables or constant generators).

What it computes follows the method as written on the pages:

* "SERQ: Saliency-Aware Low-Rank Error Reconstruction for LLM Quantization",
  research notes (dihengye.cn) -- the basic-quantization equation, Stage 1
  (static activation flattening), Stage 2 (saliency partition, the single
  compensation matrix R, the quantized inference equation), Stage 3 (offline
  permutation);
* the gist.science technical summaries (zh and pt), sections 2.1-2.3, and the
  abstract page on fugumt.com (W4A8 and W4A4 settings).

Readings of points the pages leave open (each is listed with its reason in the
design notes of the repository):

* SAF scale s_j = sqrt(max|X_cal[:, j]| / max|W[j, :]|) (SmoothQuant-style,
  alpha = 1/2); s_j = 1 when either maximum is 0.
* Saliency order: s descending, ties by ascending original channel index; the
  first r rows of the permuted weight are the salient rows.
* Granularity: per token for activations, per output channel for W-hat and R.
* Rounding: round-half-to-even of the IEEE fp32 quotient x / s, then clip to
  [-(2^(n-1)-1), 2^(n-1)-1]; a zero scale gives zero codes.
* Q(W-tilde_s) in R is the main path's own quantization of the salient rows
  (per-channel scale over the full column), so W-tilde_s = Q(W-tilde_s) + R.
* X-tilde_{s,q} is the first r columns of the same quantized activation (same
  per-token scale): the method adds no second quantization.
* MXFP4: OCP MX v1.0 -- shared scale 2^(floor(log2 amax) - 2) stored as E8M0
  (bias 127, clamped to [0, 254]); elements rounded to the E2M1 grid
  {0, .5, 1, 1.5, 2, 3, 4, 6} to nearest, ties to the even code, saturating at
  6; the sign bit is copied from the input; an all-zero block has E8M0 = 127.
* MX W4A8 (the pages' W4A8 setting in MX form): MXFP4 weights and R as above,
  activations in OCP MX FP8 E4M3 -- shared scale 2^(floor(log2 amax) - 8),
  elements rounded to the nearest E4M3 value (ties to the even code),
  saturating at 448, sign from the input.

L2QER comparator (the two-factor path the pages contrast with SERQ: notes
page, 关键公式, "L2QER 的双矩阵路径"; gist.science summary zh, section 2.1):
Y = X_q . W_q + Q(X_q . L1_q) . L2_q.  The pages give only this runtime
equation; the readings used here:

* it shares SERQ's main path (the same flattened, permuted X-hat and W-hat_q),
  so that only the error-reconstruction path differs;
* L1 [d_in][k], L2 [k][d_out] are a rank-k truncated SVD of the whole weight
  error E = W-hat - dequant(W-hat_q), split evenly: L1 = U_k sqrt(S_k),
  L2 = sqrt(S_k) V_k^T (the factorization is offline input preparation;
  numpy's SVD is the library routine);
* L1 and L2 are quantized like weights (4-bit, one scale per output column);
* the intermediate T = X_q . L1_q is dequantized in fp32 as sx[m] * (sL1[j] *
  A1[m, j]) and quantized on the fly per token exactly like the layer input
  (4-bit, the same rounding rule).

GPTQ weight quantization (the pages list RTN and GPTQ as the supported
weight quantizers: gist.science summary zh, section 3; pt summary, results):
the published algorithm (Frantar et al., "GPTQ: Accurate Post-Training
Quantization for Generative Pre-trained Transformers", 2022) in its plain
row-by-row form (its lazy block updates only reorder the same sums).
Readings:

* the salient rows keep the main path's round-to-nearest codes (R corrects
  them exactly, so propagating their error as well would correct it twice);
  GPTQ quantizes rows r..d_in-1 with the Hessian of those channels only,
  H = 2 X-hat_cal^T X-hat_cal over the flattened calibration activations;
* Q(R) is a weight quantization too: GPTQ quantizes R's r rows with the
  Hessian of the salient channels, whose quantized activations the residual
  product reads;
* one scale per output channel over the original W-hat column (as for RTN;
  R: over R's column);
* H_kk = 0 (a channel never active in calibration) is set to 1, its weights
  kept; dampening adds 1 % of the mean diagonal; the error of row k divided
  by U_kk (U the upper Cholesky factor of H^-1) is subtracted from the later
  rows with weights U_kj;
* the updates run in fp64, and each row is rounded once to fp32 before its
  code is decided with the same fp32 rule as RTN.

Precision: every step that decides a code (maxima, the SAF scale, scales,
quotients, the residual R) is one IEEE fp32 operation, as numpy float32 does
it.  Integer accumulators are exact.  The layer output Y is evaluated in fp64
from the exact accumulators / exactly dequantized operands.
"""
from __future__ import annotations

import numpy as np

INT4 = "int4"
W4A8 = "w4a8"
MXFP4 = "mxfp4"
MXW4A8 = "mxw4a8"      # MXFP4 weights and R, MXFP8 (E4M3) activations
FORMATS = (INT4, W4A8, MXFP4, MXW4A8)
MX_FORMATS = (MXFP4, MXW4A8)

MX_BLOCK = 32
# E2M1 magnitudes indexed by the 3-bit code (exponent << 1 | mantissa).
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def r_padded(r: int) -> int:
    """Residual rows are stored padded with zero rows up to a multiple of 128."""
    return (r + 127) // 128 * 128


# --------------------------------------------------------------------------
# Basic symmetric quantizer (notes page, 关键公式 / 基础量化 equation):
#   X_q = clip(round(X / s)),  s = max|X| / (2^(n-1) - 1)
# --------------------------------------------------------------------------

def qmax(n_bits: int) -> int:
    return 2 ** (n_bits - 1) - 1


def sym_quant(x: np.ndarray, n_bits: int, axis: int):
    """Quantize ``x`` along ``axis`` (one scale per slice orthogonal to it).

    Returns (codes int8, scales fp32).  All arithmetic in fp32.
    """
    x = np.asarray(x, dtype=np.float32)
    q = np.float32(qmax(n_bits))
    amax = np.max(np.abs(x), axis=axis, keepdims=True)
    s = amax / q                                   # fp32 / fp32
    safe = np.where(s > 0, s, np.float32(1))
    t = x / safe                                   # IEEE fp32 quotient
    codes = np.clip(np.rint(t), -q, q)
    codes = np.where(s > 0, codes, 0).astype(np.int8)
    return codes, np.squeeze(s, axis=axis).astype(np.float32)


# --------------------------------------------------------------------------
# MX codec (OCP MX v1.0: E8M0 shared scale per 32 elements, E2M1 elements)
# --------------------------------------------------------------------------

def e2m1_code(v: np.ndarray) -> np.ndarray:
    """Nearest E2M1 code to v (already divided by the block scale).

    Brute force over the 8 grid magnitudes; on an exact tie the even code
    (mantissa bit 0) wins; magnitudes above 6 saturate to 6.  The sign bit is
    the input's sign bit.
    """
    v = np.asarray(v, dtype=np.float64)
    flat = v.reshape(-1)
    out = np.empty(flat.shape, np.uint8)
    even = (np.arange(8) % 2) == 0
    step = 1 << 20                                     # bounded temporary memory
    for lo in range(0, flat.size, step):
        part = flat[lo:lo + step]
        dist = np.abs(np.abs(part)[:, None] - E2M1_GRID)   # [n, 8]
        is_best = dist == np.min(dist, axis=-1, keepdims=True)
        # among equally near grid points prefer an even code index
        pick_even = is_best & even
        choice = np.where(np.any(pick_even, axis=-1, keepdims=True), pick_even, is_best)
        idx = np.argmax(choice, axis=-1).astype(np.uint8)
        out[lo:lo + step] = (np.signbit(part).astype(np.uint8) << 3) | idx
    return out.reshape(v.shape)


def e2m1_value(code: np.ndarray) -> np.ndarray:
    code = np.asarray(code, dtype=np.uint8)
    mag = E2M1_GRID[code & 7]
    return np.where(code & 8, -mag, mag)


# OCP MX FP8 E4M3: sign | 4 exponent bits (bias 7) | 3 mantissa bits; exponent
# field 0 holds the subnormals m/8 * 2^-6; 0x7F / 0xFF are NaN, so the largest
# magnitude is code 0x7E = 1.75 * 2^8 = 448.
E4M3_GRID = np.array([(c & 7) / 8.0 * 2.0 ** -6 if (c >> 3) == 0 else (1 + (c & 7) / 8.0) * 2.0 ** ((c >> 3) - 7)
                      for c in range(127)], dtype=np.float64)


def e4m3_code(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code to v (already divided by the block scale): brute force
    over the 127 finite magnitudes, ties to the even code, saturating at 448;
    the sign bit is the input's sign bit."""
    v = np.asarray(v, dtype=np.float64)
    flat = v.reshape(-1)
    out = np.empty(flat.shape, np.uint8)
    even = (np.arange(127) % 2) == 0
    step = 1 << 16
    for lo in range(0, flat.size, step):
        part = flat[lo:lo + step]
        dist = np.abs(np.abs(part)[:, None] - E4M3_GRID)
        is_best = dist == np.min(dist, axis=-1, keepdims=True)
        pick_even = is_best & even
        choice = np.where(np.any(pick_even, axis=-1, keepdims=True), pick_even, is_best)
        idx = np.argmax(choice, axis=-1).astype(np.uint8)
        out[lo:lo + step] = (np.signbit(part).astype(np.uint8) << 7) | idx
    return out.reshape(v.shape)


def e4m3_value(code: np.ndarray) -> np.ndarray:
    code = np.asarray(code, dtype=np.uint8)
    mag = E4M3_GRID[np.minimum(code & 0x7F, 126)]
    return np.where(code & 0x80, -mag, mag)


# element type -> (code function, value function, largest power of two of the
# element's range: 2 for E2M1 (6 = 1.5 * 2^2), 8 for E4M3 (448 = 1.75 * 2^8))
def mx_scale_exponent(amax: np.ndarray, emax: int = 2) -> np.ndarray:
    """Unbiased shared exponent floor(log2(amax)) - emax, clamped to E8M0's
    range (emax = 2 for E2M1 elements, 8 for E4M3).

    floor(log2(a)) is read exactly from frexp: a = m * 2^e with m in [0.5, 1).
    An all-zero block takes exponent 0.
    """
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)
    e = e.astype(np.int64) - 1 - emax
    e = np.where(amax > 0, e, 0)
    return np.clip(e, -127, 127)


def _mx_element(elem: str):
    if elem == "e2m1":
        return e2m1_code, e2m1_value, 2
    assert elem == "e4m3"
    return e4m3_code, e4m3_value, 8


def mx_quant(x: np.ndarray, axis: int, elem: str = "e2m1"):
    """MX-quantize fp32 ``x`` in blocks of 32 along ``axis``.

    Returns (element codes uint8 with the same shape as x -- E2M1 or E4M3 --
    and E8M0 bytes with the blocked axis divided by 32).
    """
    code_fn, _, emax = _mx_element(elem)
    x = np.asarray(x, dtype=np.float32)
    x = np.moveaxis(x, axis, -1)
    K = x.shape[-1]
    assert K % MX_BLOCK == 0
    xb = x.reshape(x.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(xb), axis=-1)
    e = mx_scale_exponent(amax, emax)
    # division by a power of two is exact (no denormal results for these data)
    v = xb.astype(np.float64) / np.ldexp(1.0, e)[..., None]
    codes = code_fn(v).reshape(x.shape)
    e8m0 = (e + 127).astype(np.uint8)
    return np.moveaxis(codes, -1, axis), np.moveaxis(e8m0, -1, axis)


def mx_dequant(codes: np.ndarray, e8m0: np.ndarray, axis: int, elem: str = "e2m1") -> np.ndarray:
    """Exact dequantization (fp64): value(code) * 2^(E8M0 - 127)."""
    _, value_fn, _ = _mx_element(elem)
    codes = np.moveaxis(np.asarray(codes, np.uint8), axis, -1)
    e = np.moveaxis(np.asarray(e8m0, np.int64), axis, -1) - 127
    scale = np.repeat(np.ldexp(1.0, e), MX_BLOCK, axis=-1)
    return np.moveaxis(value_fn(codes) * scale, -1, axis)


# --------------------------------------------------------------------------
# Offline preparation (Stages 1-3)
# --------------------------------------------------------------------------

def saf_scales(W: np.ndarray, X_cal: np.ndarray) -> np.ndarray:
    """Static activation flattening scale, one per input channel (Stage 1).

    s_j = sqrt(max_c |X_cal[c, j]| / max_o |W[j, o]|), one fp32 division and
    one fp32 square root; s_j = 1 when either maximum is zero.
    """
    ax = np.max(np.abs(np.asarray(X_cal, np.float32)), axis=0)
    aw = np.max(np.abs(np.asarray(W, np.float32)), axis=1)
    s = np.ones(W.shape[0], dtype=np.float32)
    ok = (ax > 0) & (aw > 0)
    s[ok] = np.sqrt(ax[ok] / aw[ok])
    return s


def saliency_perm(s: np.ndarray) -> np.ndarray:
    """Saliency order (Stage 2): channels by flattening scale, largest first.

    perm[k] is the original channel placed at position k; ties keep the
    original order.
    """
    return np.argsort(-np.asarray(s, np.float32), kind="stable").astype(np.int32)


def flatten_weights(W: np.ndarray, s: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """W-hat = P . diag(s) . W (Stage 2 partition equation), one fp32 product each."""
    W = np.asarray(W, np.float32)
    return (s[perm][:, None] * W[perm, :]).astype(np.float32)


def flatten_acts(X: np.ndarray, s: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """X-hat = X . diag(s)^-1 . P^T -- what the folded producer layer emits
    (Stage 1 identity, Stage 3 permutation).  One fp32 division each."""
    X = np.asarray(X, np.float32)
    return (X[:, perm] / s[perm][None, :]).astype(np.float32)


# --------------------------------------------------------------------------
# Producers of the layer input (the layers before a SERQ linear).  The notes
# page folds the flattening scale and the permutation into the operation that
# produces X (Stage 1, Stage 3), so the runtime input is X-hat already.  For
# the two producers of a LLaMA block -- the RMSNorm in front of q/k/v and the
# SwiGLU product in front of the down projection -- these give the fp32 X the
# producer computes; flatten_acts and quant_act then finish the input exactly
# as on the unfused path.
# --------------------------------------------------------------------------

def rmsnorm(h: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """X = h / sqrt(mean(h^2) + eps) * gamma, per token (LLaMA's RMSNorm).

    Reading of the precision: the sum of squares is accumulated in fp64 (each
    square of an fp32 value is exact there), the mean is rounded once to fp32,
    then r = 1 / sqrt(mean + eps) and X = (h * r) * gamma are fp32 operations
    in that order."""
    h = np.asarray(h, np.float32)
    ss = np.sum(h.astype(np.float64) ** 2, axis=1)
    ms = (ss / h.shape[1]).astype(np.float32)
    r = (np.float32(1.0) / np.sqrt(ms + np.float32(eps))).astype(np.float32)
    return ((h * r[:, None]).astype(np.float32) * np.asarray(gamma, np.float32)[None, :]).astype(np.float32)


# Cody-Waite split of ln 2: the high part has 16 significant bits, so n * LN2_HI
# is exact for |n| <= 256; the low part is the fp32 rounding of ln 2 - LN2_HI.
LN2_HI = np.float32(0.693145751953125)
LN2_LO = np.float32(1.428606765330187e-06)
LOG2E = np.float32(1.4426950408889634)
# Taylor coefficients 1/j! (j = 2..7), each rounded to fp32.
EXP_TAYLOR = [np.float32(1.0 / f) for f in (2.0, 6.0, 24.0, 120.0, 720.0, 5040.0)]


def exp32(x: np.ndarray) -> np.ndarray:
    """e^x in fp32 by range reduction and a degree-7 Taylor polynomial, every
    step one fp32 operation (no fused multiply-add):

      n = rint(x log2 e),  r = (x - n LN2_HI) - n LN2_LO,  |r| <= ~0.35
      p = 1 + r (1 + r (1/2! + r (1/3! + ... + r / 7!)))   (Horner)
      e^x = p * 2^n

    x > 88.5 gives +inf and x < -87 gives 0 (no subnormal results).  The
    truncated series stays within ~4e-9 relative of e^r on |r| <= 0.35."""
    x = np.asarray(x, np.float32)
    xc = np.clip(x, np.float32(-87.0), np.float32(88.5)).astype(np.float32)
    n = np.rint((xc * LOG2E).astype(np.float32)).astype(np.float32)
    r = ((xc - (n * LN2_HI).astype(np.float32)).astype(np.float32) - (n * LN2_LO).astype(np.float32)).astype(np.float32)
    p = EXP_TAYLOR[-1]
    for c in reversed(EXP_TAYLOR[:-1]):
        p = (c + (r * p).astype(np.float32)).astype(np.float32)
    p = (np.float32(1.0) + (r * p).astype(np.float32)).astype(np.float32)
    p = (np.float32(1.0) + (r * p).astype(np.float32)).astype(np.float32)
    out = np.ldexp(p, n.astype(np.int32)).astype(np.float32)
    out = np.where(x > np.float32(88.5), np.float32(np.inf), out)
    return np.where(x < np.float32(-87.0), np.float32(0.0), out).astype(np.float32)


def swiglu(G: np.ndarray, U: np.ndarray) -> np.ndarray:
    """H = silu(G) * U with silu(g) = g / (1 + e^-g): fp32 operations in that
    order, e^-g by exp32."""
    G = np.asarray(G, np.float32)
    U = np.asarray(U, np.float32)
    den = (np.float32(1.0) + exp32(-G)).astype(np.float32)
    return ((G / den).astype(np.float32) * U).astype(np.float32)


def swiglu_pairs(W_gate: np.ndarray, W_up: np.ndarray, perm_next: np.ndarray) -> np.ndarray:
    """[W_gate | W_up] with its output columns in (gate, up) pairs in the
    next layer's saliency order: column 2j is gate channel perm_next[j],
    column 2j+1 up channel perm_next[j] (Stage 3: the down projection's
    permutation propagates to the gate / up output channels).  A column
    permutation, so every per-column code and scale is unchanged."""
    Wg, Wu = np.asarray(W_gate, np.float32), np.asarray(W_up, np.float32)
    p = np.asarray(perm_next)
    W = np.empty((Wg.shape[0], 2 * Wg.shape[1]), np.float32)
    W[:, 0::2] = Wg[:, p]
    W[:, 1::2] = Wu[:, p]
    return W


def swiglu_paired(Y: np.ndarray, s_next_perm: np.ndarray) -> np.ndarray:
    """The next layer's flattened input from a paired gate|up output Y
    [M][2 d]: H[m][j] = silu(Y[m][2j]) * Y[m][2j+1] / s_next[perm_next[j]]
    (fp32 operations in that order; Stage 1: the static scale folded into
    the producer)."""
    Y = np.asarray(Y, np.float32)
    return (swiglu(Y[:, 0::2], Y[:, 1::2]) / np.asarray(s_next_perm, np.float32)).astype(np.float32)


def prepare(W: np.ndarray, X_cal: np.ndarray, r: int, fmt: str, cols=None) -> dict:
    """Offline SERQ preparation of one linear layer (Stages 1-3).

    W is [d_in][d_out] (rows = input channels).  Returns a dict with
    s, perm, W_hat, the main-path codes/scales, the dequantized salient rows D,
    the exact residual R = W-hat[:r] - D, and the residual codes/scales.
    Codes are logical [K][d_out] int arrays (not yet packed).

    ``cols`` restricts everything after the flattening scale and the
    permutation (which use all of W) to those output channels: every
    per-channel quantity depends on its own column only, so sampled outputs
    of a large layer can be evaluated without preparing the others.
    """
    assert fmt in FORMATS
    W = np.asarray(W, np.float32)
    d_in, d_out = W.shape
    assert 0 <= r <= d_in
    s = saf_scales(W, X_cal)
    perm = saliency_perm(s)
    if cols is not None:
        W = W[:, np.asarray(cols)]
        d_out = W.shape[1]
    W_hat = flatten_weights(W, s, perm)
    out = {"s": s, "perm": perm, "W_hat": W_hat, "r": r, "fmt": fmt}
    if fmt in (INT4, W4A8):
        wq, sw = sym_quant(W_hat, 4, axis=0)             # per output channel
        D = (wq[:r].astype(np.float32) * sw[None, :]).astype(np.float32)
        R = (W_hat[:r] - D).astype(np.float32)
        if r > 0:
            rq, sR = sym_quant(R, 4, axis=0)
        else:
            rq, sR = np.zeros((0, d_out), np.int8), np.zeros(d_out, np.float32)
        out.update(wq=wq, sw=sw, D=D, R=R, rq=rq, sR=sR)
    else:   # MXFP4 and MX W4A8 share the weight side
        assert d_in % MX_BLOCK == 0 and r % MX_BLOCK == 0
        wq, we = mx_quant(W_hat, axis=0)                  # codes [d_in][d_out], E8M0 [d_in/32][d_out]
        D = mx_dequant(wq[:r], we[: r // MX_BLOCK], axis=0).astype(np.float32)
        R = (W_hat[:r] - D).astype(np.float32)
        if r > 0:
            rq, re = mx_quant(R, axis=0)
        else:
            rq, re = np.zeros((0, d_out), np.uint8), np.zeros((0, d_out), np.uint8)
        out.update(wq=wq, we=we, D=D, R=R, rq=rq, re=re)
    return out


def gptq_factor(Xc: np.ndarray, damp: float = 0.01) -> np.ndarray:
    """GPTQ's upper factor U of the inverse Hessian (H^-1 = U^T U) for
    calibration activations Xc [n_cal][n]: H = 2 X^T X in fp64, a channel
    never active gets H_kk = 1, damp x the mean diagonal is added."""
    X = np.asarray(Xc, np.float64)
    n = X.shape[1]
    H = 2.0 * (X.T @ X)
    dead = np.diag(H) == 0
    H[dead, dead] = 1.0
    H += damp * np.mean(np.diag(H)) * np.eye(n)
    return np.linalg.cholesky(np.linalg.inv(H)).T


def gptq_codes(W_rows: np.ndarray, Xc: np.ndarray, sw: np.ndarray, damp: float = 0.01) -> np.ndarray:
    """GPTQ codes of the rows of W_rows [n][d_out] (input channels, in order)
    for calibration activations Xc [n_cal][n] of those channels, with fixed
    per-output-channel scales sw.  Returns int8 codes [n][d_out]."""
    W = np.asarray(W_rows, np.float64).copy()
    n, d_out = W.shape
    U = gptq_factor(Xc, damp)
    sw32 = np.asarray(sw, np.float32)
    safe = np.where(sw32 > 0, sw32, np.float32(1))
    codes = np.zeros((n, d_out), np.int8)
    for k in range(n):
        w32 = W[k].astype(np.float32)
        q = np.clip(np.rint(w32 / safe), -7, 7)
        q = np.where(sw32 > 0, q, 0)
        codes[k] = q.astype(np.int8)
        d = (q.astype(np.float32) * sw32).astype(np.float64)   # one fp32 product
        err = (W[k] - d) / U[k, k]
        W[k + 1:] -= np.outer(U[k, k + 1:], err)
    return codes


def gptq_codes_mx(W_rows: np.ndarray, Xc: np.ndarray, damp: float = 0.01):
    """GPTQ for MX weights (E2M1 elements, one E8M0 per 32 consecutive rows of
    an output channel): GPTQ with groups of 32 rows.  When a group starts,
    its E8M0 comes from its rows as the errors of the earlier rows have left
    them (their fp32 values, by mx_quant's rule); then row by row the E2M1
    code of the row's fp32 value over the group's scale, and the error
    against the exactly dequantized value, divided by U_kk, is pushed into
    the later rows.  Returns (codes [n][d_out] uint8, E8M0 [n/32][d_out])."""
    W = np.asarray(W_rows, np.float64).copy()
    n, d_out = W.shape
    assert n % MX_BLOCK == 0
    U = gptq_factor(Xc, damp)
    codes = np.zeros((n, d_out), np.uint8)
    e8m0 = np.zeros((n // MX_BLOCK, d_out), np.uint8)
    for g0 in range(0, n, MX_BLOCK):
        e = mx_scale_exponent(np.max(np.abs(W[g0:g0 + MX_BLOCK].astype(np.float32)), axis=0), 2)
        e8m0[g0 // MX_BLOCK] = (e + 127).astype(np.uint8)
        scale = np.ldexp(1.0, e)                             # exact powers of two
        for k in range(g0, g0 + MX_BLOCK):
            q = e2m1_code(W[k].astype(np.float32).astype(np.float64) / scale)
            codes[k] = q
            err = (W[k] - e2m1_value(q) * scale) / U[k, k]
            W[k + 1:] -= np.outer(U[k, k + 1:], err)
    return codes, e8m0


def prepare_gptq(W: np.ndarray, X_cal: np.ndarray, r: int, fmt: str, damp: float = 0.01, cols=None) -> dict:
    """SERQ preparation with GPTQ as the weight quantizer: the salient rows
    of W-hat_q, their scales, D and R exactly as ``prepare`` (round to
    nearest: R corrects them exactly); rows r..d_in-1 re-quantized against
    the flattened calibration activations of those channels, and Q(R)
    against those of the salient channels, by ``gptq_codes`` with the
    per-channel scales sw / sR (INT formats) or by ``gptq_codes_mx`` with
    their own E8M0 groups (MX formats).
    GPTQ treats every output channel on its own (the Hessian is shared), so
    ``cols`` restricts it to sampled output channels as it does ``prepare``."""
    assert fmt in FORMATS
    p = prepare(W, X_cal, r, fmt, cols=cols)
    Xh = flatten_acts(X_cal, p["s"], p["perm"])
    p["wq"] = p["wq"].copy()
    if r < Xh.shape[1]:
        if fmt in (INT4, W4A8):
            p["wq"][r:] = gptq_codes(p["W_hat"][r:], Xh[:, r:], p["sw"], damp)
        else:
            p["we"] = p["we"].copy()
            p["wq"][r:], p["we"][r // MX_BLOCK:] = gptq_codes_mx(p["W_hat"][r:], Xh[:, r:], damp)
    if r > 0:   # Q(R) by GPTQ too, against the salient channels (R's own scales / groups)
        if fmt in (INT4, W4A8):
            p["rq"] = gptq_codes(p["R"], Xh[:, :r], p["sR"], damp)
        else:
            p["rq"], p["re"] = gptq_codes_mx(p["R"], Xh[:, :r], damp)
    p["method"] = "gptq"
    return p


# --------------------------------------------------------------------------
# Runtime (Stage 2 inference equation)
# --------------------------------------------------------------------------

def quant_act(X_hat: np.ndarray, fmt: str):
    """On-the-fly per-token activation quantization.

    INT4: 4-bit codes and fp32 scale per token; W4A8: 8-bit; MXFP4: E2M1 codes
    with an E8M0 scale per 32 channels of each token; MX W4A8: E4M3 codes,
    same blocks.
    """
    if fmt == INT4:
        return sym_quant(X_hat, 4, axis=1)
    if fmt == W4A8:
        return sym_quant(X_hat, 8, axis=1)
    if fmt == MXW4A8:
        return mx_quant(X_hat, axis=1, elem="e4m3")
    return mx_quant(X_hat, axis=1)


def int_matmul(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Exact integer product of small-integer matrices (int64 result).

    The product runs as an fp64 BLAS matmul of integer-valued arrays: every
    product and partial sum is an integer far below 2^53, so it is exact in
    any summation order.
    """
    return np.rint(np.asarray(a, np.float64) @ np.asarray(b, np.float64)).astype(np.int64)


def int_matmul_naive(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """The same product in np.int32 through numpy's own integer matmul (a
    plain loop on one thread, no BLAS): the semantic reference the fp64-BLAS
    form is cross-checked against.  Every |sum| here is below 2^31."""
    return np.matmul(np.asarray(a, np.int32), np.asarray(b, np.int32))


def accumulators(xq: np.ndarray, prep: dict):
    """A_main = X-hat_q . W-hat_q over all d_in;  A_res = X-tilde_{s,q} . Q(R),
    X-tilde_{s,q} being the first r columns of the same codes (INT formats)."""
    r = prep["r"]
    A_main = int_matmul(xq, prep["wq"])
    A_res = int_matmul(xq[:, :r], prep["rq"])
    return A_main, A_res


def linear_int(xq, sx, prep):
    """Y = sx[m] * (sw[o] * A_main + sR[o] * A_res), evaluated in fp64."""
    A_main, A_res = accumulators(xq, prep)
    Y = np.asarray(sx, np.float64)[:, None] * (
        np.asarray(prep["sw"], np.float64)[None, :] * A_main
        + np.asarray(prep["sR"], np.float64)[None, :] * A_res)
    return Y, A_main, A_res


def linear_mx(xq, xe, prep):
    """Y = X-hat_q . W-hat_q + X-tilde_{s,q} . Q(R) with MX operands dequantized
    exactly and multiplied in fp64."""
    r = prep["r"]
    Xd = mx_dequant(xq, xe, axis=1, elem="e4m3" if prep["fmt"] == MXW4A8 else "e2m1")
    Wd = mx_dequant(prep["wq"], prep["we"], axis=0)
    Y = Xd @ Wd
    if r > 0:
        Rd = mx_dequant(prep["rq"], prep["re"], axis=0)
        Y = Y + Xd[:, :r] @ Rd
    return Y


def linear_mx_blocks(xq, xe, prep):
    """The MX layer as the block-scaled sum that defines it (OCP MX: one
    power-of-two scale per 32 elements of each operand):

        Y[m, o] = sum_b 2^(ex[m, b] + ew[b, o] - 254) * sum_{k in b} x[m, k] w[k, o]

    over the main blocks, plus the same over the r residual rows with Q(R)'s
    scales.  Each block's element products are summed exactly as integers
    (E2M1 values are multiples of 1/2, E4M3 values multiples of 2^-9) with
    numpy's integer matmul; the block terms are then added in fp64."""
    r = prep["r"]
    a8 = prep["fmt"] == MXW4A8
    fx = 512 if a8 else 2
    xv = np.rint((e4m3_value(xq) if a8 else e2m1_value(xq)) * fx).astype(np.int64)
    ex = np.asarray(xe, np.int64)

    def part(wq, we, K):
        wv = np.rint(e2m1_value(wq) * 2).astype(np.int64)
        ew = np.asarray(we, np.int64)
        out = np.zeros((xv.shape[0], wv.shape[1]))
        for b in range(K // MX_BLOCK):
            sl = slice(MX_BLOCK * b, MX_BLOCK * (b + 1))
            dot = np.matmul(xv[:, sl], wv[sl])
            out += np.ldexp(dot.astype(np.float64), ex[:, b, None] + ew[None, b, :] - 254) / (2 * fx)
        return out

    Y = part(prep["wq"], prep["we"], xv.shape[1])
    if r > 0:
        Y = Y + part(prep["rq"], prep["re"], r)
    return Y


def serq_linear(X_hat: np.ndarray, prep: dict) -> dict:
    """The whole runtime path on an already flattened, permuted input."""
    fmt = prep["fmt"]
    if fmt in MX_FORMATS:
        xq, xe = quant_act(X_hat, fmt)
        return {"xq": xq, "xscale": xe, "Y": linear_mx(xq, xe, prep)}
    xq, sx = quant_act(X_hat, fmt)
    Y, A_main, A_res = linear_int(xq, sx, prep)
    return {"xq": xq, "xscale": sx, "Y": Y, "A_main": A_main, "A_res": A_res}


# --------------------------------------------------------------------------
# L2QER comparator: Y = X_q . W_q + Q(X_q . L1_q) . L2_q (notes page, the
# two-matrix path equation; zh summary section 2.1 on its intermediate
# on-the-fly quantization).  INT4 only.
# --------------------------------------------------------------------------

def weight_error(prep: dict) -> np.ndarray:
    """E = W-hat - dequant(W-hat_q) over all d_in rows (the quantity L1 . L2
    approximates): INT formats one fp32 product and one fp32 difference per
    element; MX formats the exact dequantized value (an E2M1 value times a
    power of two, exact in fp32) and one fp32 difference."""
    if prep["fmt"] in MX_FORMATS:
        D = mx_dequant(prep["wq"], prep["we"], axis=0).astype(np.float32)
    else:
        D = (prep["wq"].astype(np.float32) * prep["sw"][None, :]).astype(np.float32)
    return (prep["W_hat"] - D).astype(np.float32)


def l2qer_factors(E: np.ndarray, k: int):
    """Rank-k truncated SVD of E, split evenly: L1 = U_k sqrt(S_k) [d_in][k],
    L2 = sqrt(S_k) V_k^T [k][d_out], both rounded once to fp32."""
    U, S, Vt = np.linalg.svd(np.asarray(E, np.float64), full_matrices=False)
    h = np.sqrt(S[:k])
    return (U[:, :k] * h[None, :]).astype(np.float32), (h[:, None] * Vt[:k]).astype(np.float32)


def l2qer_prepare(L1: np.ndarray, L2: np.ndarray) -> dict:
    """Both factors quantized like weights: 4-bit RTN, one scale per output
    column (per column of L1 over d_in, per output channel of L2 over k)."""
    l1q, sl1 = sym_quant(L1, 4, axis=0)
    l2q, sl2 = sym_quant(L2, 4, axis=0)
    return {"k": L1.shape[1], "l1q": l1q, "sl1": sl1, "l2q": l2q, "sl2": sl2}


def l2qer_intermediate(xq: np.ndarray, sx: np.ndarray, fac: dict) -> np.ndarray:
    """T = X_q . L1_q dequantized in fp32: T[m, j] = fl(sx[m] * fl(sL1[j] * A1[m, j]))."""
    A1 = int_matmul(xq, fac["l1q"]).astype(np.float32)     # exact: |A1| < 2^24
    inner = (fac["sl1"][None, :].astype(np.float32) * A1).astype(np.float32)
    return (np.asarray(sx, np.float32)[:, None] * inner).astype(np.float32)


def l2qer_linear(xq: np.ndarray, sx: np.ndarray, prep: dict, fac: dict) -> dict:
    """Y = sx sw A_main + st sL2 A_res with A_main = X_q . W_q and
    A_res = Q(T) . L2_q, Q(T) = (tq, st) the per-token 4-bit quantization of
    the intermediate; Y evaluated in fp64 from the exact accumulators."""
    A_main = int_matmul(xq, prep["wq"])
    T = l2qer_intermediate(xq, sx, fac)
    tq, st = sym_quant(T, 4, axis=1)
    A_res = int_matmul(tq, fac["l2q"])
    Y = (np.asarray(sx, np.float64)[:, None] * np.asarray(prep["sw"], np.float64)[None, :] * A_main
         + np.asarray(st, np.float64)[:, None] * np.asarray(fac["sl2"], np.float64)[None, :] * A_res)
    return {"Y": Y, "T": T, "tq": tq, "st": st, "A_main": A_main, "A_res": A_res}


# MXFP4 comparator (the format the pages compare in).  Readings: L1 and L2
# are quantized like MXFP4 weights (E8M0 per 32 elements along d_in for each
# column of L1, along k for each output channel of L2; k a multiple of 32);
# the intermediate T = X_q . L1_q is the exact sum over the 32-element blocks
# of 2^(ex + e1 - 254) sum_32 x l1 (each block term is exact; they are added
# exactly, fp64 holding every sum of these data), rounded once to fp32, and
# quantized on the fly per token like an MXFP4 activation (E8M0 per 32 of k).

def l2qer_prepare_mx(L1: np.ndarray, L2: np.ndarray) -> dict:
    """Both factors quantized like MXFP4 weights: E2M1 codes, E8M0 per 32
    elements along each column (L1 over d_in, L2 over k)."""
    assert L1.shape[1] % MX_BLOCK == 0
    l1q, l1e = mx_quant(L1, axis=0)
    l2q, l2e = mx_quant(L2, axis=0)
    return {"k": L1.shape[1], "l1q": l1q, "l1e": l1e, "l2q": l2q, "l2e": l2e, "fmt": MXFP4}


def l2qer_intermediate_mx(xq: np.ndarray, xe: np.ndarray, fac: dict) -> np.ndarray:
    """T = X_q . L1_q for MXFP4 operands: per 32-element block b the exact
    term 2^(ex[m, b] + e1[b, j] - 254) * sum_{k in b} x[m, k] l1[k, j], the
    terms summed exactly (fp64) and the sum rounded once to fp32."""
    xv = e2m1_value(xq)
    lv = e2m1_value(fac["l1q"])
    ex = np.asarray(xe, np.int64)
    e1 = np.asarray(fac["l1e"], np.int64)
    M, K = xv.shape
    T = np.zeros((M, lv.shape[1]))
    for b in range(K // MX_BLOCK):
        sl = slice(MX_BLOCK * b, MX_BLOCK * (b + 1))
        T += np.ldexp(xv[:, sl] @ lv[sl], ex[:, b, None] + e1[None, b, :] - 254)
    return T.astype(np.float32)


def l2qer_linear_mx(xq: np.ndarray, xe: np.ndarray, prep: dict, fac: dict) -> dict:
    """Y = X_q . W_q + Q(T) . L2_q for MXFP4: Q(T) = (tq, te) the per-token
    MXFP4 quantization of the intermediate; operands dequantized exactly and
    multiplied in fp64."""
    T = l2qer_intermediate_mx(xq, xe, fac)
    tq, te = mx_quant(T, axis=1)
    Xd = mx_dequant(xq, xe, axis=1)
    Y = Xd @ mx_dequant(prep["wq"], prep["we"], axis=0)
    Y = Y + mx_dequant(tq, te, axis=1) @ mx_dequant(fac["l2q"], fac["l2e"], axis=0)
    return {"Y": Y, "T": T, "tq": tq, "te": te}


def packed_l2qer(fac: dict, tiled: bool = True) -> dict:
    """The quantized factors in library storage form, k padded with zeros to
    k_pad = r_padded(k): l1q as the weights of a d_in -> k_pad INT4 layer,
    l2q as an INT4 residual block [d_out][k_pad/2]; each scale buffer is fp32
    scales followed by int32 odd-k code sums, as for W-hat_q and Q(R)."""
    d_in, k = fac["l1q"].shape
    d_out = fac["l2q"].shape[1]
    kp = r_padded(k)
    if fac.get("fmt") == MXFP4:
        # l1q as the MXFP4 weights of a d_in -> k_pad layer, l2q as an MXFP4
        # Q(R) with r_pad = k_pad: zero codes and E8M0 127 in the padding
        l1 = np.zeros((d_in, kp), np.uint8)
        l1[:, :k] = fac["l1q"]
        e1 = np.full((d_in // MX_BLOCK, kp), 127, np.uint8)
        e1[:, :k] = fac["l1e"]
        l2 = np.zeros((kp, d_out), np.uint8)
        l2[:k] = fac["l2q"]
        e2 = np.full((kp // MX_BLOCK, d_out), 127, np.uint8)
        e2[: k // MX_BLOCK] = fac["l2e"]
        out = {}
        for name, codes, e8 in (("l1", l1, e1), ("l2", l2, e2)):
            rows, srows = pack_nibbles(codes.T), np.ascontiguousarray(e8.T)
            out[name + "q"] = tile_rows(rows) if tiled else rows.reshape(-1)
            out[name + "scale"] = tile_scale_rows(srows) if tiled else srows.reshape(-1)
        return out
    l1 = np.zeros((d_in, kp), np.int8)
    l1[:, :k] = fac["l1q"]
    s1 = np.zeros(kp, np.float32)
    s1[:k] = fac["sl1"]
    l2 = np.zeros((kp, d_out), np.int8)
    l2[:k] = fac["l2q"]
    out = {}
    for name, codes, sc in (("l1", l1, s1), ("l2", l2, fac["sl2"])):
        packed = pack_int4_weight(codes.T)
        out[name + "q"] = tile_rows(packed) if tiled else packed.reshape(-1)
        sums = codes.astype(np.int64)[1::2].sum(axis=0).astype(np.int32)
        out[name + "scale"] = np.concatenate([np.asarray(sc, np.float32).view(np.uint8), sums.view(np.uint8)])
    return out


# --------------------------------------------------------------------------
# Storage layout of the library's buffers (layout version 4), written
# independently so that packed buffers can be compared byte for byte.
#   Packed matrices are K-major [rows][K/2]: elements k and k+1 (k even) share
#   byte k/2.  The weights and R (every format) are then cut into 1024-byte
#   tiles of 16 rows x 64 bytes (16 output channels x 128 elements of K); the
#   tile of row block n/16 and K chunk k/128 comes at position
#   (n/16) * (K/128) + k/128, its rows in order.  Their MX E8M0 bytes form
#   groups of four K steps (16 bytes a row) for 16 rows (tile_scale_rows).
#   Activations stay row-major.
#   MXFP4 and the W4A8 weights: element k in the low nibble for even k, the
#   high nibble for odd k; W4A8 nibbles two's complement, E2M1 = sign|exp|man.
#   INT4: one nibble of every byte is two's complement (the high one) and one
#   is offset binary, code + 8 (the low one).  Activations keep even k in the
#   high nibble, odd k in the low; weights and R keep even k in the low
#   nibble, odd k in the high.  Beside them the buffers carry the code sums the
#   offset needs removed: per output channel the sum of the odd-k codes of
#   What_q (and of Q(R)); per token the running sum, at every 128-element
#   boundary, of the even-k activation codes.
# --------------------------------------------------------------------------

def pack_nibbles(codes_rows_by_k: np.ndarray) -> np.ndarray:
    c = np.asarray(codes_rows_by_k).astype(np.int64) & 0xF
    assert c.shape[-1] % 2 == 0
    lo, hi = c[..., 0::2], c[..., 1::2]
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_nibbles for two's-complement codes."""
    p = np.asarray(packed, np.uint8).astype(np.int64)
    lo, hi = p & 0xF, p >> 4
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.int64)
    out[..., 0::2], out[..., 1::2] = lo, hi
    return np.where(out >= 8, out - 16, out).astype(np.int8)


def pack_int4_act(codes: np.ndarray) -> np.ndarray:
    """INT4 activations: byte k/2 = (x_k & 0xF) << 4 | (x_{k+1} + 8), k even."""
    c = np.asarray(codes).astype(np.int64)
    assert c.shape[-1] % 2 == 0 and np.all(np.abs(c) <= 7)
    return (((c[..., 0::2] & 0xF) << 4) | (c[..., 1::2] + 8)).astype(np.uint8)


def pack_int4_weight(codes: np.ndarray) -> np.ndarray:
    """INT4 weights and R: byte k/2 = (w_{k+1} & 0xF) << 4 | (w_k + 8), k even."""
    c = np.asarray(codes).astype(np.int64)
    assert c.shape[-1] % 2 == 0 and np.all(np.abs(c) <= 7)
    return (((c[..., 1::2] & 0xF) << 4) | (c[..., 0::2] + 8)).astype(np.uint8)


def unpack_int4_act(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, np.uint8).astype(np.int64)
    hi, lo = p >> 4, p & 0xF
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.int64)
    out[..., 0::2] = np.where(hi >= 8, hi - 16, hi)
    out[..., 1::2] = lo - 8
    return out.astype(np.int8)


def unpack_int4_weight(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, np.uint8).astype(np.int64)
    hi, lo = p >> 4, p & 0xF
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.int64)
    out[..., 0::2] = lo - 8
    out[..., 1::2] = np.where(hi >= 8, hi - 16, hi)
    return out.astype(np.int8)


def act_code_sums(xq: np.ndarray) -> np.ndarray:
    """Per token, the running sum of the even-k codes at the end of every
    128-element chunk: int32 [M][K/128]."""
    ev = np.asarray(xq, np.int64)[:, 0::2]
    M, half = ev.shape
    chunks = ev.reshape(M, half // 64, 64).sum(axis=-1)
    return np.cumsum(chunks, axis=1).astype(np.int32)


def packed_weights(prep: dict, tiled: bool = True) -> dict:
    """The prepared layer in library storage form (what serq_prepare_weights
    writes), every buffer as flat bytes: wq [d_out][d_in/2] and rq
    [d_out][r_pad/2] zero-padded (in 16 x 64-byte tiles unless tiled=False),
    and the scale buffers (INT4: fp32 scales then int32 odd-k code sums;
    W4A8: fp32 scales; MX formats: E8M0 [d_out][K/32], in groups of 16 rows x
    16 bytes unless tiled=False)."""
    fmt, r = prep["fmt"], prep["r"]
    d_in, d_out = prep["W_hat"].shape
    rp = r_padded(r)
    rq_full = np.zeros((rp, d_out), np.uint8 if fmt in MX_FORMATS else np.int8)
    rq_full[:r] = prep["rq"]
    out = {"perm": prep["perm"], "s": prep["s"]}
    if fmt in MX_FORMATS:
        out["wq"], out["rq"] = pack_nibbles(prep["wq"].T), pack_nibbles(rq_full.T)
        out["wscale"] = np.ascontiguousarray(prep["we"].T).reshape(-1)   # [d_out][d_in/32]
        rs = np.full((d_out, rp // MX_BLOCK), 127, np.uint8)              # [d_out][r_pad/32]
        rs[:, : r // MX_BLOCK] = prep["re"].T                            # padding blocks: scale 2^0
        out["rscale"] = rs.reshape(-1)
    elif fmt == W4A8:
        out["wq"], out["rq"] = pack_nibbles(prep["wq"].T), pack_nibbles(rq_full.T)
        out["wscale"] = np.asarray(prep["sw"], np.float32).view(np.uint8)
        out["rscale"] = np.asarray(prep["sR"], np.float32).view(np.uint8)
    else:
        out["wq"], out["rq"] = pack_int4_weight(prep["wq"].T), pack_int4_weight(rq_full.T)
        wsum = np.asarray(prep["wq"], np.int64)[1::2].sum(axis=0).astype(np.int32)
        rsum = rq_full.astype(np.int64)[1::2].sum(axis=0).astype(np.int32)
        out["wscale"] = np.concatenate([np.asarray(prep["sw"], np.float32).view(np.uint8), wsum.view(np.uint8)])
        out["rscale"] = np.concatenate([np.asarray(prep["sR"], np.float32).view(np.uint8), rsum.view(np.uint8)])
    for k in ("wq", "rq"):
        out[k] = tile_rows(out[k]) if tiled else out[k].reshape(-1)
    if fmt in MX_FORMATS and tiled:
        out["wscale"] = tile_scale_rows(out["wscale"].reshape(d_out, -1))
        out["rscale"] = tile_scale_rows(out["rscale"].reshape(d_out, -1)) if rp else out["rscale"]
    return out


def tile_rows(rows: np.ndarray) -> np.ndarray:
    """Row-major packed bytes [N][B] -> the tiled byte sequence: 16-row x
    64-byte tiles, row blocks outermost, then 64-byte column chunks, then the
    16 rows of the tile."""
    rows = np.asarray(rows, np.uint8)
    N, Bb = rows.shape
    assert N % 16 == 0 and Bb % 64 == 0
    return np.ascontiguousarray(rows.reshape(N // 16, 16, Bb // 64, 64).transpose(0, 2, 1, 3)).reshape(-1)


def untile_rows(flat: np.ndarray, N: int, Bb: int) -> np.ndarray:
    """Inverse of tile_rows."""
    t = np.asarray(flat, np.uint8).reshape(N // 16, Bb // 64, 16, 64)
    return np.ascontiguousarray(t.transpose(0, 2, 1, 3)).reshape(N, Bb)


def tile_scale_rows(rows: np.ndarray) -> np.ndarray:
    """MX E8M0 bytes, row-major [N][K/32] (four bytes per K step of 128) -> the
    grouped byte sequence: each row padded with zero bytes to a whole number
    of 16-byte groups (four K steps), then blocks of 16 rows outermost, groups
    next, the 16 rows of a block inside a group (16 x 16 = 256 bytes)."""
    rows = np.asarray(rows, np.uint8)
    N, Bb = rows.shape
    assert N % 16 == 0 and Bb % 4 == 0
    G = (Bb + 15) // 16
    padded = np.zeros((N, 16 * G), np.uint8)
    padded[:, :Bb] = rows
    return np.ascontiguousarray(padded.reshape(N // 16, 16, G, 16).transpose(0, 2, 1, 3)).reshape(-1)


def untile_scale_rows(flat: np.ndarray, N: int, Bb: int) -> np.ndarray:
    """Inverse of tile_scale_rows (the padding bytes dropped)."""
    G = (Bb + 15) // 16
    t = np.asarray(flat, np.uint8).reshape(N // 16, G, 16, 16)
    return np.ascontiguousarray(t.transpose(0, 2, 1, 3)).reshape(N, 16 * G)[:, :Bb]


def packed_acts(xq: np.ndarray, xscale: np.ndarray, fmt: str):
    """Quantized activations in library storage form: (codes, scale bytes).
    INT4: nibbles [M][d_in/2] and fp32 sx [M] followed by int32
    act_code_sums [M][d_in/128];  W4A8: int8 [M][d_in] and fp32 sx [M];
    MXFP4: nibbles [M][d_in/2] and E8M0 [M][d_in/32]; MX W4A8: E4M3 bytes
    [M][d_in] and E8M0 [M][d_in/32]."""
    if fmt == W4A8:
        return np.asarray(xq, np.int8).view(np.uint8), np.asarray(xscale, np.float32).view(np.uint8)
    if fmt == MXFP4:
        return pack_nibbles(xq), np.asarray(xscale, np.uint8).reshape(-1)
    if fmt == MXW4A8:   # one E4M3 byte per element [M][d_in], E8M0 [M][d_in/32]
        return np.asarray(xq, np.uint8), np.asarray(xscale, np.uint8).reshape(-1)
    sums = act_code_sums(xq)
    return pack_int4_act(xq), np.concatenate([np.asarray(xscale, np.float32).view(np.uint8),
                                              sums.reshape(-1).view(np.uint8)])
