/*
 * serq.h -- C ABI of the SERQ quantized linear layer on AMD Instinct MI355X (gfx950).
 *
 * The layer is the runtime path of SERQ (saliency-aware low-rank error
 * reconstruction), as stated by the research notes page "SERQ: Saliency-Aware
 * Low-Rank Error Reconstruction for LLM Quantization" (dihengye.cn), Stage 2
 * inference equation:
 *
 *     Y ~= Xhat_q . What_q + Xtilde_{s,q} . Q(R),   R = Wtilde_s - Q(Wtilde_s)
 *
 * i.e. one packed 4-bit main GEMM over all input channels plus one rank-r
 * residual GEMM over the first r (most salient) input channels, with no
 * intermediate quantization.  Static activation flattening and the saliency
 * permutation (Stages 1 and 3) are folded offline: the runtime input Xhat is
 * already divided by s and permuted.
 *
 * Conventions for every entry point
 *  - Returns serq_status: SERQ_OK (0) or a negative error code.  Nothing
 *    throws across the ABI.  serq_last_error() gives a text for the last
 *    failing call on the calling thread.
 *  - All argument, shape and size checks run on the host before any HIP call;
 *    a failed check launches nothing and leaves every output untouched.
 *  - The caller owns every buffer.  Host functions take host pointers; the
 *    runtime functions take device pointers and a hipStream_t passed as
 *    `void *stream` (NULL = the default stream).  The library allocates no
 *    device memory, never synchronizes the stream and returns after enqueue.
 *    HIP launch errors return SERQ_ERR_HIP with hipGetErrorString's text.
 *  - Matrices are row-major and densely packed (no row padding).
 *
 * Storage layout, version 4 (the oracle packs it independently):
 *  - Packed 4-bit matrices are K-major [rows][K/2] bytes: elements k and k+1
 *    (k even) share byte k/2.
 *  - What_q and Q(R), in every format, are stored in 1024-byte tiles of 16
 *    rows (output channels) x 64 bytes (128 elements of K): the tile holding
 *    channels n..n+15 (n % 16 == 0) and elements k..k+127 (k % 128 == 0) is
 *    tile number (n / 16) * (K / 128) + k / 128, with K = d_in for What_q and
 *    r_pad for Q(R); inside it, channel n + j occupies bytes 64 j .. 64 j + 63.
 *    One wave then reads a whole tile with one 16-byte load per lane, for
 *    the bandwidth-bound decode path and the prefill copy alike.  All
 *    activations stay row-major.
 *  - MX E8M0 bytes of What_q and Q(R) (four a channel per K step of 128,
 *    blocks in K order) are grouped by four K steps: a channel's 16 bytes of
 *    steps 4q .. 4q + 3 form one group row, the rows past the last step are
 *    zero bytes; the 16 channels n..n+15 of a group share 256 bytes, channel
 *    n + j at bytes 16 j .. 16 j + 15, and the group of channels n..n+15 and
 *    steps 4q.. is group number (n / 16) * ceil(KT / 4) + q (KT = K / 128).
 *    A channel's four steps of scales are one 16-byte load, and one step's
 *    scales of 16 channels lie within 256 bytes.
 *  - MXFP4 (weights, R, activations) and W4A8 (weights, R): element k in the
 *    low nibble for even k, the high nibble for odd k.  W4A8 nibbles are
 *    two's complement codes in [-7, 7]; MXFP4 nibbles are E2M1 codes
 *    sign|exp(2)|man(1); E8M0 scale bytes are a biased exponent (bias 127):
 *    the block scale is 2^(byte - 127).
 *  - INT4: every byte holds one two's-complement nibble (the high one) and
 *    one offset-binary nibble, code + 8 (the low one).  Activations put even
 *    k high and odd k low: byte = (x_k & 15) << 4 | (x_{k+1} + 8).  Weights
 *    and R put even k low and odd k high: byte = (w_{k+1} & 15) << 4 |
 *    (w_k + 8).  A byte-wise product of the two layouts then pairs a signed
 *    high nibble (16 v) with an unsigned low nibble (v + 8), and the exact
 *    accumulator follows from  16 A + 128 (sum of even-k activation codes +
 *    sum of odd-k weight codes), whose sums travel with the scales (below).
 *  - W4A8 activations are int8 [M][d_in].
 */
#ifndef SERQ_H
#define SERQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SERQ_LAYOUT_VERSION 4
#define SERQ_MX_BLOCK 32          /* elements per E8M0 scale */
#define SERQ_K_ALIGN 128          /* d_in must be a multiple of this */
#define SERQ_N_ALIGN 16           /* d_out must be a multiple of this */

typedef enum serq_status {
    SERQ_OK = 0,
    SERQ_ERR_INVALID_ARG = -1,    /* null pointer, unknown enum, negative size */
    SERQ_ERR_SHAPE = -2,          /* d_in/d_out/r/M violate the constraints below */
    SERQ_ERR_UNSUPPORTED = -3,    /* valid request this build does not implement */
    SERQ_ERR_BUFFER = -4,         /* a caller buffer is smaller than required */
    SERQ_ERR_HIP = -5             /* a HIP runtime call or kernel launch failed */
} serq_status;

/* Quantization settings named by the pages: W4A4 in INT4 or MXFP4, and W4A8
 * (fugumt.com abstract page; gist.science summaries, contributions), the
 * latter also in MX form. */
typedef enum serq_format {
    SERQ_FMT_INT4 = 0,            /* 4-bit weights and R, 4-bit per-token activations */
    SERQ_FMT_W4A8 = 1,            /* 4-bit weights and R, 8-bit per-token activations */
    SERQ_FMT_MXFP4 = 2,           /* E2M1 elements, E8M0 scale per 32-element block */
    SERQ_FMT_MXW4A8 = 3           /* MXFP4 weights and R, MXFP8 E4M3 activations (E8M0 per 32) */
} serq_format;

typedef enum serq_dtype {
    SERQ_DT_F32 = 0,
    SERQ_DT_BF16 = 1
} serq_dtype;

/* Sizes of one prepared layer's buffers (filled by serq_query_layout). */
typedef struct serq_layout {
    int32_t d_in;                 /* input channels (K) */
    int32_t d_out;                /* output channels (N) */
    int32_t r;                    /* salient rows reconstructed by R (0 = plain W4A4) */
    int32_t r_pad;                /* r rounded up to SERQ_K_ALIGN; R's extra rows are 0 */
    int32_t fmt;                  /* serq_format */
    int32_t layout_version;       /* SERQ_LAYOUT_VERSION */
    size_t perm_bytes;            /* int32 [d_in] */
    size_t s_bytes;               /* float [d_in] */
    size_t wq_bytes;              /* d_out * d_in / 2 bytes in 16 x 64-byte tiles (every format) */
    size_t wscale_bytes;          /* INT4: float sw [d_out] then int32 odd-k code sums [d_out];
                                     W4A8: float sw [d_out];  MX: E8M0 bytes of [d_out][d_in/32]
                                     in groups of four K steps, d_out * 16 * ceil(d_in/512) bytes */
    size_t rq_bytes;              /* d_out * r_pad / 2 bytes, laid out as wq with K = r_pad */
    size_t rscale_bytes;          /* as wscale, for R: INT4 float sR + int32 sums [d_out];
                                     W4A8 float sR [d_out];  MX E8M0 bytes of [d_out][r_pad/32]
                                     in groups, d_out * 16 * ceil(r_pad/512) bytes */
} serq_layout;

/* Fills *out for a layer.  Constraints: d_in > 0, d_in % 128 == 0;
 * d_out > 0, d_out % 16 == 0; 0 <= r <= d_in; the MX formats need r % 32 == 0.
 * Errors: SERQ_ERR_INVALID_ARG (out NULL, bad fmt), SERQ_ERR_SHAPE. */
serq_status serq_query_layout(int32_t d_in, int32_t d_out, int32_t r, serq_format fmt,
                              serq_layout *out);

/* Offline preparation of one layer, on the host (Stages 1-3 of the notes
 * page; gist.science summaries sections 2.1-2.3):
 *   s_j   = sqrt(max_c |X_cal[c][j]| / max_o |W[j][o]|)  (1 if either max is 0)
 *   perm  = channels by s descending, ties by ascending index
 *   What  = P . diag(s) . W                      (rows perm[k] scaled by s)
 *   What_q, wscale: per output channel, 4-bit RTN (INT) or MXFP4 blocks along K
 *   R     = What[:r] - dequant(What_q[:r])       (exact fp32 difference)
 *   rq, rscale: R quantized per output channel (INT) or in MX blocks along r
 * W is host fp32 [d_in][d_out] (rows = input channels); X_cal is host fp32
 * [n_cal][d_in] in original channel order, n_cal >= 1.  Every output is a
 * caller-allocated host buffer of the size serq_query_layout gives; R_out may
 * be NULL, else fp32 [r][d_out].  Inputs must be finite.
 * Errors: SERQ_ERR_INVALID_ARG, SERQ_ERR_SHAPE (L inconsistent). */
serq_status serq_prepare_weights(const serq_layout *L, const float *W, const float *X_cal,
                                 int32_t n_cal, int32_t *perm, float *s, uint8_t *wq,
                                 void *wscale, uint8_t *rq, void *rscale, float *R_out);

/* The fold the producer layer performs (Stage 1 identity, Stage 3
 * permutation), on the host: Xhat[m][k] = X[m][perm[k]] / s[perm[k]] (one
 * fp32 division).  For callers that do not fold s and perm upstream.
 * Host fp32 buffers X [M][d_in], Xhat [M][d_in]; must not overlap. */
serq_status serq_flatten_act(const float *X, int64_t M, int32_t d_in, const int32_t *perm,
                             const float *s, float *Xhat);

/* Bytes of quantized activations for M tokens: codes and per-token scales.
 * INT4: xq [M][d_in/2], xscale = float sx [M] followed by int32 [M][d_in/128]
 *       running sums of the even-k codes at every 128-element boundary;
 * W4A8: xq int8 [M][d_in], xscale float [M];
 * MXFP4: xq [M][d_in/2], xscale E8M0 [M][d_in/32];
 * MX W4A8: xq E4M3 bytes [M][d_in], xscale E8M0 [M][d_in/32]. */
serq_status serq_act_bytes(int32_t M, int32_t d_in, serq_format fmt, size_t *xq_bytes,
                           size_t *xscale_bytes);

/* On-the-fly per-token activation quantization (the notes page's
 * basic-quantization equation applied per token):
 *   INT4 / W4A8: sx[m] = max_k |Xhat[m][k]| / Q, Q = 7 / 127;
 *                xq = clip(rne(Xhat / sx), -Q, Q) with an IEEE fp32 quotient;
 *                a zero row gives sx = 0 and zero codes.
 *   MXFP4:       per 32-element block, E8M0 = floor(log2 amax) - 2 + 127,
 *                E2M1 elements rounded to nearest-even, saturating at 6.
 *   MX W4A8:     per 32-element block, E8M0 = floor(log2 amax) - 8 + 127,
 *                E4M3 elements (OCP MX FP8) rounded to nearest, ties to the
 *                even code, saturating at 448; the sign bit from the input.
 * X is a device buffer [M][d_in] of xdt; xq and xscale are device buffers of
 * serq_act_bytes' sizes.  M >= 1; d_in % 128 == 0.  Asynchronous on stream. */
serq_status serq_quant_act(const void *X, serq_dtype xdt, int32_t M, int32_t d_in,
                           serq_format fmt, uint8_t *xq, void *xscale, void *stream);

/* Producers of the layer input fused with its quantization.  The notes page
 * folds the flattening scale and the permutation into the operation that
 * produces X (Stage 1: the scale goes into the preceding normalization or
 * layer; Stage 3: the permutation is applied offline), so a layer's input is
 * X-hat = X[:, perm] / s[perm].  These two entry points compute X from the
 * producer's own input, flatten and quantize it in one pass, writing xq and
 * xscale exactly as serq_quant_act would for that X-hat (same codes, scales
 * and INT4 code sums; the fp32 operations below in this order):
 *
 * serq_rmsnorm_quant -- LLaMA RMSNorm in front of q/k/v:
 *   X[m][k] = (H[m][k] * r_m) * gamma[k],  r_m = 1 / sqrt(ms_m + eps),
 *   ms_m = (sum_k H[m][k]^2 accumulated in fp64) / d, rounded to fp32.
 * serq_swiglu_quant -- SwiGLU product in front of the down projection:
 *   X[m][k] = (G / (1 + e^-G)) * U with G = GU[m][k], U = GU[m][d + k]
 *   (GU is [M][2 d]: the gate half, then the up half, as the fused gate|up
 *   layer produces it), e^x by n = rint(x log2 e), r = (x - n ln2_hi) -
 *   n ln2_lo, a degree-7 Taylor polynomial in r (Horner, no fused
 *   multiply-add) times 2^n; +inf above 88.5, 0 below -87.
 *
 * perm (int32 [d]) is the layer's saliency order; s_p and gamma_p (fp32 [d])
 * are its flattening scales and the norm weight folded into that order once
 * per layer: s_p[k] = s[perm[k]], gamma_p[k] = gamma[perm[k]] (so that the
 * formula above reads X-hat[m][k] = ((H[m][perm[k]] r_m) gamma_p[k]) /
 * s_p[k]).  All are device buffers; H / GU are [M][d] / [M][2 d] of xdt.
 * Every buffer is 16-byte aligned; perm must be a permutation of
 * 0..d-1.  For serq_swiglu_quant perm may be NULL: the layer's permutation
 * is then folded into the producer (the gate|up layer's output channels
 * ordered by it offline, Stage 3), GU arrives in saliency order and the
 * input streams through without a gather: X-hat[m][k] = ((G[m][k] / (1 +
 * e^-G[m][k])) U[m][k]) / s_p[k].  M >= 1; d % 128 == 0 and
 * d <= 16384 (the row is held in LDS; SERQ_ERR_UNSUPPORTED beyond); eps
 * finite and >= 0; inputs finite.  Asynchronous on stream; argument errors
 * return before any HIP call. */
serq_status serq_rmsnorm_quant(const void *H, serq_dtype hdt, int32_t M, int32_t d, const float *gamma_p,
                               float eps, const int32_t *perm, const float *s_p, serq_format fmt, uint8_t *xq,
                               void *xscale, void *stream);
serq_status serq_swiglu_quant(const void *GU, serq_dtype dt, int32_t M, int32_t d, const int32_t *perm,
                              const float *s_p, serq_format fmt, uint8_t *xq, void *xscale, void *stream);

/* Workspace serq_linear needs for M tokens (quantized activations). */
size_t serq_linear_workspace_bytes(const serq_layout *L, int32_t M);

/* The runtime layer (Stage 2 inference equation): quantizes Xhat per token,
 * then one fused kernel computes for every token m and output channel o
 *   INT:  Y = sx[m] * (sw[o] * A_main[m][o] + sR[o] * A_res[m][o]),
 *         A_main = sum_{k<d_in} xq[m][k] wq[k][o],  A_res = sum_{k<r} xq[m][k] rq[k][o]
 *         (exact int32 accumulators, fp32 epilogue);
 *   MX:   Y = sum over the d_in/32 main blocks and the r/32 residual blocks of
 *         2^(ex + ew - 254) * sum_{32 k} x * w, x the E2M1 (MXFP4) or E4M3
 *         (MX W4A8) activation element and w the E2M1 weight element
 *         (fp32 accumulation).
 * The residual reuses the first r columns of the same quantized activations.
 * X (device, [M][d_in] of xdt) is the flattened, permuted input; wq, wscale,
 * rq, rscale are device copies of serq_prepare_weights' outputs; Y is device
 * fp32 [M][d_out]; workspace is device memory of at least
 * serq_linear_workspace_bytes(L, M) bytes (contents are scratch).  M >= 1.
 * Errors: SERQ_ERR_INVALID_ARG, SERQ_ERR_SHAPE, SERQ_ERR_BUFFER, SERQ_ERR_HIP. */
serq_status serq_linear(const serq_layout *L, const void *X, serq_dtype xdt, int32_t M,
                        const uint8_t *wq, const void *wscale, const uint8_t *rq,
                        const void *rscale, float *Y, void *workspace, size_t workspace_bytes,
                        void *stream);

/* The gate|up layer of a SwiGLU MLP with the SwiGLU product and the next
 * layer's folded flattening in its epilogue (SERQ notes page, Stage 1: the
 * static scale folds into the preceding layer; Stage 3: the down
 * projection's saliency permutation propagates to the gate / up output
 * channels).  L is the INT4 gate|up layer prepared with its output columns
 * in (gate, up) pairs in the next layer's saliency order: column 2 j is gate
 * channel perm_next[j], column 2 j + 1 up channel perm_next[j] (a column
 * permutation of [W_gate | W_up], which leaves every code and scale as they
 * are).  The layer's fp32 output Y (as serq_linear computes it) is not
 * written; instead
 *     H[m][j] = silu(Y[m][2 j]) * Y[m][2 j + 1] / s_next[j],
 *     silu(g) = g / (1 + e^-g),
 * in fp32 operations in that order, e^x evaluated as the fused producers
 * evaluate it (serq_swiglu_quant): H is the next layer's flattened input
 * Xhat, bit for bit what serq_flatten_act gives from the unfused layer's
 * SwiGLU.  s_next: device fp32 [d_out / 2], the next layer's s[perm[j]]; H:
 * device fp32 [M][d_out / 2].  Other arguments and errors as serq_linear,
 * plus SERQ_ERR_UNSUPPORTED outside INT4 prefill shapes of the large-tile
 * kernel (M > 128, d_in % 256 == 0, r <= 256). */
serq_status serq_linear_swiglu(const serq_layout *L, const void *X, serq_dtype xdt, int32_t M,
                               const uint8_t *wq, const void *wscale, const uint8_t *rq,
                               const void *rscale, const float *s_next, float *H, void *workspace,
                               size_t workspace_bytes, void *stream);

/* The MXFP4 gate|up layer of a SwiGLU MLP with the SwiGLU product, the next
 * layer's folded flattening and the next layer's MXFP4 activation
 * quantization in its epilogue: the previous op's epilogue emits the next
 * layer's quantized input directly (SERQ notes page, Stage 1: the static
 * scale folds into the preceding layer; Stage 3: the down projection's
 * saliency permutation propagates to the gate / up output channels).  MX
 * scales are per 32-element block, so a workgroup whose output columns hold
 * whole blocks of the next layer's input can quantize them itself.  L, X,
 * the weights, s_next and the column pairing as serq_linear_swiglu, for an
 * MXFP4 layer; with H as defined there (d_out / 2 columns), xq_next and
 * xscale_next receive exactly what serq_quant_act(H, SERQ_FMT_MXFP4) would
 * write: E2M1 codes [M][d_out / 4] bytes and E8M0 bytes [M][d_out / 64].
 * Neither Y nor H is written.  Other arguments and errors as
 * serq_linear_swiglu, plus SERQ_ERR_SHAPE when d_out is not a multiple of
 * 256 (the next layer's d_in, d_out / 2, must be a multiple of 128) and
 * SERQ_ERR_UNSUPPORTED outside the LDS-direct kernel's shapes (M > 16,
 * d_in % 512 == 0, r <= 128) or for other formats. */
serq_status serq_linear_swiglu_q(const serq_layout *L, const void *X, serq_dtype xdt, int32_t M,
                                 const uint8_t *wq, const void *wscale, const uint8_t *rq,
                                 const void *rscale, const float *s_next, uint8_t *xq_next,
                                 uint8_t *xscale_next, void *workspace, size_t workspace_bytes,
                                 void *stream);

/* Bytes of device scratch serq_linear_noalloc holds per device (64 MiB). */
#define SERQ_NOALLOC_SCRATCH_BYTES (64u << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): serq_linear
 * without a workspace argument.  The quantized activations go to a device
 * array of SERQ_NOALLOC_SCRATCH_BYTES that the library holds, one copy per
 * device, from the first call on that device until the process ends; its
 * address is looked up once per device (hipGetSymbolAddress) with that
 * device current.  The call runs on the device of `stream` (the current
 * device for NULL) and allocates nothing: no hipMalloc, hipFree or library
 * allocation.  Arguments, result and errors as serq_linear, plus
 * SERQ_ERR_BUFFER when serq_linear_workspace_bytes(L, M) exceeds
 * SERQ_NOALLOC_SCRATCH_BYTES.  Every call on one device shares that device's
 * array: calls that overlap on one device (two streams, or two host threads)
 * race and must be serialized by the caller; nothing in the array needs to
 * start at zero (each call writes all it reads). */
serq_status serq_linear_noalloc(const serq_layout *L, const void *X, serq_dtype xdt, int32_t M,
                                const uint8_t *wq, const void *wscale, const uint8_t *rq,
                                const void *rscale, float *Y, void *stream);

/* The layer's GEMM + epilogue on already quantized activations (xq, xscale as
 * serq_quant_act writes them).  For INT formats, acc_main and acc_res may be
 * device int32 [M][d_out] buffers that receive the exact accumulators A_main
 * and A_res; give both or neither (NULL, NULL).  Both must be NULL for the MX
 * formats.
 * Errors: as serq_linear. */
serq_status serq_linear_q(const serq_layout *L, const uint8_t *xq, const void *xscale,
                          int32_t M, const uint8_t *wq, const void *wscale, const uint8_t *rq,
                          const void *rscale, float *Y, int32_t *acc_main, int32_t *acc_res,
                          void *stream);

/* GPTQ preparation (all formats): as serq_prepare_weights (same outputs
 * and layout) except that rows r..d_in-1 of What_q, and Q(R), are quantized
 * by GPTQ instead of round to nearest.  The pages list RTN and GPTQ as
 * SERQ's weight quantizers (gist.science summary zh, section 3; pt summary,
 * results); the algorithm is the published one (Frantar et al., "GPTQ:
 * Accurate Post-Training Quantization for Generative Pre-trained
 * Transformers", 2022) with its lazy block updates: for What_q's rows
 * H = 2 Xhat_cal^T Xhat_cal over the flattened calibration activations of the
 * non-salient channels, for R's over the salient channels (fp64), H_kk = 0
 * set to 1, damp * mean(diag H) added to the diagonal; row by row each fp64
 * row is rounded to fp32 and quantized, and its error propagates to the
 * later rows (computed from the Cholesky factor of the reversed H in blocks
 * of 32 rows, no inverse formed).  INT formats quantize with the
 * per-channel scales sw / sR (max over the column / 7, as RTN); MX formats
 * run GPTQ with groups of 32 rows: each group's E8M0 bytes are taken, as RTN
 * takes them, from the group's rows as updated by the earlier groups when
 * the group starts, and each row gets the nearest E2M1 codes over them (its
 * error measured against the exact dequantized value).  The salient rows
 * of What_q keep their round-to-nearest codes and scales (R corrects them),
 * so D and R are those of serq_prepare_weights.  Host only, multithreaded;
 * memory d_in^2 fp64 values.
 * Errors: SERQ_ERR_UNSUPPORTED for d_in above 32768; SERQ_ERR_INVALID_ARG for
 * NULL pointers or a negative or non-finite damp; SERQ_ERR_SHAPE for n_cal < 1. */
serq_status serq_prepare_weights_gptq(const serq_layout *L, const float *W, const float *X_cal, int32_t n_cal,
                                      float damp, int32_t *perm, float *s, uint8_t *wq, void *wscale, uint8_t *rq,
                                      void *rscale, float *R_out);

/* ---------------------------------------------------------------------------
 * L2QER comparator (INT4 and MXFP4 layers).  The two-factor error
 * reconstruction the pages set SERQ against: Y = X_q . W_q + Q(X_q . L1_q) . L2_q
 * (SERQ research notes, key equations, "L2QER's two-matrix path"; the zh
 * technical summary, section 2.1: the two factors run in series and the
 * intermediate needs an on-the-fly quantization).  It shares SERQ's main path
 * (the same flattened, permuted Xhat and What_q), so only the reconstruction
 * differs.
 *
 * Offline: serq_weight_error gives E = What - dequant(What_q); the caller
 * factors it (for example a rank-k truncated SVD, L1 = U_k sqrt(S_k),
 * L2 = sqrt(S_k) V_k^T) and serq_l2qer_prepare quantizes L1 [d_in][k] and
 * L2 [k][d_out] like weights of the layer's format.
 *
 * INT4 (1 <= k <= 256): 4-bit round to nearest even, one scale per output
 * column.  serq_l2qer_intermediate computes T[m][j] = sx[m] * (sL1[j] *
 * A1[m][j]) in fp32, A1 = X_q . L1_q exact, and quantizes T per token exactly
 * like a layer input of width k_pad; serq_l2qer_linear_q computes
 *   Y = sx[m] * (sw[o] * A_main) + st[m] * (sL2[o] * A_res),
 * A_res = Q(T) . L2_q, on the large-tile kernel (M > 128, d_in a multiple of
 * 256).
 * MXFP4 (k a multiple of 32, 32 <= k <= 128): E2M1 codes with an E8M0 byte
 * per 32 elements along each column of L1 (over d_in) and of L2 (over k).  T
 * is the exact sum of the per-block products 2^(ex + e1 - 254) x . l1 rounded
 * once to fp32, quantized per token like an MXFP4 layer input of width
 * k_pad; serq_l2qer_linear_q runs the wide LDS-direct MXFP4 kernel with
 * Q(T) . L2_q in the residual's place (M > 16, d_in a multiple of 512).
 * Other shapes return SERQ_ERR_UNSUPPORTED.
 *
 * k_pad = k rounded up to 128.  Buffers (caller-owned), INT4:
 *   l1q     k_pad * d_in / 2 bytes, What_q's storage for a d_in -> k_pad layer
 *   l1scale 8 * k_pad bytes: fp32 sL1 [k_pad] then int32 odd-k code sums
 *   l2q     d_out * k_pad / 2 bytes, Q(R)'s storage with r_pad = k_pad
 *   l2scale 8 * d_out bytes: fp32 sL2 [d_out] then int32 odd-k code sums
 *   tq      M * k_pad / 2 bytes, an INT4 activation of width k_pad
 *   tscale  4 * M + 4 * M * (k_pad / 128) bytes, as an INT4 xscale
 * MXFP4:
 *   l1q     k_pad * d_in / 2 bytes, What_q's storage for a d_in -> k_pad layer
 *   l1scale k_pad * 16 * ceil(d_in / 512) bytes, its E8M0 groups
 *   l2q     d_out * 64 bytes, Q(R)'s storage with r_pad = 128
 *   l2scale d_out * 16 bytes, its E8M0 group
 *   tq      M * 64 bytes: E2M1 codes [M][128 / 2], row-major
 *   tscale  M * 4 bytes: E8M0 [M][4]
 * Both: T is an optional fp32 [M][k_pad] copy of the intermediate (NULL:
 * none).  Padding columns of L1 and rows of L2 are zero codes (INT4 with
 * zero scale, MXFP4 with E8M0 127).  Errors: SERQ_ERR_UNSUPPORTED for other
 * formats, SERQ_ERR_SHAPE for k out of range, otherwise as serq_linear.
 * ------------------------------------------------------------------------- */

/* Host, offline: E [d_in][d_out] fp32, row k the permuted input channel k. */
serq_status serq_weight_error(const serq_layout *L, const float *W, const float *X_cal, int32_t n_cal, float *E);

/* Byte sizes of l1q, l1scale, l2q, l2scale for k factor columns. */
serq_status serq_l2qer_sizes(const serq_layout *L, int32_t k, size_t sizes[4]);

/* Host, offline: quantizes the factors L1 [d_in][k], L2 [k][d_out] (row-major fp32). */
serq_status serq_l2qer_prepare(const serq_layout *L, int32_t k, const float *L1, const float *L2, uint8_t *l1q,
                               void *l1scale, uint8_t *l2q, void *l2scale);

/* Workspace serq_l2qer_linear needs for M tokens (0 on invalid arguments). */
size_t serq_l2qer_workspace_bytes(const serq_layout *L, int32_t M, int32_t k);

/* Device: Q(X_q . L1_q) from a quantized input (xq, xscale as written by
 * serq_quant_act), one kernel: the product, T and its quantization. */
serq_status serq_l2qer_intermediate(const serq_layout *L, int32_t k, const uint8_t *xq, const void *xscale,
                                    int32_t M, const uint8_t *l1q, const void *l1scale, float *T, uint8_t *tq,
                                    void *tscale, void *stream);

/* Device: the layer output from the quantized input and intermediate. */
serq_status serq_l2qer_linear_q(const serq_layout *L, int32_t k, const uint8_t *xq, const void *xscale, int32_t M,
                                const uint8_t *wq, const void *wscale, const uint8_t *tq, const void *tscale,
                                const uint8_t *l2q, const void *l2scale, float *Y, void *stream);

/* Device: the whole comparator layer from Xhat (quantization, intermediate,
 * output), all scratch in workspace. */
serq_status serq_l2qer_linear(const serq_layout *L, int32_t k, const void *X, serq_dtype xdt, int32_t M,
                              const uint8_t *wq, const void *wscale, const uint8_t *l1q, const void *l1scale,
                              const uint8_t *l2q, const void *l2scale, float *Y, void *workspace,
                              size_t workspace_bytes, void *stream);

/* Short fixed text for a status code. */
const char *serq_status_string(serq_status st);

/* Detail of the last failing call on this thread ("" if none). */
const char *serq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SERQ_H */
