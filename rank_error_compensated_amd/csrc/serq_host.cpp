// Host half of the SERQ library: argument checks, buffer sizes, the offline
// weight preparation (static activation flattening, saliency permutation,
// 4-bit RTN / MXFP4 quantization, the compensation matrix R) and the
// producer-side activation fold.
//
// Method: "SERQ: Saliency-Aware Low-Rank Error Reconstruction for LLM
// Quantization" research notes (dihengye.cn), Stages 1-3; gist.science
// technical summaries, sections 2.1-2.3.  Every value that decides a code is
// a single IEEE fp32 operation (no contraction into FMA: built with
// -ffp-contract=off), so the result is reproducible bit for bit.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <numeric>
#include <string>
#include <thread>
#include <vector>

#include "serq.h"
#include "serq_internal.h"

namespace serq {

static thread_local std::string g_last_error;

serq_status fail(serq_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

void clear_error() { g_last_error.clear(); }

static int32_t round_up(int32_t v, int32_t a) { return (v + a - 1) / a * a; }

serq_status check_format(int32_t fmt) {
    if (fmt != SERQ_FMT_INT4 && fmt != SERQ_FMT_W4A8 && fmt != SERQ_FMT_MXFP4 && fmt != SERQ_FMT_MXW4A8)
        return fail(SERQ_ERR_INVALID_ARG, "unknown serq_format %d", (int)fmt);
    return SERQ_OK;
}

serq_status make_layout(int32_t d_in, int32_t d_out, int32_t r, int32_t fmt, serq_layout *L) {
    serq_status st = check_format(fmt);
    if (st) return st;
    if (d_in <= 0 || d_in % SERQ_K_ALIGN)
        return fail(SERQ_ERR_SHAPE, "d_in=%d must be a positive multiple of %d", d_in, SERQ_K_ALIGN);
    if (d_out <= 0 || d_out % SERQ_N_ALIGN)
        return fail(SERQ_ERR_SHAPE, "d_out=%d must be a positive multiple of %d", d_out, SERQ_N_ALIGN);
    if (r < 0 || r > d_in) return fail(SERQ_ERR_SHAPE, "r=%d must lie in [0, d_in=%d]", r, d_in);
    const bool mx = fmt == SERQ_FMT_MXFP4 || fmt == SERQ_FMT_MXW4A8;
    if (mx && r % SERQ_MX_BLOCK) return fail(SERQ_ERR_SHAPE, "MX formats need r %% 32 == 0 (r=%d)", r);
    serq_layout o;
    std::memset(&o, 0, sizeof o);
    o.d_in = d_in;
    o.d_out = d_out;
    o.r = r;
    o.r_pad = round_up(r, SERQ_K_ALIGN);
    o.fmt = fmt;
    o.layout_version = SERQ_LAYOUT_VERSION;
    o.perm_bytes = sizeof(int32_t) * (size_t)d_in;
    o.s_bytes = sizeof(float) * (size_t)d_in;
    o.wq_bytes = (size_t)d_out * (size_t)(d_in / 2);
    o.rq_bytes = (size_t)d_out * (size_t)(o.r_pad / 2);
    if (mx) {   // MXFP4 weights and R for both MX formats: 16-byte groups of four K steps a row
        o.wscale_bytes = (size_t)d_out * 16 * (size_t)((d_in / SERQ_K_ALIGN + 3) / 4);
        o.rscale_bytes = (size_t)d_out * 16 * (size_t)((o.r_pad / SERQ_K_ALIGN + 3) / 4);
    } else if (fmt == SERQ_FMT_INT4) {   // fp32 scales, then int32 odd-k code sums
        o.wscale_bytes = (sizeof(float) + sizeof(int32_t)) * (size_t)d_out;
        o.rscale_bytes = (sizeof(float) + sizeof(int32_t)) * (size_t)d_out;
    } else {
        o.wscale_bytes = sizeof(float) * (size_t)d_out;
        o.rscale_bytes = sizeof(float) * (size_t)d_out;
    }
    *L = o;
    return SERQ_OK;
}

serq_status check_layout(const serq_layout *L) {
    if (!L) return fail(SERQ_ERR_INVALID_ARG, "layout is NULL");
    serq_layout ref;
    serq_status st = make_layout(L->d_in, L->d_out, L->r, L->fmt, &ref);
    if (st) return st;
    if (std::memcmp(&ref, L, sizeof ref) != 0)
        return fail(SERQ_ERR_SHAPE, "layout fields are inconsistent; fill it with serq_query_layout");
    return SERQ_OK;
}

serq_status act_bytes(int32_t M, int32_t d_in, int32_t fmt, size_t *xq, size_t *xs) {
    serq_status st = check_format(fmt);
    if (st) return st;
    if (M < 1) return fail(SERQ_ERR_SHAPE, "M=%d must be >= 1", M);
    if (d_in <= 0 || d_in % SERQ_K_ALIGN)
        return fail(SERQ_ERR_SHAPE, "d_in=%d must be a positive multiple of %d", d_in, SERQ_K_ALIGN);
    if (fmt == SERQ_FMT_INT4 && d_in > SERQ_K_ALIGN * kQuantMaxChunks)
        return fail(SERQ_ERR_UNSUPPORTED, "INT4 activations support d_in <= %d (d_in=%d)",
                    SERQ_K_ALIGN * kQuantMaxChunks, d_in);
    size_t m = (size_t)M, k = (size_t)d_in;
    if (fmt == SERQ_FMT_W4A8) {
        *xq = m * k;
        *xs = m * sizeof(float);
    } else if (fmt == SERQ_FMT_INT4) {
        *xq = m * k / 2;
        *xs = m * sizeof(float) + m * (k / SERQ_K_ALIGN) * sizeof(int32_t);
    } else if (fmt == SERQ_FMT_MXW4A8) {   // one E4M3 byte per element
        *xq = m * k;
        *xs = m * (k / SERQ_MX_BLOCK);
    } else {
        *xq = m * k / 2;
        *xs = m * k / SERQ_MX_BLOCK;
    }
    return SERQ_OK;
}

// ---------------------------------------------------------------------------
// Offline preparation
// ---------------------------------------------------------------------------

// 4-bit symmetric RTN code of x with scale s (s = amax / 7): rne(x / s) in
// fp32, clipped to [-7, 7]; a zero scale gives code 0.
static inline int rtn4(float x, float s) {
    if (!(s > 0.0f)) return 0;
    float q = std::nearbyint(x / s);
    if (q > 7.0f) q = 7.0f;
    if (q < -7.0f) q = -7.0f;
    return (int)q;
}

// OCP MX shared exponent for a block maximum: floor(log2 amax) - 2, clamped
// to [-127, 127]; 0 for an all-zero block.  floor(log2) comes from frexp.
static inline int mx_exponent(float amax) {
    if (!(amax > 0.0f)) return 0;
    int e;
    std::frexp((double)amax, &e);
    int x = e - 1 - 2;
    return std::min(127, std::max(-127, x));
}

// Nearest E2M1 code of v (already divided by the block scale); ties to the
// even code, saturation at 6, sign bit from v's sign bit.
static inline uint8_t e2m1_encode(double v) {
    static const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    double a = std::fabs(v);
    int best = 0;
    double bd = std::fabs(a - grid[0]);
    for (int i = 1; i < 8; ++i) {
        double d = std::fabs(a - grid[i]);
        if (d < bd || (d == bd && (i % 2 == 0) && (best % 2 != 0))) {
            best = i;
            bd = d;
        }
    }
    return (uint8_t)((std::signbit(v) ? 8 : 0) | best);
}

static inline double e2m1_decode(uint8_t c) {
    static const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    double m = grid[c & 7];
    return (c & 8) ? -m : m;
}

// Element k of a packed row: low nibble for even k, high for odd k.
static inline void put_nibble(uint8_t *row, int k, int code) {
    uint8_t nib = (uint8_t)(code & 0xF);
    uint8_t &b = row[k >> 1];
    if (k & 1) b = (uint8_t)((b & 0x0F) | (nib << 4));
    else b = (uint8_t)((b & 0xF0) | nib);
}

// INT4 weights / R: even k offset binary in the low nibble, odd k two's
// complement in the high nibble.
static inline void put_int4_weight(uint8_t *row, int k, int code) {
    put_nibble(row, k, (k & 1) ? code : code + 8);
}

// Row-major packed rows [n_rows][row_bytes] -> 1024-byte tiles of 16 rows x
// 64 bytes: tile (n / 16, b / 64) at index (n / 16) * (row_bytes / 64) + b / 64,
// its 16 rows in order.
static void tile_rows(const uint8_t *rows, size_t n_rows, size_t row_bytes, uint8_t *out) {
    const size_t chunks = row_bytes / 64;
    for (size_t n = 0; n < n_rows; ++n)
        for (size_t c = 0; c < chunks; ++c)
            std::memcpy(out + ((n / 16) * chunks + c) * 1024 + (n % 16) * 64, rows + n * row_bytes + c * 64, 64);
}

// MX E8M0 bytes, row-major [n_rows][row_bytes] (four a K step) -> groups of
// four K steps: each row padded with zero bytes to whole 16-byte groups;
// blocks of 16 rows outermost, then the groups, the block's 16 rows inside a
// group (256 bytes).
static void tile_scale_rows(const uint8_t *rows, size_t n_rows, size_t row_bytes, uint8_t *out) {
    const size_t groups = (row_bytes + 15) / 16;
    std::memset(out, 0, n_rows * groups * 16);
    for (size_t n = 0; n < n_rows; ++n)
        for (size_t b = 0; b < row_bytes; ++b)
            out[((n / 16) * groups + b / 16) * 256 + (n % 16) * 16 + b % 16] = rows[n * row_bytes + b];
}

// Stages 1 and 2 up to What: the flattening scale s per input channel, the
// saliency order p and What = P . diag(s) . W [d_in][d_out].
static void flatten(const serq_layout *L, const float *W, const float *X_cal, int32_t n_cal, std::vector<int32_t> &p,
                    std::vector<float> &s, std::vector<float> &Wh) {
    const int d_in = L->d_in;
    const size_t N = (size_t)L->d_out;
    std::vector<float> ax(d_in, 0.0f), aw(d_in, 0.0f);
    s.assign(d_in, 1.0f);
    for (int c = 0; c < n_cal; ++c) {
        const float *row = X_cal + (size_t)c * d_in;
        for (int j = 0; j < d_in; ++j) ax[j] = std::max(ax[j], std::fabs(row[j]));
    }
    for (int j = 0; j < d_in; ++j) {
        const float *row = W + (size_t)j * N;
        float m = 0.0f;
        for (size_t o = 0; o < N; ++o) m = std::max(m, std::fabs(row[o]));
        aw[j] = m;
    }
    for (int j = 0; j < d_in; ++j)
        if (ax[j] > 0.0f && aw[j] > 0.0f) s[j] = std::sqrt(ax[j] / aw[j]);

    // Stage 2: saliency order (largest scale first, stable).
    p.resize(d_in);
    std::iota(p.begin(), p.end(), 0);
    std::stable_sort(p.begin(), p.end(), [&](int32_t a, int32_t b) { return s[a] > s[b]; });

    // What = P . diag(s) . W  (row k is input channel perm[k] times its scale)
    Wh.resize((size_t)d_in * N);
    for (int k = 0; k < d_in; ++k) {
        const float sk = s[p[k]];
        const float *src = W + (size_t)p[k] * N;
        float *dst = Wh.data() + (size_t)k * N;
        for (size_t o = 0; o < N; ++o) dst[o] = sk * src[o];
    }
}

// GPTQ, defined further down: the factor of the Hessian of a range of
// permuted input channels, the INT codes of rows over those channels with
// fixed per-channel scales, and their MX codes with per-group E8M0 bytes.
struct GptqFactor {
    int n = 0;
    std::vector<double> Vc;   // Vc[k * n + j] = V[j][k] (j <= k), V upper with H = V V^T
};
static GptqFactor gptq_factor(const float *X_cal, int32_t n_cal, const std::vector<int32_t> &p,
                              const std::vector<float> &s, int d_in, int c0, int c1, double damp);
static void gptq_codes(const float *rows, const GptqFactor &F, size_t N, const std::vector<float> &sc,
                       std::vector<int8_t> &codes);
static void gptq_codes_mx(const float *rows, const GptqFactor &F, size_t N, std::vector<uint8_t> &codes,
                          std::vector<uint8_t> &e8);

// Offline preparation; gptq_damp < 0 quantizes What by round to nearest,
// otherwise rows r..d_in-1 by GPTQ with that dampening.
static serq_status prepare_impl(const serq_layout *L, const float *W, const float *X_cal, int32_t n_cal,
                                int32_t *perm, float *s_out, uint8_t *wq_out, void *wscale, uint8_t *rq_out,
                                void *rscale, float *R_out, double gptq_damp) {
    const int d_in = L->d_in, d_out = L->d_out, r = L->r, r_pad = L->r_pad;
    const size_t N = (size_t)d_out;
    std::vector<int32_t> p;
    std::vector<float> s, Wh;
    flatten(L, W, X_cal, n_cal, p, s, Wh);
    std::memcpy(perm, p.data(), sizeof(int32_t) * d_in);
    std::memcpy(s_out, s.data(), sizeof(float) * d_in);

    std::memset(wq_out, 0, L->wq_bytes);
    std::memset(rq_out, 0, L->rq_bytes);
    const size_t wrow = (size_t)d_in / 2, rrow = (size_t)r_pad / 2;
    std::vector<float> R((size_t)r * N);

    if (L->fmt != SERQ_FMT_MXFP4 && L->fmt != SERQ_FMT_MXW4A8) {
        const bool int4 = L->fmt == SERQ_FMT_INT4;
        auto put = int4 ? put_int4_weight : put_nibble;
        // packed row-major first, tiled at the end
        std::vector<uint8_t> wrows(N * wrow, 0), rrows(N * rrow, 0);
        if (int4) {   // offset nibbles of zero codes (R's padding rows included) are 8
            for (size_t o = 0; o < N; ++o) {
                for (int k = 0; k < d_in; k += 2) put(wrows.data() + o * wrow, k, 0);
                for (int k = 0; k < r_pad; k += 2) put(rrows.data() + o * rrow, k, 0);
            }
        }
        std::vector<int32_t> wsum(N, 0), rsum(N, 0);   // odd-k code sums
        // per-output-channel scales over all d_in rows
        std::vector<float> amax(N, 0.0f), sw(N), sR(N, 0.0f);
        for (int k = 0; k < d_in; ++k) {
            const float *row = Wh.data() + (size_t)k * N;
            for (size_t o = 0; o < N; ++o) amax[o] = std::max(amax[o], std::fabs(row[o]));
        }
        for (size_t o = 0; o < N; ++o) sw[o] = amax[o] / 7.0f;
        std::vector<int8_t> gq, gqr;
        if (gptq_damp >= 0.0 && r < d_in)
            gptq_codes(Wh.data() + (size_t)r * N, gptq_factor(X_cal, n_cal, p, s, d_in, r, d_in, gptq_damp), N, sw,
                       gq);
        for (int k = 0; k < d_in; ++k) {
            const float *row = Wh.data() + (size_t)k * N;
            for (size_t o = 0; o < N; ++o) {
                int q = (k >= r && !gq.empty()) ? (int)gq[(size_t)(k - r) * N + o] : rtn4(row[o], sw[o]);
                put(wrows.data() + o * wrow, k, q);
                if (k & 1) wsum[o] += q;
                if (k < r) {
                    float d = (float)q * sw[o];         // dequantized salient weight
                    R[(size_t)k * N + o] = row[o] - d;  // exact (Sterbenz)
                }
            }
        }
        if (r > 0) {
            std::fill(amax.begin(), amax.end(), 0.0f);
            for (int k = 0; k < r; ++k)
                for (size_t o = 0; o < N; ++o) amax[o] = std::max(amax[o], std::fabs(R[(size_t)k * N + o]));
            for (size_t o = 0; o < N; ++o) sR[o] = amax[o] / 7.0f;
            // GPTQ, if asked for, quantizes R too, against the salient channels
            if (gptq_damp >= 0.0)
                gptq_codes(R.data(), gptq_factor(X_cal, n_cal, p, s, d_in, 0, r, gptq_damp), N, sR, gqr);
            for (int k = 0; k < r; ++k)
                for (size_t o = 0; o < N; ++o) {
                    const int q = gqr.empty() ? rtn4(R[(size_t)k * N + o], sR[o]) : (int)gqr[(size_t)k * N + o];
                    put(rrows.data() + o * rrow, k, q);
                    if (k & 1) rsum[o] += q;
                }
        }
        tile_rows(wrows.data(), N, wrow, wq_out);
        tile_rows(rrows.data(), N, rrow, rq_out);
        std::memcpy(wscale, sw.data(), sizeof(float) * N);
        std::memcpy(rscale, sR.data(), sizeof(float) * N);
        if (int4) {
            std::memcpy((uint8_t *)wscale + sizeof(float) * N, wsum.data(), sizeof(int32_t) * N);
            std::memcpy((uint8_t *)rscale + sizeof(float) * N, rsum.data(), sizeof(int32_t) * N);
        }
    } else {
        // MX blocks of 32 rows per output channel; codes and E8M0 bytes
        // row-major first, tiled and grouped at the end
        const int kb = d_in / SERQ_MX_BLOCK, rb = r_pad / SERQ_MX_BLOCK;
        std::vector<uint8_t> wrows(N * wrow, 0), rrows(N * rrow, 0), werows(N * (size_t)kb, 0);
        std::vector<uint8_t> rerows(N * (size_t)rb, 127);   // padding blocks r..r_pad: scale 2^0
        uint8_t *wq = wrows.data(), *rq = rrows.data(), *we = werows.data(), *re = rerows.data();
        std::vector<float> bmax(N);
        auto quant_blocks = [&](const float *src, int rows, uint8_t *codes, size_t crow, uint8_t *sc,
                                int sc_row, float *deq) {
            for (int b = 0; b < rows / SERQ_MX_BLOCK; ++b) {
                std::fill(bmax.begin(), bmax.end(), 0.0f);
                for (int k = b * SERQ_MX_BLOCK; k < (b + 1) * SERQ_MX_BLOCK; ++k)
                    for (size_t o = 0; o < N; ++o) bmax[o] = std::max(bmax[o], std::fabs(src[(size_t)k * N + o]));
                for (size_t o = 0; o < N; ++o) {
                    int e = mx_exponent(bmax[o]);
                    sc[o * (size_t)sc_row + b] = (uint8_t)(e + 127);
                    double scale = std::ldexp(1.0, e);
                    for (int k = b * SERQ_MX_BLOCK; k < (b + 1) * SERQ_MX_BLOCK; ++k) {
                        uint8_t c = e2m1_encode((double)src[(size_t)k * N + o] / scale);
                        put_nibble(codes + o * crow, k, c);
                        if (deq) deq[(size_t)k * N + o] = (float)(e2m1_decode(c) * scale);
                    }
                }
            }
        };
        std::vector<float> D((size_t)r * N);
        quant_blocks(Wh.data(), r, wq, wrow, we, kb, D.data());
        // the remaining main-path blocks (rows r..d_in) need no dequantized
        // copy; GPTQ, if asked for, quantizes them instead of round to nearest
        if (gptq_damp >= 0.0 && r < d_in) {
            std::vector<uint8_t> gc, ge;
            gptq_codes_mx(Wh.data() + (size_t)r * N, gptq_factor(X_cal, n_cal, p, s, d_in, r, d_in, gptq_damp), N, gc,
                          ge);
            const int b0 = r / SERQ_MX_BLOCK;
            for (size_t o = 0; o < N; ++o) {
                for (int k = r; k < d_in; ++k) put_nibble(wq + o * wrow, k, gc[(size_t)(k - r) * N + o]);
                for (int b = b0; b < kb; ++b) we[o * (size_t)kb + b] = ge[(size_t)(b - b0) * N + o];
            }
        } else {
            const int b0 = r / SERQ_MX_BLOCK;
            for (int b = b0; b < kb; ++b) {
                std::fill(bmax.begin(), bmax.end(), 0.0f);
                for (int k = b * SERQ_MX_BLOCK; k < (b + 1) * SERQ_MX_BLOCK; ++k)
                    for (size_t o = 0; o < N; ++o) bmax[o] = std::max(bmax[o], std::fabs(Wh[(size_t)k * N + o]));
                for (size_t o = 0; o < N; ++o) {
                    int e = mx_exponent(bmax[o]);
                    we[o * (size_t)kb + b] = (uint8_t)(e + 127);
                    double scale = std::ldexp(1.0, e);
                    for (int k = b * SERQ_MX_BLOCK; k < (b + 1) * SERQ_MX_BLOCK; ++k)
                        put_nibble(wq + o * wrow, k, e2m1_encode((double)Wh[(size_t)k * N + o] / scale));
                }
            }
        }
        for (size_t i = 0; i < (size_t)r * N; ++i) R[i] = Wh[i] - D[i];
        if (r > 0 && gptq_damp >= 0.0) {   // GPTQ for Q(R) too, against the salient channels
            std::vector<uint8_t> gc, ge;
            gptq_codes_mx(R.data(), gptq_factor(X_cal, n_cal, p, s, d_in, 0, r, gptq_damp), N, gc, ge);
            for (size_t o = 0; o < N; ++o) {
                for (int k = 0; k < r; ++k) put_nibble(rq + o * rrow, k, gc[(size_t)k * N + o]);
                for (int b = 0; b < r / SERQ_MX_BLOCK; ++b) re[o * (size_t)rb + b] = ge[(size_t)b * N + o];
            }
        } else if (r > 0) {
            quant_blocks(R.data(), r, rq, rrow, re, rb, nullptr);
        }
        tile_rows(wrows.data(), N, wrow, wq_out);
        tile_rows(rrows.data(), N, rrow, rq_out);
        tile_scale_rows(werows.data(), N, (size_t)kb, (uint8_t *)wscale);
        tile_scale_rows(rerows.data(), N, (size_t)rb, (uint8_t *)rscale);
    }
    if (R_out && r > 0) std::memcpy(R_out, R.data(), sizeof(float) * (size_t)r * N);
    return SERQ_OK;
}

serq_status prepare(const serq_layout *L, const float *W, const float *X_cal, int32_t n_cal,
                    int32_t *perm, float *s_out, uint8_t *wq, void *wscale, uint8_t *rq,
                    void *rscale, float *R_out) {
    return prepare_impl(L, W, X_cal, n_cal, perm, s_out, wq, wscale, rq, rscale, R_out, -1.0);
}

// ---------------------------------------------------------------------------
// GPTQ (the published algorithm of Frantar et al., "GPTQ: Accurate
// Post-Training Quantization for Generative Pre-trained Transformers", 2022,
// with its lazy block updates) for rows over a range of permuted input
// channels: H = 2 Xhat^T Xhat over the flattened calibration activations of
// those channels (fp64); a channel never active gets H_kk = 1; damp x the mean
// diagonal is added.  The textbook form runs row by row with U, the upper
// Cholesky factor of H^-1: the row is quantized and its error divided by
// U_kk is subtracted from the later rows with weights U_kj.  With V upper and
// H = V V^T (V = J L' J for the lower Cholesky factor L' of the reversed J H
// J), U = V^-1, and the row each step quantizes works out to
//     w_k + (sum_{j<k} V[j][k] (w_j - d_j)) / V[k][k]
// with w the original rows and d_j the dequantized codes already decided, so
// no inverse is formed: the rows are taken in blocks of 32, a block's sums
// over all earlier rows are one product of V's columns with the earlier
// errors, and the sums inside the block follow row by row.  (For MX, the
// group's rows as the earlier groups have left them -- from which its E8M0
// bytes are taken -- are w + z with V_g^T z = the same sums, V_g the group's
// diagonal block, a forward substitution.)  fp64 throughout; each row is
// rounded once to fp32 and its code decided with the round-to-nearest rule.
// ---------------------------------------------------------------------------

static unsigned worker_count() {
    const unsigned hw = std::thread::hardware_concurrency();
    return hw == 0 ? 1u : std::min(hw, 16u);
}

// Runs f(lo, hi) over [0, n) split into contiguous ranges on worker threads.
template <class F>
static void parallel_ranges(size_t n, F f) {
    const unsigned T = (unsigned)std::min<size_t>(worker_count(), std::max<size_t>(n, 1));
    if (T <= 1) {
        f((size_t)0, n);
        return;
    }
    std::vector<std::thread> th;
    for (unsigned t = 0; t < T; ++t) {
        const size_t lo = n * t / T, hi = n * (t + 1) / T;
        th.emplace_back([=] { f(lo, hi); });
    }
    for (auto &x : th) x.join();
}

// Runs f(item) for items 0..n-1 on worker threads, handed out one at a time
// (for items of very different sizes).
template <class F>
static void parallel_items(size_t n, F f) {
    const unsigned T = (unsigned)std::min<size_t>(worker_count(), std::max<size_t>(n, 1));
    std::atomic<size_t> next{0};
    auto work = [&] {
        for (size_t it; (it = next.fetch_add(1)) < n;) f(it);
    };
    if (T <= 1) {
        work();
        return;
    }
    std::vector<std::thread> th;
    for (unsigned t = 0; t < T; ++t) th.emplace_back(work);
    for (auto &x : th) x.join();
}

// Lower Cholesky factor of the row-major n x n matrix A (lower triangle
// used), in place, by column panels of CB: the panel's diagonal block and
// the rows below it, then the trailing rows minus the panel's products.
// Every element receives its subtractions one at a time in increasing k,
// so the result is the unblocked algorithm's, bit for bit.
static void cholesky_lower(std::vector<double> &A, int n) {
    constexpr int CB = 64, RT = 32, CT = 256;   // panel width; row and column tiles of the trailing update
    std::vector<double> PT((size_t)CB * n);     // the panel transposed: PT[k][j] = A[j][k0 + k]
    for (int k0 = 0; k0 < n; k0 += CB) {
        const int k1 = std::min(k0 + CB, n), kb = k1 - k0;
        for (int i = k0; i < k1; ++i) {   // diagonal block
            double *Ai = A.data() + (size_t)i * n;
            for (int j = k0; j <= i; ++j) {
                const double *Aj = A.data() + (size_t)j * n;
                double acc = Ai[j];
                for (int k = k0; k < j; ++k) acc -= Ai[k] * Aj[k];
                Ai[j] = (j == i) ? std::sqrt(acc) : acc / Aj[j];
            }
        }
        if (k1 == n) break;
        parallel_ranges((size_t)(n - k1), [&](size_t lo, size_t hi) {   // the panel's rows below it
            for (size_t ii = lo; ii < hi; ++ii) {
                double *Ai = A.data() + (size_t)(k1 + ii) * n;
                for (int j = k0; j < k1; ++j) {
                    const double *Aj = A.data() + (size_t)j * n;
                    double acc = Ai[j];
                    for (int k = k0; k < j; ++k) acc -= Ai[k] * Aj[k];
                    Ai[j] = acc / Aj[j];
                }
            }
        });
        parallel_ranges((size_t)(n - k1), [&](size_t lo, size_t hi) {
            for (size_t j = k1 + lo; j < k1 + hi; ++j)
                for (int k = 0; k < kb; ++k) PT[(size_t)k * n + j] = A[j * (size_t)n + k0 + k];
        });
        // trailing rows: A[i][j] -= sum_k A[i][k0 + k] PT[k][j] for k1 <= j <= i,
        // by row tiles (largest first) and column tiles kept in cache
        const int tiles = (n - k1 + RT - 1) / RT;
        parallel_items((size_t)tiles, [&](size_t it) {
            const int i0 = k1 + (tiles - 1 - (int)it) * RT, i1 = std::min(i0 + RT, n);
            for (int j0 = k1; j0 < i1; j0 += CT) {
                const int j1 = std::min(j0 + CT, i1);
                for (int i = i0; i < i1; ++i) {
                    double *Ai = A.data() + (size_t)i * n;
                    const int je = std::min(j1, i + 1);
                    for (int k = 0; k < kb; ++k) {
                        const double a = Ai[k0 + k];
                        const double *P = PT.data() + (size_t)k * n;
                        for (int j = j0; j < je; ++j) Ai[j] -= a * P[j];
                    }
                }
            }
        });
    }
}

static GptqFactor gptq_factor(const float *X_cal, int32_t n_cal, const std::vector<int32_t> &p,
                              const std::vector<float> &s, int d_in, int c0, int c1, double damp) {
    (void)d_in;
    const int n = c1 - c0;
    // flattened calibration activations of the channels, channel-major,
    // reversed (row i = channel c1 - 1 - i; one fp32 division each)
    std::vector<double> XT((size_t)n * n_cal);
    for (int i = 0; i < n; ++i) {
        const int ch = p[c1 - 1 - i];
        for (int c = 0; c < n_cal; ++c) XT[(size_t)i * n_cal + c] = (double)(X_cal[(size_t)c * d_in + ch] / s[ch]);
    }
    // A = J H J (the Hessian in reversed channel order), lower triangle
    std::vector<double> A((size_t)n * n, 0.0);
    parallel_items((size_t)n, [&](size_t i) {
        const double *xi = XT.data() + i * n_cal;
        for (size_t j = 0; j <= i; ++j) {
            const double *xj = XT.data() + j * n_cal;
            double acc = 0.0;
            for (int c = 0; c < n_cal; ++c) acc += xi[c] * xj[c];
            A[i * n + j] = 2.0 * acc;
        }
    });
    XT.clear();
    XT.shrink_to_fit();
    double mean = 0.0;
    for (int i = 0; i < n; ++i) {
        double &d = A[(size_t)i * n + i];
        if (d == 0.0) d = 1.0;
        mean += d;
    }
    mean /= n;
    for (int i = 0; i < n; ++i) A[(size_t)i * n + i] += damp * mean;
    cholesky_lower(A, n);   // L' of J H J
    // V[j][k] = L'[n-1-j][n-1-k] (j <= k); stored as Vc[k][j], the
    // reflection of the lower triangle across its anti-diagonal, in place
    for (int k = 0; k < n; ++k)
        for (int j = 0; j <= k; ++j) {
            const size_t a = (size_t)k * n + j, b = (size_t)(n - 1 - j) * n + (n - 1 - k);
            if (a < b) std::swap(A[a], A[b]);
        }
    GptqFactor F;
    F.n = n;
    F.Vc = std::move(A);
    return F;
}

// The sums s_k = sum_{j < b} V[j][k] delta_j for the block rows k = b ..
// b + nb - 1 (delta rows of w columns, row-major): one pass over the earlier
// rows, each contributing to every block row.
static void block_sums(const GptqFactor &F, const std::vector<double> &delta, size_t w, int b, int nb,
                       std::vector<double> &y) {
    std::fill(y.begin(), y.begin() + (size_t)nb * w, 0.0);
    for (int j = 0; j < b; ++j) {
        const double *dj = delta.data() + (size_t)j * w;
        for (int kk = 0; kk < nb; ++kk) {
            const double v = F.Vc[(size_t)(b + kk) * F.n + j];
            if (v == 0.0) continue;
            double *yk = y.data() + (size_t)kk * w;
            for (size_t o = 0; o < w; ++o) yk[o] += v * dj[o];
        }
    }
}

// INT codes of rows [n][N] (fp32) over the factor's channels with the fixed
// per-column scales sc; output columns are independent, so they split over
// threads.
static void gptq_codes(const float *rows, const GptqFactor &F, size_t N, const std::vector<float> &sc,
                       std::vector<int8_t> &codes) {
    const int n = F.n, B = SERQ_MX_BLOCK;
    codes.assign((size_t)n * N, 0);
    parallel_ranges(N, [&](size_t lo, size_t hi) {
        const size_t w = hi - lo;
        if (w == 0) return;
        std::vector<double> delta((size_t)n * w), y((size_t)B * w), acc(w);
        for (int b = 0; b < n; b += B) {
            const int nb = std::min(B, n - b);
            block_sums(F, delta, w, b, nb, y);
            for (int kk = 0; kk < nb; ++kk) {
                const int k = b + kk;
                const double *Vk = F.Vc.data() + (size_t)k * n;
                for (size_t o = 0; o < w; ++o) acc[o] = y[(size_t)kk * w + o];
                for (int j = b; j < k; ++j) {
                    const double v = Vk[j], *dj = delta.data() + (size_t)j * w;
                    for (size_t o = 0; o < w; ++o) acc[o] += v * dj[o];
                }
                const float *wk = rows + (size_t)k * N + lo;
                double *dk = delta.data() + (size_t)k * w;
                for (size_t o = 0; o < w; ++o) {
                    const float x = (float)((double)wk[o] + acc[o] / Vk[k]);
                    const int q = rtn4(x, sc[lo + o]);
                    codes[(size_t)k * N + lo + o] = (int8_t)q;
                    dk[o] = (double)wk[o] - (double)((float)q * sc[lo + o]);
                }
            }
        }
    });
}

// MX codes of rows [n][N] (n a multiple of 32), GPTQ with groups of 32 rows:
// when a group starts, each output channel's E8M0 is taken, by the
// round-to-nearest rule, from the group's rows as the earlier groups have
// left them (fp32); then row by row the E2M1 code of the row's fp32 value
// over the group scale, its error measured against the exact dequantized
// value.
static void gptq_codes_mx(const float *rows, const GptqFactor &F, size_t N, std::vector<uint8_t> &codes,
                          std::vector<uint8_t> &e8) {
    const int n = F.n, G = SERQ_MX_BLOCK;
    codes.assign((size_t)n * N, 0);
    e8.assign((size_t)(n / G) * N, 127);
    parallel_ranges(N, [&](size_t lo, size_t hi) {
        const size_t w = hi - lo;
        if (w == 0) return;
        std::vector<double> delta((size_t)n * w), y((size_t)G * w), z((size_t)G * w), acc(w), scale(w);
        for (int g0 = 0; g0 < n; g0 += G) {
            block_sums(F, delta, w, g0, G, y);
            // the group's rows as the earlier groups left them: w + z, V_g^T z = y
            for (int kk = 0; kk < G; ++kk) {
                const double *Vk = F.Vc.data() + (size_t)(g0 + kk) * n;
                double *zk = z.data() + (size_t)kk * w;
                for (size_t o = 0; o < w; ++o) zk[o] = y[(size_t)kk * w + o];
                for (int m = 0; m < kk; ++m) {
                    const double v = Vk[g0 + m], *zm = z.data() + (size_t)m * w;
                    for (size_t o = 0; o < w; ++o) zk[o] -= v * zm[o];
                }
                for (size_t o = 0; o < w; ++o) zk[o] /= Vk[g0 + kk];
            }
            for (size_t o = 0; o < w; ++o) {
                float bmax = 0.0f;
                for (int kk = 0; kk < G; ++kk)
                    bmax = std::max(bmax, std::fabs((float)((double)rows[(size_t)(g0 + kk) * N + lo + o] +
                                                            z[(size_t)kk * w + o])));
                const int e = mx_exponent(bmax);
                e8[(size_t)(g0 / G) * N + lo + o] = (uint8_t)(e + 127);
                scale[o] = std::ldexp(1.0, e);
            }
            for (int kk = 0; kk < G; ++kk) {
                const int k = g0 + kk;
                const double *Vk = F.Vc.data() + (size_t)k * n;
                for (size_t o = 0; o < w; ++o) acc[o] = y[(size_t)kk * w + o];
                for (int j = g0; j < k; ++j) {
                    const double v = Vk[j], *dj = delta.data() + (size_t)j * w;
                    for (size_t o = 0; o < w; ++o) acc[o] += v * dj[o];
                }
                const float *wk = rows + (size_t)k * N + lo;
                double *dk = delta.data() + (size_t)k * w;
                for (size_t o = 0; o < w; ++o) {
                    const float x = (float)((double)wk[o] + acc[o] / Vk[k]);
                    const uint8_t c = e2m1_encode((double)x / scale[o]);
                    codes[(size_t)k * N + lo + o] = c;
                    dk[o] = (double)wk[o] - e2m1_decode(c) * scale[o];
                }
            }
        }
    });
}

// ---------------------------------------------------------------------------
// L2QER comparator, offline side
// ---------------------------------------------------------------------------

// Largest d_in GPTQ prepares (its Hessian factor is d_in^2 fp64: 8 GiB here).
constexpr int kGptqMaxRows = 32768;

static int32_t l2qer_kpad(int32_t k) { return round_up(k, SERQ_K_ALIGN); }

static serq_status check_l2qer_host(const serq_layout *L, int32_t k) {
    serq_status st = check_layout(L);
    if (st) return st;
    if (L->fmt == SERQ_FMT_MXFP4) {   // MXFP4: k a whole number of 32-element blocks, one K step
        if (k < 32 || k > 128 || k % SERQ_MX_BLOCK)
            return fail(SERQ_ERR_SHAPE, "MXFP4: k=%d must be a multiple of 32 in [32, 128]", k);
        return SERQ_OK;
    }
    if (L->fmt != SERQ_FMT_INT4)
        return fail(SERQ_ERR_UNSUPPORTED, "the L2QER comparator is built for INT4 and MXFP4 layers");
    if (k < 1 || k > 256) return fail(SERQ_ERR_SHAPE, "k=%d must be in [1, 256]", k);
    return SERQ_OK;
}

// E = What - dequant(What_q): the per-channel 4-bit code times its scale
// (one fp32 product), subtracted from What (one fp32 difference).
serq_status weight_error(const serq_layout *L, const float *W, const float *X_cal, int32_t n_cal, float *E) {
    const int d_in = L->d_in;
    const size_t N = (size_t)L->d_out;
    std::vector<int32_t> p;
    std::vector<float> s, Wh;
    flatten(L, W, X_cal, n_cal, p, s, Wh);
    if (L->fmt == SERQ_FMT_MXFP4 || L->fmt == SERQ_FMT_MXW4A8) {
        // MX round to nearest per 32-row block; the dequantized value is
        // exact in fp32, so one fp32 difference
        std::vector<float> bmax(N);
        for (int b = 0; b < d_in / SERQ_MX_BLOCK; ++b) {
            std::fill(bmax.begin(), bmax.end(), 0.0f);
            for (int k = b * SERQ_MX_BLOCK; k < (b + 1) * SERQ_MX_BLOCK; ++k)
                for (size_t o = 0; o < N; ++o) bmax[o] = std::max(bmax[o], std::fabs(Wh[(size_t)k * N + o]));
            for (size_t o = 0; o < N; ++o) {
                const double scale = std::ldexp(1.0, mx_exponent(bmax[o]));
                for (int k = b * SERQ_MX_BLOCK; k < (b + 1) * SERQ_MX_BLOCK; ++k) {
                    const float w = Wh[(size_t)k * N + o];
                    const float d = (float)(e2m1_decode(e2m1_encode((double)w / scale)) * scale);
                    E[(size_t)k * N + o] = w - d;
                }
            }
        }
        return SERQ_OK;
    }
    std::vector<float> amax(N, 0.0f), sw(N);
    for (int k = 0; k < d_in; ++k)
        for (size_t o = 0; o < N; ++o) amax[o] = std::max(amax[o], std::fabs(Wh[(size_t)k * N + o]));
    for (size_t o = 0; o < N; ++o) sw[o] = amax[o] / 7.0f;
    for (int k = 0; k < d_in; ++k)
        for (size_t o = 0; o < N; ++o) {
            const float w = Wh[(size_t)k * N + o];
            const float d = (float)rtn4(w, sw[o]) * sw[o];
            E[(size_t)k * N + o] = w - d;
        }
    return SERQ_OK;
}

// One factor quantized like weights: src [K][N] row-major, 4-bit per output
// column n over its K rows; written as N_pad packed rows of K_pad elements
// (INT4 weight nibbles, zero codes in the padding), tiled, plus fp32 scales
// [N_pad] and int32 odd-k code sums [N_pad].
static void quantize_factor(const float *src, int K, int N, int K_pad, int N_pad, uint8_t *packed, void *scale) {
    const size_t rb = (size_t)K_pad / 2;
    std::vector<uint8_t> rows((size_t)N_pad * rb, 0);
    std::vector<float> amax(N_pad, 0.0f), sc(N_pad, 0.0f);
    std::vector<int32_t> sums(N_pad, 0);
    for (int n = 0; n < N_pad; ++n)
        for (int k = 0; k < K_pad; k += 2) put_int4_weight(rows.data() + n * rb, k, 0);
    for (int k = 0; k < K; ++k)
        for (int n = 0; n < N; ++n) amax[n] = std::max(amax[n], std::fabs(src[(size_t)k * N + n]));
    for (int n = 0; n < N; ++n) sc[n] = amax[n] / 7.0f;
    for (int k = 0; k < K; ++k)
        for (int n = 0; n < N; ++n) {
            const int q = rtn4(src[(size_t)k * N + n], sc[n]);
            put_int4_weight(rows.data() + n * rb, k, q);
            if (k & 1) sums[n] += q;
        }
    tile_rows(rows.data(), (size_t)N_pad, rb, packed);
    std::memcpy(scale, sc.data(), sizeof(float) * N_pad);
    std::memcpy((uint8_t *)scale + sizeof(float) * N_pad, sums.data(), sizeof(int32_t) * N_pad);
}

// One factor quantized like MXFP4 weights: src [K][N] row-major, E8M0 per 32
// rows of each column n; written as N_pad code rows of K_pad elements (zero
// codes and E8M0 127 in the padding), tiled, and their E8M0 bytes grouped.
static void quantize_factor_mx(const float *src, int K, int N, int K_pad, int N_pad, uint8_t *packed,
                               uint8_t *scale) {
    const size_t rb = (size_t)K_pad / 2, sb = (size_t)K_pad / SERQ_MX_BLOCK;
    std::vector<uint8_t> rows((size_t)N_pad * rb, 0), srows((size_t)N_pad * sb, 127);
    for (int b = 0; b < K / SERQ_MX_BLOCK; ++b)
        for (int n = 0; n < N; ++n) {
            float bmax = 0.0f;
            for (int k = b * SERQ_MX_BLOCK; k < (b + 1) * SERQ_MX_BLOCK; ++k)
                bmax = std::max(bmax, std::fabs(src[(size_t)k * N + n]));
            const int e = mx_exponent(bmax);
            srows[(size_t)n * sb + b] = (uint8_t)(e + 127);
            const double sc = std::ldexp(1.0, e);
            for (int k = b * SERQ_MX_BLOCK; k < (b + 1) * SERQ_MX_BLOCK; ++k)
                put_nibble(rows.data() + (size_t)n * rb, k, e2m1_encode((double)src[(size_t)k * N + n] / sc));
        }
    tile_rows(rows.data(), (size_t)N_pad, rb, packed);
    tile_scale_rows(srows.data(), (size_t)N_pad, sb, scale);
}

}  // namespace serq

using namespace serq;

extern "C" {

serq_status serq_query_layout(int32_t d_in, int32_t d_out, int32_t r, serq_format fmt,
                              serq_layout *out) {
    clear_error();
    if (!out) return fail(SERQ_ERR_INVALID_ARG, "out is NULL");
    return make_layout(d_in, d_out, r, (int32_t)fmt, out);
}

serq_status serq_prepare_weights(const serq_layout *L, const float *W, const float *X_cal,
                                 int32_t n_cal, int32_t *perm, float *s, uint8_t *wq,
                                 void *wscale, uint8_t *rq, void *rscale, float *R_out) {
    clear_error();
    serq_status st = check_layout(L);
    if (st) return st;
    if (!W || !X_cal || !perm || !s || !wq || !wscale || !rq || !rscale)
        return fail(SERQ_ERR_INVALID_ARG, "a required pointer is NULL");
    if (n_cal < 1) return fail(SERQ_ERR_SHAPE, "n_cal=%d must be >= 1", n_cal);
    return prepare(L, W, X_cal, n_cal, perm, s, wq, wscale, rq, rscale, R_out);
}

serq_status serq_prepare_weights_gptq(const serq_layout *L, const float *W, const float *X_cal, int32_t n_cal,
                                      float damp, int32_t *perm, float *s, uint8_t *wq, void *wscale, uint8_t *rq,
                                      void *rscale, float *R_out) {
    clear_error();
    serq_status st = check_layout(L);
    if (st) return st;
    if (!W || !X_cal || !perm || !s || !wq || !wscale || !rq || !rscale)
        return fail(SERQ_ERR_INVALID_ARG, "a required pointer is NULL");
    if (n_cal < 1) return fail(SERQ_ERR_SHAPE, "n_cal=%d must be >= 1", n_cal);
    if (!(damp >= 0.0f) || !std::isfinite(damp)) return fail(SERQ_ERR_INVALID_ARG, "damp must be finite and >= 0");
    if (L->d_in > kGptqMaxRows)   // the factor of the Hessian is d_in^2 fp64 values
        return fail(SERQ_ERR_UNSUPPORTED, "GPTQ preparation supports d_in up to %d (got %d)", kGptqMaxRows, L->d_in);
    return prepare_impl(L, W, X_cal, n_cal, perm, s, wq, wscale, rq, rscale, R_out, (double)damp);
}

serq_status serq_weight_error(const serq_layout *L, const float *W, const float *X_cal, int32_t n_cal, float *E) {
    clear_error();
    serq_status st = check_layout(L);
    if (st) return st;

    if (!W || !X_cal || !E) return fail(SERQ_ERR_INVALID_ARG, "a required pointer is NULL");
    if (n_cal < 1) return fail(SERQ_ERR_SHAPE, "n_cal=%d must be >= 1", n_cal);
    return weight_error(L, W, X_cal, n_cal, E);
}

serq_status serq_l2qer_sizes(const serq_layout *L, int32_t k, size_t sizes[4]) {
    clear_error();
    serq_status st = check_l2qer_host(L, k);
    if (st) return st;
    if (!sizes) return fail(SERQ_ERR_INVALID_ARG, "sizes is NULL");
    const size_t kp = (size_t)l2qer_kpad(k);
    sizes[0] = kp * (size_t)L->d_in / 2;
    sizes[2] = (size_t)L->d_out * kp / 2;
    if (L->fmt == SERQ_FMT_MXFP4) {   // E8M0 bytes in groups of four K steps
        sizes[1] = kp * 16 * (size_t)((L->d_in / SERQ_K_ALIGN + 3) / 4);
        sizes[3] = (size_t)L->d_out * 16 * ((kp / SERQ_K_ALIGN + 3) / 4);
    } else {
        sizes[1] = 8 * kp;
        sizes[3] = 8 * (size_t)L->d_out;
    }
    return SERQ_OK;
}

serq_status serq_l2qer_prepare(const serq_layout *L, int32_t k, const float *L1, const float *L2, uint8_t *l1q,
                               void *l1scale, uint8_t *l2q, void *l2scale) {
    clear_error();
    serq_status st = check_l2qer_host(L, k);
    if (st) return st;
    if (!L1 || !L2 || !l1q || !l1scale || !l2q || !l2scale) return fail(SERQ_ERR_INVALID_ARG, "a required pointer is NULL");
    const int kp = l2qer_kpad(k);
    // L1 [d_in][k]: the weights of a d_in -> k_pad layer; L2 [k][d_out]: a
    // residual block with r_pad = k_pad
    if (L->fmt == SERQ_FMT_MXFP4) {
        quantize_factor_mx(L1, L->d_in, k, L->d_in, kp, l1q, (uint8_t *)l1scale);
        quantize_factor_mx(L2, k, L->d_out, kp, L->d_out, l2q, (uint8_t *)l2scale);
        return SERQ_OK;
    }
    quantize_factor(L1, L->d_in, k, L->d_in, kp, l1q, l1scale);
    quantize_factor(L2, k, L->d_out, kp, L->d_out, l2q, l2scale);
    return SERQ_OK;
}

serq_status serq_flatten_act(const float *X, int64_t M, int32_t d_in, const int32_t *perm,
                             const float *s, float *Xhat) {
    clear_error();
    if (!X || !perm || !s || !Xhat) return fail(SERQ_ERR_INVALID_ARG, "a required pointer is NULL");
    if (M < 1 || d_in < 1) return fail(SERQ_ERR_SHAPE, "M=%lld and d_in=%d must be >= 1", (long long)M, d_in);
    for (int32_t k = 0; k < d_in; ++k)
        if (perm[k] < 0 || perm[k] >= d_in) return fail(SERQ_ERR_INVALID_ARG, "perm[%d]=%d out of range", k, perm[k]);
    for (int64_t m = 0; m < M; ++m) {
        const float *x = X + m * d_in;
        float *y = Xhat + m * d_in;
        for (int32_t k = 0; k < d_in; ++k) y[k] = x[perm[k]] / s[perm[k]];
    }
    return SERQ_OK;
}

serq_status serq_act_bytes(int32_t M, int32_t d_in, serq_format fmt, size_t *xq_bytes,
                           size_t *xscale_bytes) {
    clear_error();
    if (!xq_bytes || !xscale_bytes) return fail(SERQ_ERR_INVALID_ARG, "a required pointer is NULL");
    return act_bytes(M, d_in, (int32_t)fmt, xq_bytes, xscale_bytes);
}

const char *serq_status_string(serq_status st) {
    switch (st) {
    case SERQ_OK: return "ok";
    case SERQ_ERR_INVALID_ARG: return "invalid argument";
    case SERQ_ERR_SHAPE: return "unsupported or inconsistent shape";
    case SERQ_ERR_UNSUPPORTED: return "not supported by this build";
    case SERQ_ERR_BUFFER: return "buffer too small";
    case SERQ_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *serq_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
