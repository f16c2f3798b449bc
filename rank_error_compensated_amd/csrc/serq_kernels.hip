// Device half of the SERQ library for gfx950 (CDNA4): the on-the-fly
// activation quantizer and the fused linear kernels, plus the runtime entry
// points of serq.h that launch them.
//
// The runtime layer follows the Stage 2 inference equation of the SERQ
// research notes (dihengye.cn):  Y ~= Xhat_q . What_q + Xtilde_{s,q} . Q(R).
// The residual product reuses the first r columns of the same quantized
// activation (no intermediate quantization, gist.science summaries section
// 2.2) and is fused into the main GEMM: it runs on activation tiles the K
// loop has already staged.
//
// INT4 / W4A8 run on int8 MFMA (v_mfma_i32_16x16x64_i8) with nibbles expanded
// in registers; MXFP4 runs on the block-scaled FP4 MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4), whose 32-element scale blocks are the
// MX blocks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "serq.h"
#include "serq_internal.h"

namespace serq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ===========================================================================
// Activation quantization (notes page, basic-quantization equation, applied
// per token; MX blocks per the OCP MX definition).  One workgroup of NT
// threads per token: 256 when there are enough tokens to fill the chip, 1024
// for a handful of tokens (decode), where each token's workgroup is alone on
// its compute unit and the per-thread encode work sets the time.  Thread t
// owns the 4-element chunks t, t + NT, t + 2 NT, ... of its row, so every
// load and store instruction of a wave touches one contiguous span.
// ===========================================================================

constexpr int QA_THREADS = 256;          // workgroup size when the tokens fill the chip
constexpr int QA_THREADS_FEW = 1024;     // workgroup size for a few tokens
template <int NT>
constexpr int qa_maxch() { return kQuantMaxInReg / (4 * NT); }   // chunks kept in registers

template <bool BF16>
__device__ __forceinline__ float4 load4(const void *X, size_t idx) {
    if constexpr (BF16) {
        const uint2 u = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(X) + idx);
        return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                           __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
    } else {
        return *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(X) + idx);
    }
}

__device__ __forceinline__ float amax4(float4 v) {
    return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// Symmetric RTN code: rne(x / s) of the IEEE fp32 quotient, clipped to +-Q.
template <int Q>
__device__ __forceinline__ int rtn_code(float x, float s) {
    const float q = rintf(x / s);
    return (int)fminf(fmaxf(q, -(float)Q), (float)Q);
}

// Source of the quantizers: element chunk j (elements 4j..4j+3) of token m's
// X-hat row, read from a row-major fp32 / bf16 matrix.
template <bool BF16>
struct GlobalRow {
    const void *X;
    size_t base;
    __device__ __forceinline__ float4 operator()(int j) const { return load4<BF16>(X, base + 4 * (size_t)j); }
};

// INT4 (Q = 7) writes the activation nibbles (even k two's complement high,
// odd k offset binary low) and, per token, the running sum of the even-k codes at
// every 128-element boundary; W4A8 (Q = 127) writes int8 codes.  One
// workgroup of NT threads per token; thread t owns the 4-element chunks t,
// t + NT, ...; CH chunks per thread stay in registers (CH = ceil(d_in / 4 NT)
// rounded up to a power of two, so short rows keep registers, and with them
// occupancy, low); rows longer than 4 NT CH are read twice.
template <int Q, int CH, int NT, class Src>
__device__ __forceinline__ void quant_int_row(const Src &src, int m, int d_in, uint8_t *__restrict__ xq,
                                              float *__restrict__ sx, int *__restrict__ xsum) {
    constexpr bool INT4 = Q == 7;
    const int t = threadIdx.x;
    const int nch = d_in >> 2;
    const int KT = d_in >> 7;
    const size_t base = (size_t)m * (size_t)d_in;
    const bool inreg = nch <= CH * NT;
    float4 v[CH];
    float amax = 0.0f;
    if (inreg) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int j = t + c * NT;
            if (j < nch) {
                v[c] = src(j);
                amax = fmaxf(amax, amax4(v[c]));
            }
        }
    } else {
        for (int j = t; j < nch; j += NT) amax = fmaxf(amax, amax4(src(j)));
    }
    __shared__ float red[NT / 64];
    __shared__ int csum[INT4 ? kQuantMaxChunks : 1];
    amax = wave_max(amax);
    if ((t & 63) == 0) red[t >> 6] = amax;
    __syncthreads();
    amax = red[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) amax = fmaxf(amax, red[w]);
    const float s = amax / (float)Q;
    if (t == 0) sx[m] = s;

    auto encode = [&](float4 u, int j) {
        int q0 = 0, q1 = 0, q2 = 0, q3 = 0;
        if (s > 0.0f) {
            q0 = rtn_code<Q>(u.x, s);
            q1 = rtn_code<Q>(u.y, s);
            q2 = rtn_code<Q>(u.z, s);
            q3 = rtn_code<Q>(u.w, s);
        }
        if constexpr (INT4) {
            const uint32_t b = ((uint32_t)(q0 & 15) << 4) | (uint32_t)(q1 + 8) |
                               ((uint32_t)(q2 & 15) << 12) | ((uint32_t)(q3 + 8) << 8);
            *reinterpret_cast<uint16_t *>(xq + (size_t)m * (size_t)(d_in >> 1) + 2 * (size_t)j) = (uint16_t)b;
            // even-k codes of this 128-element chunk: 32 consecutive lanes
            int e = q0 + q2;
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) e += __shfl_xor(e, o);
            if ((t & 31) == 0) csum[j >> 5] = e;
        } else {
            const uint32_t b = (uint32_t)(q0 & 255) | ((uint32_t)(q1 & 255) << 8) |
                               ((uint32_t)(q2 & 255) << 16) | ((uint32_t)(q3 & 255) << 24);
            *reinterpret_cast<uint32_t *>(xq + base + 4 * (size_t)j) = b;
        }
    };
    if (inreg) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int j = t + c * NT;
            if (j < nch) encode(v[c], j);
        }
    } else {
        for (int j = t; j < nch; j += NT) encode(src(j), j);
    }
    if constexpr (INT4) {
        // running sums over the chunks: one wave, 64 chunks per pass
        __syncthreads();
        if (t < 64) {
            int carry = 0;
            for (int c0 = 0; c0 < KT; c0 += 64) {
                int x = c0 + t < KT ? csum[c0 + t] : 0;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const int y = __shfl_up(x, o);
                    if (t >= o) x += y;
                }
                x += carry;
                if (c0 + t < KT) xsum[(size_t)m * KT + c0 + t] = x;
                carry = __shfl(x, 63);
            }
        }
    }
}

template <int Q, bool BF16, int CH, int NT>
__global__ __launch_bounds__(NT) void k_quant_int(const void *__restrict__ X, int d_in,
                                                  uint8_t *__restrict__ xq,
                                                  float *__restrict__ sx,
                                                  int *__restrict__ xsum) {
    const int m = blockIdx.x;
    quant_int_row<Q, CH, NT>(GlobalRow<BF16>{X, (size_t)m * (size_t)d_in}, m, d_in, xq, sx, xsum);
}

// OCP MX shared exponent floor(log2 amax) - EMAX from the fp32 exponent
// field (EMAX = 2 for E2M1 elements, 8 for E4M3), clamped to E8M0's range;
// 0 for an all-zero block.
template <int EMAX = 2>
__device__ __forceinline__ int mx_exponent(float amax) {
    if (!(amax > 0.0f)) return 0;
    const int e = (int)((__float_as_uint(amax) >> 23) & 0xffu) - 127 - EMAX;
    return min(127, max(-127, e));
}

// Nearest OCP FP8 E4M3 code (ties to the even code, saturating at 448 =
// code 0x7E), sign bit copied from the input.  Below 2^-6 the subnormal code
// is rint(|v| 2^9); above, with e = floor(log2 |v|), the code is
// 8 (e + 7) + rint((|v| 2^-e - 1) 8) -- a carry out of the mantissa lands on
// the next binade's code, which is the right one.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
    const float a = fabsf(v);
    uint32_t c;
    if (a < 0.015625f) {
        c = (uint32_t)rintf(a * 512.0f);
    } else {
        const int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;
        const float m = a * __uint_as_float((uint32_t)(127 - e) << 23);   // |v| 2^-e in [1, 2), exact
        c = (uint32_t)(8 * (e + 7)) + (uint32_t)rintf((m - 1.0f) * 8.0f);
    }
    return min(c, 126u) | ((__float_as_uint(v) >> 24) & 0x80u);
}

// Nearest E2M1 code (ties to the even code, saturating at 6).  Rounding to a
// 1-mantissa-bit float is rint at the binade's step: 0.5 below 2, 1 in [2, 4),
// 2 from 4 on.  Sign bit copied from the input.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
    const float a = fabsf(v);
    uint32_t idx;
    if (a < 2.0f) idx = (uint32_t)rintf(a * 2.0f);              // 0, .5, 1, 1.5, 2 -> 0..4
    else if (a < 4.0f) idx = (uint32_t)rintf(a) + 2u;          // 2, 3, 4 -> 4..6
    else idx = rintf(a * 0.5f) >= 3.0f ? 7u : 6u;               // 4 -> 6, 6 (and above) -> 7
    return idx | ((__float_as_uint(v) >> 28) & 8u);
}

// One 4-element chunk j of an MX row of d elements, its 32-element block
// held by 8 consecutive lanes (chunks 8 b .. 8 b + 7): the block maximum by
// shuffles, E8M0 written by the block's first lane, then the chunk's E2M1
// nibbles (MXFP4) or E4M3 bytes (MX W4A8).  xq_row, xe_row: the row's codes
// and E8M0 bytes.
template <bool FP8>
__device__ __forceinline__ void mx_encode_chunk(float4 u, int j, uint8_t *__restrict__ xq_row,
                                                uint8_t *__restrict__ xe_row) {
    float a = amax4(u);
    a = fmaxf(a, __shfl_xor(a, 1));
    a = fmaxf(a, __shfl_xor(a, 2));
    a = fmaxf(a, __shfl_xor(a, 4));
    const int e = mx_exponent<FP8 ? 8 : 2>(a);
    if ((j & 7) == 0) xe_row[j >> 3] = (uint8_t)(e + 127);
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);   // 2^-e, exact
    if constexpr (FP8) {
        const uint32_t b = e4m3_code(u.x * inv) | (e4m3_code(u.y * inv) << 8) | (e4m3_code(u.z * inv) << 16) |
                           (e4m3_code(u.w * inv) << 24);
        *reinterpret_cast<uint32_t *>(xq_row + 4 * (size_t)j) = b;
    } else {
        const uint32_t b = e2m1_code(u.x * inv) | (e2m1_code(u.y * inv) << 4) | (e2m1_code(u.z * inv) << 8) |
                           (e2m1_code(u.w * inv) << 12);
        *reinterpret_cast<uint16_t *>(xq_row + 2 * (size_t)j) = (uint16_t)b;
    }
}

// MX activations, one 32-element block per group of 8 lanes: E2M1 nibbles
// (MXFP4) or E4M3 bytes (MX W4A8) and the block's E8M0.
template <bool FP8, int NT, class Src>
__device__ __forceinline__ void quant_mx_row(const Src &src, int m, int d_in, uint8_t *__restrict__ xq,
                                             uint8_t *__restrict__ xe) {
    const int t = threadIdx.x;
    const int nch = d_in >> 2;   // a multiple of 32: groups of 8 lanes (one MX block) stay whole
    uint8_t *const xq_row = xq + (size_t)m * (size_t)(FP8 ? d_in : d_in >> 1);
    uint8_t *const xe_row = xe + (size_t)m * (size_t)(d_in >> 5);
    for (int j = t; j < nch; j += NT) mx_encode_chunk<FP8>(src(j), j, xq_row, xe_row);
}

template <bool BF16, bool FP8, int NT>
__global__ __launch_bounds__(NT) void k_quant_mx(const void *__restrict__ X, int d_in,
                                                 uint8_t *__restrict__ xq,
                                                 uint8_t *__restrict__ xe) {
    const int m = blockIdx.x;
    quant_mx_row<FP8, NT>(GlobalRow<BF16>{X, (size_t)m * (size_t)d_in}, m, d_in, xq, xe);
}

// ===========================================================================
// Producers of the layer input, fused with its quantization.  The notes page
// folds the flattening scale and the channel permutation into whatever
// produces X (Stage 1, Stage 3); for the two producers of a LLaMA block these
// kernels emit the quantized X-hat directly from the producer's input, with
// the fp32 operations of the unfused path in the same order, so the codes and
// scales are those of serq_quant_act on the flattened X:
//   RMSNorm (in front of q/k/v):  X = (h * r) * gamma,  r = 1 / sqrt(mean(h^2) + eps)
//     (sum of squares accumulated in fp64);
//   SwiGLU (in front of the down projection):  X = (g / (1 + e^-g)) * u
//     (e^x by the range reduction + degree-7 Taylor polynomial below);
// then X-hat[k] = X[perm[k]] / s[perm[k]].  One workgroup per token; the
// producer's row sits in LDS (fp32, in original channel order) and the
// quantizer gathers it through the permutation.  gamma and s are passed in
// saliency order (gamma[perm[k]], s[perm[k]]), folded once per layer.
// ===========================================================================

// e^x in fp32, every step one fp32 operation (no fused multiply-add):
// n = rint(x log2 e), r = (x - n ln2_hi) - n ln2_lo (Cody-Waite; ln2_hi has 16
// significant bits, so n ln2_hi is exact), p = 1 + r (1 + r (1/2! + ... +
// r / 7!)) by Horner, e^x = p 2^n.  +inf above 88.5, 0 below -87.
__device__ __forceinline__ float exp32(float x) {
    const float LN2_HI = 0.693145751953125f, LN2_LO = 1.428606765330187e-06f, LOG2E = 1.4426950408889634f;
    const float xc = fminf(fmaxf(x, -87.0f), 88.5f);
    const float n = rintf(xc * LOG2E);
    const float r = (xc - n * LN2_HI) - n * LN2_LO;
    float p = (float)(1.0 / 5040.0);
    p = (float)(1.0 / 720.0) + r * p;
    p = (float)(1.0 / 120.0) + r * p;
    p = (float)(1.0 / 24.0) + r * p;
    p = (float)(1.0 / 6.0) + r * p;
    p = 0.5f + r * p;
    p = 1.0f + r * p;
    p = 1.0f + r * p;
    float e = ldexpf(p, (int)n);
    if (x > 88.5f) e = __builtin_inff();
    if (x < -87.0f) e = 0.0f;
    return e;
}

// X-hat chunk j from the producer's row in LDS, gathered through perm; the
// scales (and RMSNorm's gamma) come in saliency order, so they load
// contiguously beside perm.
struct PermutedRow {
    const float *row;          // LDS, original channel order (already the producer's X)
    const int32_t *perm;
    const float *sp;           // s[perm[k]]
    __device__ __forceinline__ float4 operator()(int j) const {
        const int4 p = *reinterpret_cast<const int4 *>(perm + 4 * (size_t)j);
        const float4 d = *reinterpret_cast<const float4 *>(sp + 4 * (size_t)j);
        return make_float4(row[p.x] / d.x, row[p.y] / d.y, row[p.z] / d.z, row[p.w] / d.w);
    }
};

// RMSNorm: the raw row of h in LDS; X is formed in the gather.
struct RmsRow {
    const float *row;          // LDS, h in original channel order
    const float *gp;           // gamma[perm[k]]
    const int32_t *perm;
    const float *sp;           // s[perm[k]]
    float r;
    __device__ __forceinline__ float4 operator()(int j) const {
        const int4 p = *reinterpret_cast<const int4 *>(perm + 4 * (size_t)j);
        const float4 g = *reinterpret_cast<const float4 *>(gp + 4 * (size_t)j);
        const float4 d = *reinterpret_cast<const float4 *>(sp + 4 * (size_t)j);
        return make_float4(((row[p.x] * r) * g.x) / d.x, ((row[p.y] * r) * g.y) / d.y,
                           ((row[p.z] * r) * g.z) / d.z, ((row[p.w] * r) * g.w) / d.w);
    }
};

// Q = 7 (INT4), 127 (W4A8), 0 (MXFP4) or 1 (MX W4A8).
template <int Q, int CH, int NT, class Src>
__device__ __forceinline__ void quant_row(const Src &src, int m, int d, uint8_t *xq, void *xscale, int M) {
    if constexpr (Q == 0 || Q == 1) {
        quant_mx_row<Q == 1, NT>(src, m, d, xq, (uint8_t *)xscale);
    } else {
        float *sx = (float *)xscale;
        int *xsum = (int *)((uint8_t *)xscale + sizeof(float) * (size_t)M);
        quant_int_row<Q, CH, NT>(src, m, d, xq, sx, xsum);
    }
}

template <int Q, bool BF16, int CH, int NT>
__global__ __launch_bounds__(NT) void k_rmsnorm_quant(const void *__restrict__ H, int M, int d,
                                                      const float *__restrict__ gamma, float eps,
                                                      const int32_t *__restrict__ perm,
                                                      const float *__restrict__ s, uint8_t *xq,
                                                      void *xscale) {
    extern __shared__ __attribute__((aligned(16))) float row[];
    __shared__ double part[NT / 64];
    const int m = blockIdx.x, t = threadIdx.x;
    const size_t base = (size_t)m * (size_t)d;
    double ss = 0.0;
#pragma unroll 4
    for (int j = t; j < (d >> 2); j += NT) {
        const float4 v = load4<BF16>(H, base + 4 * (size_t)j);
        *reinterpret_cast<float4 *>(row + 4 * j) = v;
        ss += (double)v.x * (double)v.x + (double)v.y * (double)v.y + (double)v.z * (double)v.z +
              (double)v.w * (double)v.w;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    if ((t & 63) == 0) part[t >> 6] = ss;
    __syncthreads();
    double tot = part[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) tot += part[w];
    const float ms = (float)(tot / (double)d);
    const float r = 1.0f / sqrtf(ms + eps);
    quant_row<Q, CH, NT>(RmsRow{row, gamma, perm, s, r}, m, d, xq, xscale, M);   // gamma, s in saliency order
}

// SwiGLU with the permutation folded into the producer: gate and up already
// in saliency order, X-hat[k] = ((g / (1 + e^-g)) * u) / s_p[k], streamed.
template <bool BF16>
struct SwigluRow {
    const void *GU;
    size_t base;               // row start; gate in [0, d), up in [d, 2 d)
    int d;
    const float *sp;
    __device__ __forceinline__ float4 operator()(int j) const {
        const float4 g = load4<BF16>(GU, base + 4 * (size_t)j);
        const float4 u = load4<BF16>(GU, base + (size_t)d + 4 * (size_t)j);
        const float4 q = *reinterpret_cast<const float4 *>(sp + 4 * (size_t)j);
        return make_float4(((g.x / (1.0f + exp32(-g.x))) * u.x) / q.x, ((g.y / (1.0f + exp32(-g.y))) * u.y) / q.y,
                           ((g.z / (1.0f + exp32(-g.z))) * u.z) / q.z, ((g.w / (1.0f + exp32(-g.w))) * u.w) / q.w);
    }
};

template <int Q, bool BF16, int CH, int NT>
__global__ __launch_bounds__(NT) void k_swiglu_quant_folded(const void *__restrict__ GU, int M, int d,
                                                            const float *__restrict__ sp, uint8_t *xq,
                                                            void *xscale) {
    const int m = blockIdx.x;
    quant_row<Q, CH, NT>(SwigluRow<BF16>{GU, (size_t)m * (size_t)(2 * d), d, sp}, m, d, xq, xscale, M);
}

template <int Q, bool BF16, int CH, int NT>
__global__ __launch_bounds__(NT) void k_swiglu_quant(const void *__restrict__ GU, int M, int d,
                                                     const int32_t *__restrict__ perm,
                                                     const float *__restrict__ s, uint8_t *xq,
                                                     void *xscale) {
    extern __shared__ __attribute__((aligned(16))) float row[];
    const int m = blockIdx.x, t = threadIdx.x;
    const size_t base = (size_t)m * (size_t)(2 * d);      // gate in [0, d), up in [d, 2d)
#pragma unroll 4
    for (int j = t; j < (d >> 2); j += NT) {
        const float4 g = load4<BF16>(GU, base + 4 * (size_t)j);
        const float4 u = load4<BF16>(GU, base + (size_t)d + 4 * (size_t)j);
        float4 h;
        h.x = (g.x / (1.0f + exp32(-g.x))) * u.x;
        h.y = (g.y / (1.0f + exp32(-g.y))) * u.y;
        h.z = (g.z / (1.0f + exp32(-g.z))) * u.z;
        h.w = (g.w / (1.0f + exp32(-g.w))) * u.w;
        *reinterpret_cast<float4 *>(row + 4 * j) = h;
    }
    __syncthreads();
    quant_row<Q, CH, NT>(PermutedRow{row, perm, s}, m, d, xq, xscale, M);
}

// ===========================================================================
// Fused GEMM building blocks
// ===========================================================================

// W4A8 weights (two's-complement nibbles, element k in byte k/2, low nibble
// first): hi() keeps the odd elements in the high half of each byte (int8
// value 16 w), lo() moves the even ones there.  Products are 16 x w and the
// exact int32 sum is shifted back in the epilogue.
__device__ __forceinline__ int nib_hi(uint32_t p) { return (int)(p & 0xF0F0F0F0u); }
__device__ __forceinline__ int nib_lo(uint32_t p) { return (int)((p << 4) & 0xF0F0F0F0u); }

// 16 packed W4A8 bytes (32 nibbles) -> the two 16x16x64 operands of this lane.
__device__ __forceinline__ void unpack32(u32x4 p, v4i &op0, v4i &op1) {
    op0 = v4i{nib_lo(p.x), nib_hi(p.x), nib_lo(p.y), nib_hi(p.y)};
    op1 = v4i{nib_lo(p.z), nib_hi(p.z), nib_lo(p.w), nib_hi(p.w)};
}

// 16 int8 activations -> the element order unpack32 produces (even elements
// of each 8-group, then odd ones).
__device__ __forceinline__ v4i reorder16(u32x4 a) {
    const uint32_t E = 0x06040200u, O = 0x07050301u;
    return v4i{(int)__builtin_amdgcn_perm(a.y, a.x, E), (int)__builtin_amdgcn_perm(a.y, a.x, O),
               (int)__builtin_amdgcn_perm(a.w, a.z, E), (int)__builtin_amdgcn_perm(a.w, a.z, O)};
}

// INT4 layout-2 operands, one AND per word.  Activation bytes hold the even
// element in the high nibble (two's complement: int8 value 16 x) and the odd
// element + 8 in the low nibble; weight bytes the even element + 8 low and
// the odd element high.  Pairing (act high, weight low) and (act low, weight
// high) gives 16 x w + 128 x_even + 128 w_odd per element pair.
constexpr uint32_t NIB_HI = 0xF0F0F0F0u, NIB_LO = 0x0F0F0F0Fu;
__device__ __forceinline__ void split_hi_lo(u32x4 p, v4i &hi, v4i &lo) {
    hi = v4i{(int)(p.x & NIB_HI), (int)(p.y & NIB_HI), (int)(p.z & NIB_HI), (int)(p.w & NIB_HI)};
    lo = v4i{(int)(p.x & NIB_LO), (int)(p.y & NIB_LO), (int)(p.z & NIB_LO), (int)(p.w & NIB_LO)};
}

// LDS tiles hold rows of 64 (or 128) bytes split into 16-byte columns.  A
// lane group reads one column of 16 consecutive rows; XOR-ing the column with
// these row functions spreads those rows over all banks.
__device__ __forceinline__ int swz4(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }
__device__ __forceinline__ int swz8(int row) { return (row ^ (row >> 3)) & 7; }
// For 128-byte rows read as 16-row fragments: chunk c of row r sits at
// position c ^ (r & 7).  Measured on gfx950 with 8 waves per CU, fragment
// reads run at 214 B/clk per CU in this placement against 128 B/clk with
// swz8 (the 16-byte copy writes run at ~100 B/clk in both), and blocks 16
// rows apart differ by a constant, which the LDS reads carry as an
// immediate offset instead of a register each.
__device__ __forceinline__ int swz7(int row) { return row & 7; }

// Tile order of the large-tile kernels: workgroup ids are first made
// XCD-contiguous (consecutive ranks run on the same XCD), then ranks walk
// groups of gm token tiles, token tiles fastest inside a group, so that the
// tiles one XCD runs together share few activation and weight rows in its L2.
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int gm, int &tm, int &tn) {
    const int nwg = gridDim.x;
    int bid = blockIdx.x;
    if ((nwg & 7) == 0) bid = (bid & 7) * (nwg >> 3) + (bid >> 3);
    const int per = gm * tiles_n;
    const int grp = bid / per, rem = bid % per;
    const int gsz = min(gm, tiles_m - grp * gm);   // the last group may be short
    tm = grp * gm + rem % gsz;
    tn = rem / gsz;
}

__device__ __forceinline__ u32x4 lds16(const uint8_t *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ u32x4 gld16(const uint8_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

// 16 bytes of Y from a prefill GEMM, stored non-temporally: Y is written once
// and not read back by the kernel, and large outputs (gate|up: 235 MB) stored
// the ordinary way fill the memory-side cache with dirty lines whose
// write-back then slows the kernels that follow.
__device__ __forceinline__ void store_y(float *p, float4 y) {
    __builtin_nontemporal_store(v4f{y.x, y.y, y.z, y.w}, reinterpret_cast<v4f *>(p));
}

// Raw buffer loads: the base address lives in a scalar buffer descriptor and
// each lane supplies a 32-bit byte offset, so a copy plan costs one VGPR per
// load instead of a 64-bit pointer.  Reads past `bytes` return zero.  Every
// row-dependent part of an address goes into the per-lane offset, so that a
// row past the buffer reads zero whether or not the range check counts the
// scalar offset, which carries only a K step's offset within a row.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, size_t bytes) {
    const int n = bytes >= 0xffffffffull ? -1 : (int)(uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}
__device__ __forceinline__ u32x4 bld16(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint2 bld8(rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
    return make_uint2(v[0], v[1]);
}

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Arguments of the INT4 / W4A8 kernels.  For INT4, xsum holds the running
// even-k code sums [M][K/128] and wsum / rsum the odd-k code sums [N] of
// What_q / Q(R) (layout 3); for W4A8 they are unused.
struct IntArgs {
    // L2QER comparator only: the residual reads these (the quantized
    // intermediate Q(X_q . L1_q), its per-token scales and code sums) in
    // place of the first r_pad columns of xq
    const uint8_t *tq = nullptr;
    const float *st = nullptr;
    const int *tsum = nullptr;
    const uint8_t *xq;
    const float *sx;
    const int *xsum;
    const uint8_t *wq;
    const float *sw;
    const int *wsum;
    const uint8_t *rq;
    const float *sR;
    const int *rsum;
    float *Y;
    int *acc_main;
    int *acc_res;
    int M, N, K, r_pad;
    int gm;                    // token tiles per group in the large-tile order
    int direct_y = 0;          // large-tile kernel: store Y straight from registers
    // SwiGLU epilogue (large-tile kernel only): output columns come in
    // (gate, up) pairs; instead of Y the kernel writes H [M][N / 2], H[m][j]
    // = silu(Y[m][2 j]) * Y[m][2 j + 1] / sdown[j]
    const float *sdown = nullptr;
    float *H = nullptr;
};

// Per-token epilogue terms: the scale and (INT4) the even-k code sums over K
// and over the first r_pad columns.
struct IntRow {
    float sxr;
    int xfull, xres;
    __device__ __forceinline__ void load(const IntArgs &a, bool a8, int row) {
        const int r = min(row, a.M - 1);
        sxr = a.sx[r];
        xfull = xres = 0;
        if (!a8) {
            const int KT = a.K >> 7, RT = a.r_pad >> 7;
            xfull = a.xsum[(size_t)r * KT + KT - 1];
            if (RT > 0) xres = a.xsum[(size_t)r * KT + RT - 1];
        }
    }
};

// Per-output-channel epilogue terms: scales and (INT4) odd-k code sums.
struct IntCol {
    float swc, src;
    int wsum, rsum;
    __device__ __forceinline__ void load(const IntArgs &a, bool a8, int col) {
        const int c = min(col, a.N - 1);
        swc = a.sw[c];
        src = a.sR[c];
        wsum = rsum = 0;
        if (!a8) {
            wsum = a.wsum[c];
            rsum = a.rsum[c];
        }
    }
};

// Raw MFMA sums -> exact accumulators -> Y = sx[m] * (sw[o] A_main + sR[o] A_res).
template <bool A8>
__device__ __forceinline__ void int_store(const IntArgs &a, int row, int col, int raw_main, int raw_res,
                                          const IntRow &r, const IntCol &c) {
    int am, ar;
    if constexpr (A8) {
        am = raw_main >> 4;
        ar = raw_res >> 4;
    } else {
        am = (raw_main - 128 * (r.xfull + c.wsum)) >> 4;
        ar = (raw_res - 128 * (r.xres + c.rsum)) >> 4;
    }
    const size_t o = (size_t)row * (size_t)a.N + col;
    a.Y[o] = r.sxr * fmaf(c.swc, (float)am, c.src * (float)ar);
    if (a.acc_main) {
        a.acc_main[o] = am;
        a.acc_res[o] = ar;
    }
}

constexpr int G_BM = 128, G_BN = 128, G_THREADS = 256;

// ===========================================================================
// General prefill INT4 / W4A8 kernel (any r_pad).  Tile 128 x 128 x (K step
// 128), 4 waves in a 2 x 2 grid, each wave 64 x 64 = 4 x 4 MFMA blocks of
// 16 x 16.  Two int32 accumulators per block: the main product over all K and
// the residual product over the first r_pad columns (same staged activation
// tile, Q(R) tile instead of What_q).  Double-buffered LDS, one barrier per
// K step.
// ===========================================================================
template <bool A8>
__global__ __launch_bounds__(G_THREADS) void k_gemm_int(IntArgs args) {
    const int M = args.M, N = args.N, K = args.K, r_pad = args.r_pad;
    constexpr int A_ROWB = A8 ? 128 : 64;          // bytes of an activation row per K step
    constexpr int A_BYTES = G_BM * A_ROWB;
    constexpr int B_BYTES = G_BN * 64;
    constexpr int STAGE = A_BYTES + 2 * B_BYTES;   // activation, What_q and Q(R) tiles
    constexpr int A_CH = A_BYTES / 16 / G_THREADS; // 16-byte copies per thread
    constexpr int A_CPR = A_ROWB / 16;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int i = lane & 15, g = lane >> 4;
    const int wm = w >> 1, wn = w & 1;
    const int m0 = blockIdx.y * G_BM, n0 = blockIdx.x * G_BN;
    const int KT = K >> 7, RT = r_pad >> 7;
    const size_t a_ld = A8 ? (size_t)K : (size_t)(K >> 1);

    // global -> LDS copy plan (rows past M or N re-read the last row; their
    // results are never stored)
    const uint8_t *a_src[A_CH];
    int a_dst[A_CH];
#pragma unroll
    for (int u = 0; u < A_CH; ++u) {
        const int c = t + u * G_THREADS, row = c / A_CPR, col = c % A_CPR;
        a_src[u] = args.xq + (size_t)min(m0 + row, M - 1) * a_ld + col * 16;
        a_dst[u] = row * A_ROWB + (col ^ (A8 ? swz8(row) : swz4(row))) * 16;
    }
    // What_q / Q(R) are 16-row x 64-byte tiles: one K step of a 16-channel
    // block is one 1024-byte tile, 64 consecutive threads copy it
    const uint8_t *w_src[2], *r_src[2];
    int b_dst[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int c = t + u * G_THREADS, row = c >> 2, col = c & 3;
        const int n = min(n0 + row, N - 1);
        const size_t in_tile = (size_t)(n & 15) * 64 + col * 16;
        w_src[u] = args.wq + (size_t)(n >> 4) * KT * 1024 + in_tile;
        r_src[u] = args.rq + (size_t)(n >> 4) * RT * 1024 + in_tile;
        b_dst[u] = row * 64 + (col ^ swz4(row)) * 16;
    }
    u32x4 ra[A_CH], rw[2], rr[2];
    auto gload = [&](int kt, bool res) {
#pragma unroll
        for (int u = 0; u < A_CH; ++u) ra[u] = gld16(a_src[u] + (size_t)kt * A_ROWB);
#pragma unroll
        for (int u = 0; u < 2; ++u) rw[u] = gld16(w_src[u] + (size_t)kt * 1024);
        if (res) {
#pragma unroll
            for (int u = 0; u < 2; ++u) rr[u] = gld16(r_src[u] + (size_t)kt * 1024);
        }
    };
    auto sstore = [&](int buf, bool res) {
        uint8_t *s = smem + buf * STAGE;
#pragma unroll
        for (int u = 0; u < A_CH; ++u) *reinterpret_cast<u32x4 *>(s + a_dst[u]) = ra[u];
#pragma unroll
        for (int u = 0; u < 2; ++u) *reinterpret_cast<u32x4 *>(s + A_BYTES + b_dst[u]) = rw[u];
        if (res) {
#pragma unroll
            for (int u = 0; u < 2; ++u) *reinterpret_cast<u32x4 *>(s + A_BYTES + B_BYTES + b_dst[u]) = rr[u];
        }
    };
    // the two operand pairs of a 16 x 16 block for this lane: (a0, b0), (a1, b1)
    auto a_frag = [&](const uint8_t *s, int row, v4i &o0, v4i &o1) {
        if constexpr (A8) {
            o0 = reorder16(lds16(s + row * 128 + (((2 * g) ^ swz8(row)) * 16)));
            o1 = reorder16(lds16(s + row * 128 + (((2 * g + 1) ^ swz8(row)) * 16)));
        } else {
            split_hi_lo(lds16(s + row * 64 + ((g ^ swz4(row)) * 16)), o0, o1);
        }
    };
    auto b_frag = [&](const uint8_t *s, int col, v4i &o0, v4i &o1) {
        const u32x4 p = lds16(s + col * 64 + ((g ^ swz4(col)) * 16));
        if constexpr (A8) unpack32(p, o0, o1);
        else split_hi_lo(p, o1, o0);   // weight low nibbles pair with activation high ones
    };

    v4i accm[4][4], accr[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) accm[a][b] = accr[a][b] = v4i{0, 0, 0, 0};

    gload(0, RT > 0);
    sstore(0, RT > 0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const bool nxt = kt + 1 < KT;
        if (nxt) gload(kt + 1, kt + 1 < RT);
        const uint8_t *s = smem + (kt & 1) * STAGE;
        v4i a0[4], a1[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) a_frag(s, wm * 64 + rb * 16 + i, a0[rb], a1[rb]);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            v4i b0, b1;
            b_frag(s + A_BYTES, wn * 64 + cb * 16 + i, b0, b1);
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                accm[rb][cb] = mfma_i8(a0[rb], b0, accm[rb][cb]);
                accm[rb][cb] = mfma_i8(a1[rb], b1, accm[rb][cb]);
            }
        }
        if (kt < RT) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                v4i b0, b1;
                b_frag(s + A_BYTES + B_BYTES, wn * 64 + cb * 16 + i, b0, b1);
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    accr[rb][cb] = mfma_i8(a0[rb], b0, accr[rb][cb]);
                    accr[rb][cb] = mfma_i8(a1[rb], b1, accr[rb][cb]);
                }
            }
        }
        if (nxt) sstore((kt + 1) & 1, kt + 1 < RT);
        __syncthreads();
    }

    // epilogue.  MFMA block layout: lane (g, i) holds rows 4g..4g+3 of column i.
    IntCol cc[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) cc[cb].load(args, A8, n0 + wn * 64 + cb * 16 + i);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int row = m0 + wm * 64 + rb * 16 + 4 * g + v;
            IntRow rr_;
            rr_.load(args, A8, row);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const int col = n0 + wn * 64 + cb * 16 + i;
                if (row < M && col < N) int_store<A8>(args, row, col, accm[rb][cb][v], accr[rb][cb][v], rr_, cc[cb]);
            }
        }
    }
}

// ===========================================================================
// Large-tile prefill INT4 kernel.  Tile 256 tokens x 128 output channels,
// K steps of 256 (128 bytes of every row), WGM x WGN waves with 64 x 64 wave
// tiles and ONE int32 accumulator per 16 x 16 block.  The MFMA row operand is
// the weight tile and the column operand the activation tile, so a lane's four
// accumulator values are four consecutive output channels of one token and
// leave in a single 16-byte store.  Global loads run two K steps ahead (two
// alternating sets of staging registers, 96 KB in flight per workgroup) into
// a double-buffered LDS tile.  The residual A_res = Xtilde_{s,q} . Q(R) is not
// carried through the K loop: the first step's activation tile is also kept
// in LDS (Q(R), r_pad <= 256, is loaded there up front), and the epilogue
// multiplies them block by block (r_pad/64 MFMAs per block) right before it
// writes Y.  The workgroup order is remapped so that each XCD (workgroup id
// modulo 8) walks a contiguous run of tiles, token tiles fastest.
// ===========================================================================
constexpr int L_BM = 256, L_BN = 128;

template <int WGM, int WGN, bool PF>
__global__ __launch_bounds__(64 * WGM * WGN) void k_gemm_int_big(IntArgs args) {
    const int M = args.M, N = args.N, K = args.K, r_pad = args.r_pad;
    constexpr int NT = 64 * WGM * WGN;                  // threads
    constexpr int WR = L_BM / WGM, WC = L_BN / WGN;     // wave tile (tokens x channels)
    constexpr int MB = WR / 16, NB = WC / 16;           // 16 x 16 blocks per wave
    constexpr int ROWB = 128;                           // bytes of a row per K step
    constexpr int A_BYTES = L_BM * ROWB;                // 32 KB
    constexpr int W_BYTES = L_BN * ROWB;                // 16 KB
    constexpr int STAGE = A_BYTES + W_BYTES;
    constexpr int ACH = A_BYTES / 16 / NT, WCH = W_BYTES / 16 / NT;   // 16-byte copies per thread
    constexpr int RSTEP = NT / 8;                       // rows covered by one copy round
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t *const ares = smem + 2 * STAGE;             // the first step's activation tile
    uint8_t *const rtile = ares + A_BYTES;              // Q(R): 128 rows x r_pad/2 bytes
    // the epilogue's operands, staged while the K loop runs: per token sx,
    // the even-code sums (total, at r_pad) and the L2QER scale; per channel
    // sw, sR and the odd-code sums of What_q and Q(R)
    float *const e_sx = reinterpret_cast<float *>(rtile + L_BN * ROWB);
    int *const e_xf = reinterpret_cast<int *>(e_sx + L_BM);
    int *const e_xr = e_xf + L_BM;
    float *const e_st = reinterpret_cast<float *>(e_xr + L_BM);
    float *const e_sw = e_st + L_BM;
    float *const e_sr = e_sw + L_BN;
    int *const e_ws = reinterpret_cast<int *>(e_sr + L_BN);
    int *const e_rs = e_ws + L_BN;

    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int i = lane & 15, g = lane >> 4;
    const int wm = w / WGN, wn = w % WGN;
    int tm, tn;
    tile_coords((M + L_BM - 1) / L_BM, (N + L_BN - 1) / L_BN, args.gm, tm, tn);
    const int m0 = tm * L_BM, n0 = tn * L_BN;
    const int KT = K >> 8, RT = r_pad >> 7;             // K steps of 256; residual chunks of 128
    const uint32_t ld = (uint32_t)(K >> 1);

    // copy plan: thread t moves 16-byte column (t & 7) of rows (t >> 3) + RSTEP * u.
    // What_q is stored in 16-row x 64-byte tiles: one step of 256 elements of
    // a row is 64 bytes in each of two consecutive tiles.
    const int crow = t >> 3, ccol = t & 7;
    uint32_t a_off[ACH], w_off[WCH];
    int a_dst[ACH], b_dst[WCH];
#pragma unroll
    for (int u = 0; u < ACH; ++u) {
        const int row = crow + RSTEP * u;
        a_off[u] = (uint32_t)min(m0 + row, M - 1) * ld + ccol * 16;
        a_dst[u] = row * ROWB + (ccol ^ swz7(row)) * 16;
    }
#pragma unroll
    for (int u = 0; u < WCH; ++u) {
        const int row = crow + RSTEP * u;
        const int n = min(n0 + row, N - 1);
        w_off[u] = ((uint32_t)(n >> 4) * (uint32_t)(K >> 7) + (ccol >> 2)) * 1024 + (n & 15) * 64 + (ccol & 3) * 16;
        b_dst[u] = row * ROWB + (ccol ^ swz7(row)) * 16;
    }

    struct Regs {
        u32x4 a[ACH], w[WCH];
    };
    auto gload = [&](Regs &R, int kt) {
        const uint32_t k = (uint32_t)kt * ROWB;
#pragma unroll
        for (int u = 0; u < ACH; ++u) R.a[u] = gld16(args.xq + a_off[u] + k);
#pragma unroll
        for (int u = 0; u < WCH; ++u) R.w[u] = gld16(args.wq + w_off[u] + (uint32_t)kt * 2048);
    };
    auto sstore = [&](const Regs &R, int buf, bool keep) {
        uint8_t *s = smem + buf * STAGE;
#pragma unroll
        for (int u = 0; u < ACH; ++u) *reinterpret_cast<u32x4 *>(s + a_dst[u]) = R.a[u];
#pragma unroll
        for (int u = 0; u < WCH; ++u) *reinterpret_cast<u32x4 *>(s + A_BYTES + b_dst[u]) = R.w[u];
        if (keep) {   // the salient columns' activation tile, for the epilogue
#pragma unroll
            for (int u = 0; u < ACH; ++u) *reinterpret_cast<u32x4 *>(ares + a_dst[u]) = R.a[u];
        }
    };
    // 16-byte column c of a tile row (32 elements of K for this lane group)
    auto frag = [&](const uint8_t *s, int row, int c, v4i &hi, v4i &lo) {
        split_hi_lo(lds16(s + row * ROWB + ((c ^ swz7(row)) * 16)), hi, lo);
    };

    v4i acc[NB][MB];
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
        for (int b = 0; b < MB; ++b) acc[a][b] = v4i{0, 0, 0, 0};

    auto compute = [&](int buf) {
        const uint8_t *s = smem + buf * STAGE;
#pragma unroll
        for (int h = 0; h < 2; ++h) {                   // two halves of 128 elements
            v4i ahi[MB], alo[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) frag(s, wm * WR + mb * 16 + i, 4 * h + g, ahi[mb], alo[mb]);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                v4i whi, wlo;
                frag(s + A_BYTES, wn * WC + nb * 16 + i, 4 * h + g, whi, wlo);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    acc[nb][mb] = mfma_i8(wlo, ahi[mb], acc[nb][mb]);
                    acc[nb][mb] = mfma_i8(whi, alo[mb], acc[nb][mb]);
                }
            }
        }
    };

    // prologue: Q(R) (kept for the epilogue; r_pad <= 256, so at most 1024
    // 16-byte pieces, two per thread) and the first two steps.  The Q(R)
    // loads go out first and land in LDS after the step loads are issued.
    // The prefetch is issued unconditionally (past the last step it re-reads
    // step KT - 1 and the data is dropped): a branch around it would make the
    // compiler wait for every outstanding load before each LDS store.
    constexpr int RCH = L_BN * 8 / NT;                  // Q(R) pieces per thread at r_pad = 256
    const int cpr = r_pad >> 5;                         // 16-byte columns per Q(R) row
    u32x4 rv[RCH];
#pragma unroll
    for (int u = 0; u < RCH; ++u) {
        const int c = t + u * NT, row = c / max(cpr, 1), col = c % max(cpr, 1);
        const int n = min(n0 + row, N - 1);
        const uint32_t off = ((uint32_t)(n >> 4) * (uint32_t)RT + (col >> 2)) * 1024 + (n & 15) * 64 + (col & 3) * 16;
        if (c < L_BN * cpr) rv[u] = gld16(args.rq + off);
    }
    const bool l2 = args.tq != nullptr;                 // L2QER residual from the intermediate
    const int KC = K >> 7;                               // running-sum entries per token
    // epilogue operands: threads 0..255 one token each, 256..383 one channel
    float e0 = 0.0f, e3 = 0.0f;
    int e1 = 0, e2 = 0;
    if (t < L_BM) {
        const int rl = min(m0 + t, M - 1);
        e0 = args.sx[rl];
        e1 = args.xsum[(size_t)rl * KC + KC - 1];
        if (l2) {
            e3 = args.st[rl];
            e2 = RT > 0 ? args.tsum[(size_t)rl * RT + RT - 1] : 0;
        } else {
            e2 = RT > 0 ? args.xsum[(size_t)rl * KC + RT - 1] : 0;
        }
    } else if (t < L_BM + L_BN) {
        const int cl = min(n0 + t - L_BM, N - 1);
        e0 = args.sw[cl];
        e3 = args.sR[cl];
        e1 = args.wsum[cl];
        e2 = args.rsum[cl];
    }
    Regs R0, R1;
    gload(R0, 0);
    gload(R1, min(1, KT - 1));
#pragma unroll
    for (int u = 0; u < RCH; ++u) {
        const int c = t + u * NT, row = c / max(cpr, 1), col = c % max(cpr, 1);
        if (c < L_BN * cpr) *reinterpret_cast<u32x4 *>(rtile + row * ROWB + (col ^ swz7(row)) * 16) = rv[u];
    }
    sstore(R0, 0, RT > 0 && !l2);
    if (t < L_BM) {
        e_sx[t] = e0;
        e_xf[t] = e1;
        e_xr[t] = e2;
        e_st[t] = e3;
    } else if (t < L_BM + L_BN) {
        e_sw[t - L_BM] = e0;
        e_sr[t - L_BM] = e3;
        e_ws[t - L_BM] = e1;
        e_rs[t - L_BM] = e2;
    }
    if (l2) {   // its tile: 256 rows x r_pad/2 bytes, placed as the kept activation tile
        const uint32_t tld = (uint32_t)(r_pad >> 1);
#pragma unroll
        for (int u = 0; u < (L_BM * 8) / NT; ++u) {
            const int c = t + u * NT, row = c / max(cpr, 1), col = c % max(cpr, 1);
            if (c < L_BM * cpr) {
                const u32x4 v = gld16(args.tq + (size_t)min(m0 + row, M - 1) * tld + col * 16);
                *reinterpret_cast<u32x4 *>(ares + row * ROWB + (col ^ swz7(row)) * 16) = v;
            }
        }
    }
    if constexpr (PF) gload(R0, min(2, KT - 1));
    __syncthreads();
    int kt = 0;
    if constexpr (PF) {
        // Fragments pipelined across half steps: while the MFMAs of one half
        // step run, the packed fragments of the next are read from LDS; the
        // next step's stage buffer is written at the top of a step and the
        // one barrier sits between its halves, so that the second half can
        // already read the next buffer.  A buffer is rewritten only after the
        // barrier that follows its last read; staging loads run two steps
        // ahead of their LDS stores.
        u32x4 pa[MB], pw[NB];
        v4i ahi[MB], alo[MB], whi[NB], wlo[NB];
        auto pread = [&](int buf, int h) {
            const uint8_t *s = smem + buf * STAGE;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int row = wm * WR + mb * 16 + i;
                pa[mb] = lds16(s + row * ROWB + (((4 * h + g) ^ swz7(row)) * 16));
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int row = wn * WC + nb * 16 + i;
                pw[nb] = lds16(s + A_BYTES + row * ROWB + (((4 * h + g) ^ swz7(row)) * 16));
            }
        };
        auto unpack = [&]() {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) split_hi_lo(pa[mb], ahi[mb], alo[mb]);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) split_hi_lo(pw[nb], whi[nb], wlo[nb]);
        };
        auto mm = [&]() {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    acc[nb][mb] = mfma_i8(wlo[nb], ahi[mb], acc[nb][mb]);
                    acc[nb][mb] = mfma_i8(whi[nb], alo[mb], acc[nb][mb]);
                }
        };
        pread(0, 0);
        for (; kt + 2 <= KT; kt += 2) {
            // step kt from buffer 0; step kt + 1 (in R1) goes to buffer 1
            sstore(R1, 1, false);
            gload(R1, min(kt + 3, KT - 1));
            unpack();
            pread(0, 1);
            mm();
            __syncthreads();
            unpack();
            pread(1, 0);
            mm();
            // step kt + 1 from buffer 1; step kt + 2 (in R0) goes to buffer 0
            if (kt + 2 < KT) sstore(R0, 0, false);
            gload(R0, min(kt + 4, KT - 1));
            unpack();
            pread(1, 1);
            mm();
            __syncthreads();
            unpack();
            if (kt + 2 < KT) pread(0, 0);
            mm();
        }
        if (kt < KT) {   // odd step count: the last step sits in buffer 0
            unpack();
            pread(0, 1);
            mm();
            unpack();
            mm();
            kt = KT;
        }
    } else {
        for (; kt + 2 <= KT; kt += 2) {
            // even step: LDS buffer 0 holds step kt, R1 carries step kt + 1
            gload(R0, min(kt + 2, KT - 1));
            __builtin_amdgcn_sched_barrier(0);   // keep the prefetch at the top of the step
            compute(0);
            sstore(R1, 1, false);
            __syncthreads();
            // odd step: LDS buffer 1 holds step kt + 1, R0 carries step kt + 2
            gload(R1, min(kt + 3, KT - 1));
            __builtin_amdgcn_sched_barrier(0);
            compute(1);
            if (kt + 2 < KT) sstore(R0, 0, false);
            __syncthreads();
        }
        if (kt < KT) compute(0);   // odd step count: the last step sits in buffer 0
    }

    // epilogue: residual product per block from the kept tiles, then Y.  Lane
    // (g, i) of block (nb, mb) holds channels 4g..4g+3 of token i.
    float sxr[MB], str[MB];
    int xfull[MB], xres[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {                    // this lane's tokens (staged in LDS)
        const int tl = wm * WR + mb * 16 + i;
        sxr[mb] = e_sx[tl];
        xfull[mb] = e_xf[tl];
        xres[mb] = e_xr[tl];
        str[mb] = e_st[tl];
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int col = n0 + wn * WC + nb * 16 + 4 * g;  // first of this lane's 4 channels
        const int cw = wn * WC + nb * 16 + 4 * g;        // its place in the tile (N % 16 == 0)
        const float4 swc = *reinterpret_cast<const float4 *>(e_sw + cw);
        const float4 src = *reinterpret_cast<const float4 *>(e_sr + cw);
        const int4 wsm = *reinterpret_cast<const int4 *>(e_ws + cw);
        const int4 rsm = *reinterpret_cast<const int4 *>(e_rs + cw);
        // the residual blocks of this channel block: MB independent MFMA chains
        v4i res[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) res[mb] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            if (c < RT) {
                v4i rhi, rlo;
                frag(rtile, wn * WC + nb * 16 + i, 4 * c + g, rhi, rlo);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    v4i ahi, alo;
                    frag(ares, wm * WR + mb * 16 + i, 4 * c + g, ahi, alo);
                    res[mb] = mfma_i8(rlo, ahi, res[mb]);
                    res[mb] = mfma_i8(rhi, alo, res[mb]);
                }
            }
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int row = m0 + wm * WR + mb * 16 + i;
            const v4i am = (acc[nb][mb] - 128 * (xfull[mb] + v4i{wsm.x, wsm.y, wsm.z, wsm.w})) >> 4;
            const v4i ar = (res[mb] - 128 * (xres[mb] + v4i{rsm.x, rsm.y, rsm.z, rsm.w})) >> 4;
            float4 y;
            if (!l2) {
                y.x = sxr[mb] * fmaf(swc.x, (float)am[0], src.x * (float)ar[0]);
                y.y = sxr[mb] * fmaf(swc.y, (float)am[1], src.y * (float)ar[1]);
                y.z = sxr[mb] * fmaf(swc.z, (float)am[2], src.z * (float)ar[2]);
                y.w = sxr[mb] * fmaf(swc.w, (float)am[3], src.w * (float)ar[3]);
            } else {   // the residual carries the intermediate's own token scale
                y.x = sxr[mb] * (swc.x * (float)am[0]) + str[mb] * (src.x * (float)ar[0]);
                y.y = sxr[mb] * (swc.y * (float)am[1]) + str[mb] * (src.y * (float)ar[1]);
                y.z = sxr[mb] * (swc.z * (float)am[2]) + str[mb] * (src.z * (float)ar[2]);
                y.w = sxr[mb] * (swc.w * (float)am[3]) + str[mb] * (src.w * (float)ar[3]);
            }
            if (args.H) {   // SwiGLU: channels col, col + 1 and col + 2, col + 3 are two (gate, up) pairs
                const int hc = min(col, N - 4) >> 1;
                const float2 sd = *reinterpret_cast<const float2 *>(args.sdown + hc);
                const float h0 = ((y.x / (1.0f + exp32(-y.x))) * y.y) / sd.x;
                const float h1 = ((y.z / (1.0f + exp32(-y.z))) * y.w) / sd.y;
                acc[nb][mb] = v4i{__float_as_int(h0), __float_as_int(h1), 0, 0};
            } else if (args.acc_main || args.direct_y) {   // direct stores (and the accumulators, if requested)
                if (row < M && col < N) {
                    const size_t o = (size_t)row * (size_t)N + col;
                    store_y(args.Y + o, y);
                    if (args.acc_main) {
                        *reinterpret_cast<v4i *>(args.acc_main + o) = am;
                        *reinterpret_cast<v4i *>(args.acc_res + o) = ar;
                    }
                }
            } else {
                acc[nb][mb] = v4i{__float_as_int(y.x), __float_as_int(y.y), __float_as_int(y.z), __float_as_int(y.w)};
            }
        }
    }
    if (args.acc_main || (args.direct_y && !args.H)) return;
    // Y through LDS: a lane holds 4 channels of one token, so direct stores
    // write 64-byte pieces of rows.  Each wave instead parks 32 tokens x 64
    // channels of its results in its own 8 KB of the (now idle) stage buffers
    // and reads them back as whole 256-byte rows, 4 rows per store
    // instruction.  16-byte chunk q of token row t sits at q ^ (t & 15).
    // The host takes this path when the tiles outnumber the CUs: a tile's
    // epilogue then overlaps other tiles' K loops and the whole rows pay.
    // With a single round of tiles every epilogue is exposed and the direct
    // stores, which skip the round trip through LDS, finish sooner.
    // With an even step count the K loop ended on a barrier after its last
    // read of the stage buffers; with an odd one the tail step read buffer 0.
    if (KT & 1) __syncthreads();
    uint8_t *const ybuf = smem + w * 8192;
    if (args.H) {
        // H: the wave's 64 channels are 32 hidden units, a lane's two at
        // hidden column 8 nb + 2 g of the wave; 32 tokens x 128 bytes parked
        // (16-byte chunk q of token row t at q ^ (t & 7)), then stored as
        // whole 128-byte rows, 8 rows per instruction
        const int Nh = N >> 1, h0 = (n0 + wn * WC) >> 1;
#pragma unroll
        for (int half = 0; half < MB / 2; ++half) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int ml = 0; ml < 2; ++ml) {
                    const int tl = ml * 16 + i, q = nb * 2 + (g >> 1);
                    *reinterpret_cast<int2 *>(ybuf + tl * 128 + ((q ^ (tl & 7)) * 16) + (g & 1) * 8) =
                        int2{acc[nb][2 * half + ml][0], acc[nb][2 * half + ml][1]};
                }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int tl = k * 8 + (lane >> 3), q = lane & 7;
                const float4 h = *reinterpret_cast<const float4 *>(ybuf + tl * 128 + ((q ^ (tl & 7)) * 16));
                const int row = m0 + wm * WR + half * 32 + tl, hcol = h0 + q * 4;
                if (row < M && hcol < Nh) store_y(args.H + (size_t)row * (size_t)Nh + hcol, h);
            }
        }
        return;
    }
#pragma unroll
    for (int half = 0; half < MB / 2; ++half) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int ml = 0; ml < 2; ++ml) {
                const int tl = ml * 16 + i, q = nb * 4 + g;
                *reinterpret_cast<v4i *>(ybuf + tl * 256 + ((q ^ (tl & 15)) * 16)) = acc[nb][2 * half + ml];
            }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int tl = k * 4 + (lane >> 4), q = lane & 15;
            const float4 y = *reinterpret_cast<const float4 *>(ybuf + tl * 256 + ((q ^ (tl & 15)) * 16));
            const int row = m0 + wm * WR + half * 32 + tl, col = n0 + wn * WC + q * 4;
            if (row < M && col < N) store_y(args.Y + (size_t)row * (size_t)N + col, y);
        }
    }
}

// ===========================================================================
// Prefill MXFP4 kernel.  Tile 128 x 128; one K step of 128 is one scaled
// MFMA per block, each lane group's 16 bytes being one 32-element MX block
// whose E8M0 scale the lane supplies.  The residual blocks are extra K blocks
// of the same fp32 accumulator: Q(R) carries its own block scales, so the
// extended K loop is literal.
// ===========================================================================
__global__ __launch_bounds__(G_THREADS) void k_gemm_mx(
    const uint8_t *__restrict__ xq, const uint8_t *__restrict__ xe, int M,
    const uint8_t *__restrict__ wq, const uint8_t *__restrict__ we,
    const uint8_t *__restrict__ rq, const uint8_t *__restrict__ re,
    int N, int K, int r_pad, float *__restrict__ Y) {
    constexpr int T_BYTES = G_BM * 64;              // one packed tile (A, W or R)
    constexpr int SC_BYTES = G_BM * 4;              // 4 E8M0 bytes per row per K step
    constexpr int STAGE = 3 * T_BYTES + 3 * SC_BYTES;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int i = lane & 15, g = lane >> 4;
    const int wm = w >> 1, wn = w & 1;
    const int m0 = blockIdx.y * G_BM, n0 = blockIdx.x * G_BN;
    const int KT = K >> 7, RT = r_pad >> 7;
    const size_t ld = (size_t)(K >> 1), sld = (size_t)(K >> 5);
    const size_t kg = (size_t)((KT + 3) / 4), rg = (size_t)((RT + 3) / 4);   // E8M0 groups of four steps a row

    // What_q and Q(R) rows sit in 1 KB tiles of 16 rows x one K step; the
    // weights' E8M0 bytes in 256-byte groups of 16 rows x four steps
    const uint8_t *a_src[2], *w_src[2], *r_src[2];
    int dst[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int c = t + u * G_THREADS, row = c >> 2, col = c & 3;
        a_src[u] = xq + (size_t)min(m0 + row, M - 1) * ld + col * 16;
        const size_t n = (size_t)min(n0 + row, N - 1);
        w_src[u] = wq + (n >> 4) * (size_t)KT * 1024 + (n & 15) * 64 + col * 16;
        r_src[u] = rq + (n >> 4) * (size_t)RT * 1024 + (n & 15) * 64 + col * 16;
        dst[u] = row * 64 + (col ^ swz4(row)) * 16;
    }
    // scale copies: threads 0..127 the activation rows, 128..255 the W and R rows
    const int srow = t & 127;
    const bool s_act = t < 128;
    const size_t sn = (size_t)min(n0 + srow, N - 1);
    const uint8_t *s_src = s_act ? xe + (size_t)min(m0 + srow, M - 1) * sld : we + ((sn >> 4) * kg * 16 + (sn & 15)) * 16;
    const uint8_t *sr_src = re + ((sn >> 4) * rg * 16 + (sn & 15)) * 16;
    // a step's E8M0 word: row-major for activations, in its group for weights
    auto sc_off = [](int kt, bool grouped) {
        return grouped ? (size_t)(kt >> 2) * 256 + (size_t)(kt & 3) * 4 : (size_t)kt * 4;
    };

    u32x4 ra[2], rw[2], rr[2];
    uint32_t rs = 0, rsr = 0;
    auto gload = [&](int kt, bool res) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            ra[u] = gld16(a_src[u] + (size_t)kt * 64);
            rw[u] = gld16(w_src[u] + (size_t)kt * 1024);
        }
        rs = *reinterpret_cast<const uint32_t *>(s_src + sc_off(kt, !s_act));
        if (res) {
#pragma unroll
            for (int u = 0; u < 2; ++u) rr[u] = gld16(r_src[u] + (size_t)kt * 1024);
            if (!s_act) rsr = *reinterpret_cast<const uint32_t *>(sr_src + sc_off(kt, true));
        }
    };
    auto sstore = [&](int buf, bool res) {
        uint8_t *s = smem + buf * STAGE;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            *reinterpret_cast<u32x4 *>(s + dst[u]) = ra[u];
            *reinterpret_cast<u32x4 *>(s + T_BYTES + dst[u]) = rw[u];
        }
        uint32_t *sc = reinterpret_cast<uint32_t *>(s + 3 * T_BYTES);
        sc[(s_act ? 0 : G_BM) + srow] = rs;
        if (res) {
#pragma unroll
            for (int u = 0; u < 2; ++u) *reinterpret_cast<u32x4 *>(s + 2 * T_BYTES + dst[u]) = rr[u];
            if (!s_act) sc[2 * G_BM + srow] = rsr;
        }
    };

    v4f acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};

    gload(0, RT > 0);
    sstore(0, RT > 0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const bool nxt = kt + 1 < KT;
        if (nxt) gload(kt + 1, kt + 1 < RT);
        const uint8_t *s = smem + (kt & 1) * STAGE;
        const uint8_t *sc = s + 3 * T_BYTES;
        v8i a[4];
        int sa[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            const int row = wm * 64 + rb * 16 + i;
            const u32x4 p = lds16(s + row * 64 + ((g ^ swz4(row)) * 16));
            a[rb] = v8i{(int)p.x, (int)p.y, (int)p.z, (int)p.w, 0, 0, 0, 0};
            sa[rb] = sc[row * 4 + g];
        }
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const int col = wn * 64 + cb * 16 + i;
            const u32x4 p = lds16(s + T_BYTES + col * 64 + ((g ^ swz4(col)) * 16));
            const v8i b = v8i{(int)p.x, (int)p.y, (int)p.z, (int)p.w, 0, 0, 0, 0};
            const int sb = sc[G_BM * 4 + col * 4 + g];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
                acc[rb][cb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[rb], b, acc[rb][cb], 4, 4,
                                                                              0, sa[rb], 0, sb);
        }
        if (kt < RT) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const int col = wn * 64 + cb * 16 + i;
                const u32x4 p = lds16(s + 2 * T_BYTES + col * 64 + ((g ^ swz4(col)) * 16));
                const v8i b = v8i{(int)p.x, (int)p.y, (int)p.z, (int)p.w, 0, 0, 0, 0};
                const int sb = sc[2 * G_BM * 4 + col * 4 + g];
#pragma unroll
                for (int rb = 0; rb < 4; ++rb)
                    acc[rb][cb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[rb], b, acc[rb][cb], 4,
                                                                                  4, 0, sa[rb], 0, sb);
            }
        }
        if (nxt) sstore((kt + 1) & 1, kt + 1 < RT);
        __syncthreads();
    }

#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const int col = n0 + wn * 64 + cb * 16 + i;
        if (col >= N) continue;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = m0 + wm * 64 + rb * 16 + 4 * g + v;
                if (row < M) Y[(size_t)row * (size_t)N + col] = acc[rb][cb][v];
            }
    }
}

// ===========================================================================
// MX W4A8 kernel: MXFP4 weights and Q(R) against MXFP8 (E4M3) activations on
// the same scaled MFMA (weights as the FP4 row operand, activations as the
// FP8 column operand, each lane giving its 32-element block's E8M0).  Every
// M.  Tile 256 tokens x 128 channels, 4 waves (128 x 64 each, one per SIMD,
// accumulators in AGPRs), K steps of 128 elements: 128 activation bytes and 64
// weight bytes a row.  A stage holds the activation, What_q and Q(R) tiles of
// one step and their E8M0 bytes; Q(R) is staged only for the first r_pad/128
// steps and adds its blocks to the same fp32 accumulators, so any r works.
// The FP8 operand of this MFMA is split in 16-byte halves: lane (g, i) holds
// elements 16 g .. 16 g + 15 in its first four registers and 64 + 16 g ..
// 64 + 16 g + 15 in the last four (found by a one-wave probe against host
// products; its E8M0 still scales the 32-element block g).  So a lane reads
// chunks g and g + 4 of a 128-byte activation row.  LDS placements (measured
// conflict-free on gfx950 for these reads): chunk c of a 64-byte weight row r
// at c ^ ((r >> 1) & 3), chunk c of an activation row at c ^ (r & 7).  Y
// leaves through LDS as in the other large-tile kernels.
// ===========================================================================
constexpr int M8_A = L_BM * 128, M8_W = L_BN * 64;
constexpr int M8_STAGE = M8_A + 2 * M8_W + (L_BM + 2 * L_BN) * 4;   // tiles + 4 E8M0 bytes a row
constexpr size_t kMx8Lds = 2 * M8_STAGE;

__device__ __forceinline__ int a8_pos(int c, int row) { return c ^ (row & 7); }
__device__ __forceinline__ int w4_pos(int c, int row) { return c ^ ((row >> 1) & 3); }

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_mx8(
    const uint8_t *__restrict__ xq, const uint8_t *__restrict__ xe, int M,
    const uint8_t *__restrict__ wq, const uint8_t *__restrict__ we,
    const uint8_t *__restrict__ rq, const uint8_t *__restrict__ re,
    int N, int K, int r_pad, float *__restrict__ Y, int gm) {
    constexpr int NT = 256, WR = 128, WC = 64, MB = WR / 16, NB = WC / 16;
    constexpr int ACH = M8_A / 16 / NT, WCH = M8_W / 16 / NT;       // 8 and 2 copies per thread
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int i = lane & 15, g = lane >> 4;
    const int wm = w >> 1, wn = w & 1;
    int tm, tn;
    tile_coords((M + L_BM - 1) / L_BM, (N + L_BN - 1) / L_BN, gm, tm, tn);
    const int m0 = tm * L_BM, n0 = tn * L_BN;
    const int KT = K >> 7, RT = r_pad >> 7;
    const uint32_t a_ld = (uint32_t)K, w_ld = (uint32_t)(K >> 1), r_ld = (uint32_t)(r_pad >> 1);
    const uint32_t s_ld = (uint32_t)(K >> 5);
    const uint32_t kg = (uint32_t)((KT + 3) / 4), rg = (uint32_t)((RT + 3) / 4);   // E8M0 groups of four steps

    // copy plan (rows past M or N lie past the end of their buffer and read
    // as zero).  What_q and Q(R) rows sit in 1 KB tiles of 16 rows x one K
    // step (a round of 64 rows is four whole tiles of the step); the weights'
    // E8M0 bytes in 256-byte groups of 16 rows x four steps.
    const int crow = t >> 3, ccol = t & 7;          // activation: 32 rows x 8 chunks per round
    const int wrow = t >> 2, wcol = t & 3;          // weights / Q(R): 64 rows x 4 chunks per round
    const uint32_t a_off = (uint32_t)(m0 + crow) * a_ld + ccol * 16;
    const uint32_t wn_ = (uint32_t)(n0 + wrow);
    const uint32_t w_off = (wn_ >> 4) * (uint32_t)KT * 1024 + (wn_ & 15) * 64 + wcol * 16;
    const uint32_t r_off = (wn_ >> 4) * (uint32_t)RT * 1024 + (wn_ & 15) * 64 + wcol * 16;
    const int a_dst = crow * 128 + a8_pos(ccol, crow) * 16;        // + u * 32 rows (a8_pos repeats every 8)
    const int w_dst = wrow * 64 + w4_pos(wcol, wrow) * 16;         // + u * 64 rows
    const rsrc_t ra = make_rsrc(xq, (size_t)M * a_ld), rw = make_rsrc(wq, (size_t)N * w_ld);
    const rsrc_t rr = make_rsrc(rq, (size_t)N * r_ld);
    const rsrc_t rsa = make_rsrc(xe, (size_t)M * s_ld), rsw = make_rsrc(we, (size_t)N * kg * 16);
    const rsrc_t rsr = make_rsrc(re, (size_t)N * rg * 16);
    // scale bytes: thread t moves activation row t; waves 0-1 weight row t,
    // waves 2-3 Q(R) row t - 128
    const bool w_sc = w < 2;
    const uint32_t sa_off = (uint32_t)(m0 + t) * s_ld;
    const uint32_t sw_n = (uint32_t)(n0 + (w_sc ? t : t - 128));
    const uint32_t sw_off = ((sw_n >> 4) * (w_sc ? kg : rg) * 16 + (sw_n & 15)) * 16;
    constexpr int SC = M8_A + 2 * M8_W;                               // scale bytes within a stage

    struct Regs {
        u32x4 a[ACH], w[WCH], r[WCH];
        uint32_t sa, sw;
    };
    auto gload = [&](Regs &R, int kt) {
        const bool res = kt < RT;
#pragma unroll
        for (int u = 0; u < ACH; ++u)
            R.a[u] = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)(a_off + u * 32 * a_ld), (int)((uint32_t)kt * 128), 0);
        const uint32_t gs = (uint32_t)(kt >> 2) * 256 + (uint32_t)(kt & 3) * 4;   // the step's word in its group
#pragma unroll
        for (int u = 0; u < WCH; ++u)
            R.w[u] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(w_off + u * 4 * (uint32_t)KT * 1024),
                                                           (int)((uint32_t)kt * 1024), 0);
        if (res) {
#pragma unroll
            for (int u = 0; u < WCH; ++u)
                R.r[u] = __builtin_amdgcn_raw_buffer_load_b128(rr, (int)(r_off + u * 4 * (uint32_t)RT * 1024),
                                                               (int)((uint32_t)kt * 1024), 0);
        }
        R.sa = __builtin_amdgcn_raw_buffer_load_b32(rsa, (int)(sa_off + (uint32_t)kt * 4), 0, 0);
        if (w_sc) R.sw = __builtin_amdgcn_raw_buffer_load_b32(rsw, (int)(sw_off + gs), 0, 0);
        else if (res) R.sw = __builtin_amdgcn_raw_buffer_load_b32(rsr, (int)(sw_off + gs), 0, 0);
    };
    auto sstore = [&](const Regs &R, int buf, int kt) {
        const bool res = kt < RT;
        uint8_t *s = smem + buf * M8_STAGE;
#pragma unroll
        for (int u = 0; u < ACH; ++u) *reinterpret_cast<u32x4 *>(s + a_dst + u * 32 * 128) = R.a[u];
#pragma unroll
        for (int u = 0; u < WCH; ++u) *reinterpret_cast<u32x4 *>(s + M8_A + w_dst + u * 64 * 64) = R.w[u];
        if (res) {
#pragma unroll
            for (int u = 0; u < WCH; ++u) *reinterpret_cast<u32x4 *>(s + M8_A + M8_W + w_dst + u * 64 * 64) = R.r[u];
        }
        *reinterpret_cast<uint32_t *>(s + SC + t * 4) = R.sa;
        if (w_sc) *reinterpret_cast<uint32_t *>(s + SC + (L_BM + t) * 4) = R.sw;
        else if (res) *reinterpret_cast<uint32_t *>(s + SC + (L_BM + L_BN + t - 128) * 4) = R.sw;
    };

    v4f acc[NB][MB];
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
        for (int b = 0; b < MB; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};

    // One step from LDS buffer buf (with Q(R) for the first RT steps).
    // Weights are the MFMA row operand: lane (g, i) of block (nb, mb) holds
    // channels 4 g .. 4 g + 3 of token i.
    auto compute = [&](int buf, bool with_res) {
        const uint8_t *s = smem + buf * M8_STAGE;
        v8i af[MB];
        int sa[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int row = wm * WR + mb * 16 + i;
            const u32x4 lo = lds16(s + row * 128 + a8_pos(g, row) * 16);
            const u32x4 hi = lds16(s + row * 128 + a8_pos(g + 4, row) * 16);
            af[mb] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            sa[mb] = s[SC + row * 4 + g];
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int row = wn * WC + nb * 16 + i;
            const u32x4 p = lds16(s + M8_A + row * 64 + w4_pos(g, row) * 16);
            const v8i bf = v8i{(int)p.x, (int)p.y, (int)p.z, (int)p.w, 0, 0, 0, 0};
            const int sb = s[SC + (L_BM + row) * 4 + g];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                acc[nb][mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af[mb], acc[nb][mb], 4, 0, 0, sb,
                                                                              0, sa[mb]);
        }
        if (with_res) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int row = wn * WC + nb * 16 + i;
                const u32x4 p = lds16(s + M8_A + M8_W + row * 64 + w4_pos(g, row) * 16);
                const v8i rf = v8i{(int)p.x, (int)p.y, (int)p.z, (int)p.w, 0, 0, 0, 0};
                const int sr = s[SC + (L_BM + L_BN + row) * 4 + g];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[nb][mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(rf, af[mb], acc[nb][mb], 4, 0, 0,
                                                                                  sr, 0, sa[mb]);
            }
        }
    };

    // Two register sets carry the prefetch two steps ahead (issued
    // unconditionally: past the last step it re-reads step KT - 1).
    Regs R0, R1;
    gload(R0, 0);
    gload(R1, min(1, KT - 1));
    sstore(R0, 0, 0);
    __syncthreads();
    int kt = 0;
    for (; kt + 2 <= KT; kt += 2) {
        gload(R0, min(kt + 2, KT - 1));
        __builtin_amdgcn_sched_barrier(0);
        compute(0, kt < RT);
        sstore(R1, 1, kt + 1);
        __syncthreads();
        gload(R1, min(kt + 3, KT - 1));
        __builtin_amdgcn_sched_barrier(0);
        compute(1, kt + 1 < RT);
        if (kt + 2 < KT) sstore(R0, 0, kt + 2);
        __syncthreads();
    }
    if (kt < KT) compute(0, kt < RT);   // odd step count: the last step sits in buffer 0

    // Y through LDS: each wave parks 32 tokens x 64 channels at a time in its
    // own 8 KB of the idle stage buffers and stores whole 256-byte rows.
    if (KT & 1) __syncthreads();
    uint8_t *const ybuf = smem + w * 8192;
#pragma unroll
    for (int part = 0; part < MB / 2; ++part) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int ml = 0; ml < 2; ++ml) {
                const int tl = ml * 16 + i, q = nb * 4 + g;
                *reinterpret_cast<v4f *>(ybuf + tl * 256 + ((q ^ (tl & 15)) * 16)) = acc[nb][2 * part + ml];
            }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int tl = k * 4 + (lane >> 4), q = lane & 15;
            const float4 y = *reinterpret_cast<const float4 *>(ybuf + tl * 256 + ((q ^ (tl & 15)) * 16));
            const int row = m0 + wm * WR + part * 32 + tl, col = n0 + wn * WC + q * 4;
            if (row < M && col < N) store_y(Y + (size_t)row * (size_t)N + col, y);
        }
    }
}

// ===========================================================================
// L2QER comparator: the intermediate T = X_q . L1_q and its on-the-fly
// quantization (the two-matrix path of the SERQ notes page, key equations;
// the zh technical summary, section 2.1, on why it costs latency), one
// kernel.  A workgroup of NW waves owns one block of 16 tokens and all
// k_pad = 16 NB columns; wave w takes the w-th of NW slices of K.  Operands
// come straight from global memory: a token row's 16-byte chunk per lane and
// the tiled L1_q (one coalesced 1 KB tile per 16 columns and 128 elements),
// D chunks in flight.  The exact int32 slices are summed in LDS; the code-sum
// offsets (128 (even-k activation codes + odd-k L1_q codes), the raw sum
// being 16 times the true product otherwise) are removed; then 32 lanes per
// token dequantize T = sx * (sL1 * A1) in fp32 and quantize it per token
// exactly like a layer input of width k_pad (codes, fp32 scale, running
// even-k code sums per 128 columns).
// ===========================================================================
constexpr int L2Q_NW = 8;

template <int NB>
__global__ __launch_bounds__(64 * L2Q_NW) void k_l2qer(const uint8_t *__restrict__ xq, const float *__restrict__ sx,
                                                      const int *__restrict__ xsum, int M, int K,
                                                      const uint8_t *__restrict__ l1q, const float *__restrict__ sl1,
                                                      const int *__restrict__ l1sum, float *__restrict__ T,
                                                      uint8_t *__restrict__ tq, float *__restrict__ st,
                                                      int *__restrict__ tsum) {
    constexpr int KP = NB * 16;
    extern __shared__ __attribute__((aligned(16))) int red[];     // [NW][16][KP] int32
    const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int i = lane & 15, g = lane >> 4;
    const int m0 = blockIdx.x * 16;
    const int KC = K >> 7;
    const int c0 = (int)((long)KC * w / L2Q_NW), c1 = (int)((long)KC * (w + 1) / L2Q_NW);
    const int row = min(m0 + i, M - 1);
    const uint8_t *xr = xq + (size_t)row * (size_t)(K >> 1) + g * 16;
    const uint8_t *wr = l1q + i * 64 + g * 16;
    struct Frag {
        u32x4 x, w[NB];
    };
    auto ld = [&](Frag &F, int c) {
        F.x = gld16(xr + (size_t)c * 64);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) F.w[nb] = gld16(wr + ((size_t)nb * KC + c) * 1024);
    };
    v4i acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = v4i{0, 0, 0, 0};
    auto mma = [&](const Frag &F) {
        v4i ahi, alo;
        split_hi_lo(F.x, ahi, alo);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            v4i whi, wlo;
            split_hi_lo(F.w[nb], whi, wlo);
            acc[nb] = mfma_i8(wlo, ahi, acc[nb]);
            acc[nb] = mfma_i8(whi, alo, acc[nb]);
        }
    };
    if (c0 < c1) {   // wave-uniform; a slice is empty only when K / 128 < NW
        // D chunks in flight (a ring indexed at compile time; one chunk at
        // k_pad = 256, whose fragments and accumulators alone take 132
        // registers); no load is issued past the slice (the tests on c are
        // wave-uniform, scalar branches), so nothing is left in flight for
        // the epilogue to wait on
        constexpr int D = NB <= 8 ? 4 : 1;
        Frag F[D];
#pragma unroll
        for (int d = 0; d < D; ++d)
            if (c0 + d < c1) ld(F[d], c0 + d);
        for (int c = c0; c < c1; c += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                if (c + d < c1) mma(F[d]);
                if (c + d + D < c1) ld(F[d], c + d + D);
            }
        }
    }
    // lane (g, i) of block nb holds columns 16 nb + 4 g .. + 3 of token i
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        *reinterpret_cast<v4i *>(red + (w * 16 + i) * KP + nb * 16 + 4 * g) = acc[nb];
    __syncthreads();

    // 32 lanes per token: token r = t / 32 (16 tokens x 32 = 512 threads),
    // lane u of the token owns 4-column chunks u + 32 v, v < KP / 128
    constexpr int CPL = KP / 128;
    const int r = t >> 5, u = t & 31, m = m0 + r;
    const int mc = min(m, M - 1);
    const float sxm = sx[mc];
    const int xoff = xsum[(size_t)mc * KC + KC - 1];
    float4 tv[CPL];
    float amax = 0.0f;
#pragma unroll
    for (int v = 0; v < CPL; ++v) {
        const int j = u + 32 * v;
        v4i a = v4i{0, 0, 0, 0};
#pragma unroll
        for (int ww = 0; ww < L2Q_NW; ++ww) a += *reinterpret_cast<const v4i *>(red + (ww * 16 + r) * KP + 4 * j);
        const int4 ws = *reinterpret_cast<const int4 *>(l1sum + 4 * j);
        const float4 sc = *reinterpret_cast<const float4 *>(sl1 + 4 * j);
        const v4i A = (a - 128 * (v4i{ws.x, ws.y, ws.z, ws.w} + xoff)) >> 4;
        tv[v] = make_float4(sxm * (sc.x * (float)A[0]), sxm * (sc.y * (float)A[1]), sxm * (sc.z * (float)A[2]),
                            sxm * (sc.w * (float)A[3]));
        amax = fmaxf(amax, amax4(tv[v]));
    }
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const float s = amax / 7.0f;
    const bool live = m < M;
    if (live && u == 0) st[m] = s;
    int run = 0;
#pragma unroll
    for (int v = 0; v < CPL; ++v) {
        const int j = u + 32 * v;
        const float4 x = tv[v];
        int q0 = 0, q1 = 0, q2 = 0, q3 = 0;
        if (s > 0.0f) {
            q0 = rtn_code<7>(x.x, s);
            q1 = rtn_code<7>(x.y, s);
            q2 = rtn_code<7>(x.z, s);
            q3 = rtn_code<7>(x.w, s);
        }
        // activation nibbles: even k two's complement high, odd k offset low
        const uint32_t b = ((uint32_t)(q0 & 15) << 4) | (uint32_t)(q1 + 8) | ((uint32_t)(q2 & 15) << 12) |
                           ((uint32_t)(q3 + 8) << 8);
        int e = q0 + q2;                                   // even-k codes of 128-column block v
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) e += __shfl_xor(e, o);
        run += e;
        if (live) {
            *reinterpret_cast<uint16_t *>(tq + (size_t)m * (KP / 2) + 2 * j) = (uint16_t)b;
            if (T) *reinterpret_cast<float4 *>(T + (size_t)m * KP + 4 * j) = x;
            if (u == 0) tsum[(size_t)m * CPL + v] = run;
        }
    }
}

// ===========================================================================
// L2QER intermediate in MXFP4: T = X_q . L1_q and its per-token MXFP4
// quantization (k_pad = 128).  Every 32-element block's scaled product is
// exact (E2M1 products are multiples of 1/4, 32 of them sum to at most 1152,
// and the E8M0 scales are powers of two), so each K step runs four MFMAs,
// each with one block's L1 fragment and the others zero, and adds the four
// exact results in fp64.  An fp64 sum of such terms stays exact while their
// scales span fewer than about 30 binades, so T is the exact block sum
// rounded once to fp32 whatever the order of the additions.  (One MFMA per
// step would sum the four blocks in its own fp32 order.)  L1_q is stored as
// the MXFP4 weights of a d_in -> k_pad layer (1 KB tiles of 16 columns x 128
// elements, E8M0 groups).  T goes through LDS to be quantized like an MXFP4
// activation row of width k_pad (the activation quantizer's chunk encoding).
// ===========================================================================
constexpr int L2X_KP = 128;   // k_pad of the MXFP4 comparator
constexpr int L2X_CG = 32;    // intermediate columns per workgroup: one MX block of each token
constexpr int L2X_KS = 8;     // K splits (waves) per workgroup

// One workgroup: 16 tokens x 32 columns of T, eight waves, each on both
// 16-column blocks for every eighth pair of K steps (wave q takes pairs q,
// q + 8, ..., starting at a pair rotated by the token block so that the
// workgroups do not all ask for the same L1 lines at once).  Within a pair
// (256 elements, eight MX blocks) lane group g holds blocks 2g and 2g + 1 --
// 32 contiguous bytes of a row, one request for the two steps -- and the
// pair's two MFMA steps take the even and the odd blocks; L1's lanes follow
// the same assignment, so each MFMA still pairs one block of X with the same
// block of L1.  The loads of the next pair go out before the current pair's
// MFMAs.  The eight partial fp64 sums meet in LDS, are rounded to fp32 and
// quantized as the tokens' MX block of those 32 columns.  Workgroup b sits on
// XCD b % 8; the four column groups of one token block are consecutive on
// one XCD, so they share its L2 copy of the activation rows.
__global__ __launch_bounds__(64 * L2X_KS) void k_l2qer_mx(
    const uint8_t *__restrict__ xq, const uint8_t *__restrict__ xe, int M, int K,
    const uint8_t *__restrict__ l1q, const uint8_t *__restrict__ l1e, float *__restrict__ T,
    uint8_t *__restrict__ tq, uint8_t *__restrict__ te) {
    constexpr uint32_t kOut = 0x80000000u;                      // an offset past every buffer: reads zero
    const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int i = lane & 15, g = lane >> 4;
    const int b = blockIdx.x, xcd = b & 7, loc = b >> 3;
    const int tb = (loc >> 2) * 8 + xcd, cg = loc & 3;          // token block, column group
    const int m0 = tb * 16;
    if (m0 >= M) return;                                         // the grid is rounded up to whole XCD rounds
    const int KT = K >> 7, NP = (KT + 1) >> 1;                   // K steps, pairs (the last may be half)
    const uint32_t KG = (uint32_t)((KT + 3) / 4);
    const rsrc_t ra = make_rsrc(xq, (size_t)M * (size_t)(K >> 1)), rsa = make_rsrc(xe, (size_t)M * (size_t)(K >> 5));
    const rsrc_t rw = make_rsrc(l1q, (size_t)L2X_KP * (size_t)(K >> 1)), rsw = make_rsrc(l1e, (size_t)L2X_KP * KG * 16);
    const bool row_in = m0 + i < M;
    const uint32_t aro = (uint32_t)(m0 + i) * (uint32_t)(K >> 1) + g * 32;   // + 128 p
    const uint32_t aso = (uint32_t)(m0 + i) * (uint32_t)(K >> 5);            // + 8 p
    const int gh = g >> 1, gl = g & 1;                           // the step of the pair holding blocks 2g, 2g + 1
    const uint32_t wro0 = (uint32_t)(cg * 2) * (uint32_t)KT * 1024 + i * 64 + gl * 32;   // + (2p + gh) 1 KB
    const uint32_t wso0 = (uint32_t)(cg * 2) * KG * 256 + i * 16;
    struct Pair {
        u32x4 a0, a1, b0[2], b1[2];
        uint32_t sa0, sa1, sw[2];
    };
    auto load = [&](int p, Pair &P) {   // p >= NP, rows past M, steps past KT: zero
        const int kt = 2 * p + gh;
        const bool in = p < NP && kt < KT;
        const uint32_t ao = in && row_in ? aro + (uint32_t)p * 128 : kOut;
        P.a0 = bld16(ra, ao);
        P.a1 = bld16(ra, ao + 16);
        const uint32_t so = p < NP && row_in ? aso + (uint32_t)p * 8 : kOut;
        P.sa0 = __builtin_amdgcn_raw_buffer_load_b32(rsa, (int)so, 0, 0);
        P.sa1 = __builtin_amdgcn_raw_buffer_load_b32(rsa, (int)(so + 4), 0, 0);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const uint32_t wo = in ? wro0 + (uint32_t)cb * (uint32_t)KT * 1024 + (uint32_t)kt * 1024 : kOut;
            P.b0[cb] = bld16(rw, wo);
            P.b1[cb] = bld16(rw, wo + 16);
            P.sw[cb] = __builtin_amdgcn_raw_buffer_load_b32(
                rsw, (int)(in ? wso0 + (uint32_t)cb * KG * 256 + (uint32_t)(kt >> 2) * 256 + (uint32_t)(kt & 3) * 4 : kOut),
                0, 0);
        }
    };
    double acc[2][4] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};
    // one MFMA step: lane group g's block (its X fragment a, L1 fragment bw and
    // their E8M0 bytes), four MFMAs with one lane group live each
    auto step = [&](const u32x4 &a, const u32x4 &bw, int s_a, int s_w, double *ac) {
        const v8i af = v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
#pragma unroll
        for (int g0 = 0; g0 < 4; ++g0) {
            const bool on = g == g0;
            const v8i bf = v8i{on ? (int)bw.x : 0, on ? (int)bw.y : 0, on ? (int)bw.z : 0, on ? (int)bw.w : 0, 0, 0, 0, 0};
            const v4f r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af, v4f{0.f, 0.f, 0.f, 0.f}, 4, 4, 0,
                                                                           s_w, 0, s_a);
#pragma unroll
            for (int v = 0; v < 4; ++v) ac[v] += (double)r[v];
        }
    };
    auto pair = [&](const Pair &P) {
        const uint32_t sa = gh ? P.sa1 : P.sa0;                  // the dword of blocks 4 gh .. 4 gh + 3
        const int a_even = (int)((sa >> (16 * gl)) & 255u), a_odd = (int)((sa >> (16 * gl + 8)) & 255u);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const int w_even = (int)((P.sw[cb] >> (16 * gl)) & 255u), w_odd = (int)((P.sw[cb] >> (16 * gl + 8)) & 255u);
            step(P.a0, P.b0[cb], a_even, w_even, acc[cb]);
            step(P.a1, P.b1[cb], a_odd, w_odd, acc[cb]);
        }
    };
    const int q = w;                                              // K part
    const int J = NP > q ? (NP - q + L2X_KS - 1) / L2X_KS : 0;   // pairs of this wave
    const int rot = J > 0 ? tb % J : 0;
    auto pidx = [&](int j) {                                      // the wave's j-th pair; past the last: NP (zero)
        if (j >= J) return NP;
        int r = j + rot;
        if (r >= J) r -= J;
        return q + L2X_KS * r;
    };
    // the next pair's loads go out before this pair's MFMAs (the copy at the
    // end of an iteration waits for them: deeper prefetch variants measured
    // slower, the load path being throughput-bound)
    Pair cur, nxt;
    load(pidx(0), cur);
    for (int j = 0; j < J; ++j) {
        load(pidx(j + 1), nxt);
        pair(cur);
        cur = nxt;
    }
    // lane (i, g): token m0 + i, columns 16 cb + 4 g .. + 3 of the group
    __shared__ double part[L2X_KS][16][L2X_CG + 1];
    __shared__ float tt[16][L2X_CG + 4];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int v = 0; v < 4; ++v) part[q][i][cb * 16 + 4 * g + v] = acc[cb][v];
    __syncthreads();
    {   // one (token, column) a thread
        const int tok = t >> 5, c = t & 31;
        double y = part[0][tok][c];
#pragma unroll
        for (int k = 1; k < L2X_KS; ++k) y += part[k][tok][c];
        tt[tok][c] = (float)y;
        if (T && m0 + tok < M) T[(size_t)(m0 + tok) * L2X_KP + cg * L2X_CG + c] = (float)y;
    }
    __syncthreads();
    // quantization: threads 0 .. 127, token t / 8, chunk t % 8 of the group's block
    if (t < 128) {
        const int tok = t >> 3, c = t & 7;
        const float4 u = make_float4(tt[tok][4 * c], tt[tok][4 * c + 1], tt[tok][4 * c + 2], tt[tok][4 * c + 3]);
        if (m0 + tok < M)
            mx_encode_chunk<false>(u, cg * 8 + c, tq + (size_t)(m0 + tok) * (L2X_KP / 2),
                                   te + (size_t)(m0 + tok) * (L2X_KP / 32));
    }
}

// ===========================================================================
// Wide MXFP4 kernel with LDS-direct copies (r_pad <= 128, d_in % 512 == 0).
// 256 tokens x 32 NB channels per workgroup (NB = 6, 7 or 8 blocks of 16
// channels per wave: the host picks the width whose tile count fills the
// last round of workgroups best), 4 waves of 128 x 16 NB with up to 256 fp32
// accumulators in AGPRs, K steps of 128; at 128 channels, NW = 8 waves of
// 64 x 64, two per SIMD.  Per MFMA a 128 x 16 NB wave tile moves fewer LDS
// bytes than a 128 x 64 one, whose LDS traffic at the MX MFMA rates comes
// close to the LDS's own limit.  The global reads go straight into LDS: buffer loads with an LDS destination write each lane's
// 16 bytes to consecutive LDS in lane order, so no VGPRs and no LDS store
// instructions carry the copies; the fragment registers that frees hold two
// steps, and the LDS reads of step k + 1 go out between step k's MFMAs.
// What bounds the copies is the L2's request rate, not its bytes (counters:
// its channels 93 % busy with 64-byte pieces and 4-byte E8M0 loads): every
// load lane group that touches a 128-byte line is one request however few
// bytes it brings.  So each copy moves whole 128-byte row pieces -- two K
// steps -- into stages of two steps (two stages, refilled one pair ahead),
// and the E8M0 bytes come 16 per row (four steps of four groups) once every
// four steps, with stage 0; when a lane reads the fragments of step 4q it
// also takes its own scale byte of each block for steps 4q .. 4q + 3, packed
// into one register (byte s for step 4q + s) that the MFMA's scale byte
// select then picks.  Q(R) (one 64-byte row per channel at r_pad = 128) and
// its E8M0 bytes come into a tile of their own in the prologue; its MFMAs
// run against step 0's activation fragments before the K loop.
// The LDS layout keeps 64-byte rows with the swizzle of k_gemm_mx8's weight
// rows (16-byte chunk c of row r at c ^ ((r >> 1) & 3)): a copy's 1 KB holds its eight
// rows' first step, then their second, and since the LDS placement is fixed
// by the lane, each lane fetches the global chunk that belongs at its slot.
// The stages are separate LDS arrays and the loop is unrolled over four
// steps, so the compiler can tell which stage a fragment read depends on;
// the barriers are bare s_barrier with explicit counter waits, because a
// workgroup fence would wait for every LDS-direct load in flight.
// ===========================================================================
#define SERQ_LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

template <int NB, int NW, bool TQ = false>
struct MxDma {
    static constexpr int BN = 32 * NB;                 // channels per tile
    static constexpr int A = L_BM * 128;               // activation rows of two steps: 256 x 128 bytes
    static constexpr int STAGE = A + NB * 4096;        // + weight rows of two steps: 32 NB x 128 bytes
    static constexpr int GA = STAGE, GW = GA + 4096;   // stage 0 only: E8M0 of four steps, 256 x 16 bytes each
    static constexpr int STAGE0 = GW + 4096;
    // Q(R) tile and its E8M0 (with TQ the L2 factor's, and the tile not
    // rounded up to whole 4 KB, to leave room for Q(T))
    static constexpr int QW = TQ ? BN * 64 : ((BN * 64 + 4095) / 4096) * 4096, QR = QW + 256 * 4;
    static constexpr int TT = TQ ? L_BM * 64 : 0, TQS = TQ ? TT + L_BM * 4 : 16;   // Q(T) tile and its E8M0
    static constexpr int UA = 32 / NW, UW = 4 * NB / NW;   // activation / weight copies per thread and pair
    static constexpr int ND = UA + UW;                 // LDS-direct loads per thread and pair of steps
    static constexpr int NG = 8 / NW;                  // + the E8M0 group's, into stage 0
};

// Issue pattern of one K step of NM MFMAs: MFMA k follows a copy when
// floor((k + 1) ND / NM) > floor(k ND / NM), so the ND copies spread evenly
// over the step, and, for k < NR, one fragment read.  A copy is 1 KB through
// the CU's vector memory path, which takes about as long as three FP4 MFMAs
// issue; bunched at the start of a step, the copies stall the in-order MFMA
// issue behind them.
template <int K, int NM, int ND, int NR>
__device__ __forceinline__ void sched_spread() {
    if constexpr (K < NM) {
        if constexpr (((K + 1) * ND) / NM > (K * ND) / NM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read
        if constexpr (K < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                // LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                                     // MFMA
        sched_spread<K + 1, NM, ND, NR>();
    }
}

// s_waitcnt with vmcnt <= vm and lgkmcnt <= lgkm (15: no wait), expcnt untouched
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }

template <int NB, int NW, bool TQ = false, bool SQ = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void k_gemm_mxd(
    const uint8_t *__restrict__ xq, const uint8_t *__restrict__ xe, int M,
    const uint8_t *__restrict__ wq, const uint8_t *__restrict__ we,
    const uint8_t *__restrict__ rq, const uint8_t *__restrict__ re,
    int N, int K, int r_pad, float *__restrict__ Y, int gm,
    const uint8_t *__restrict__ tq = nullptr, const uint8_t *__restrict__ te = nullptr,
    const float *__restrict__ s_next = nullptr, uint8_t *__restrict__ xqn = nullptr,
    uint8_t *__restrict__ xen = nullptr) {
    using L = MxDma<NB, NW, TQ>;
    static_assert(NW == 4 || (NW == 8 && NB == 4), "four waves, or eight at 128 channels");
    static_assert(!TQ || NB <= 7, "Q(T) fits beside the stages up to 224 channels");
    static_assert(!SQ || (NB * 8) % 32 == 0, "SQ: a wave's columns hold whole MX blocks of the next layer's input");
    constexpr int WR = 512 / NW, WC = NB * 16, MB = WR / 16, BN = L::BN, ND = L::ND, NG = L::NG;
    constexpr int UA = L::UA, UW = L::UW;
    __shared__ __attribute__((aligned(16))) uint8_t st0[L::STAGE0], st1[L::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t qr[L::QR];
    __shared__ __attribute__((aligned(16))) uint8_t tqs[L::TQS];   // TQ: Q(T) rows, then their E8M0 bytes
    const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int i = lane & 15, g = lane >> 4;
    const int wm = w >> 1, wn = w & 1;
    int tm, tn;
    tile_coords((M + L_BM - 1) / L_BM, (N + BN - 1) / BN, gm, tm, tn);
    const int m0 = tm * L_BM, n0 = tn * BN;
    const int KT = K >> 7;
    const uint32_t ld = (uint32_t)(K >> 1), s_ld = (uint32_t)(K >> 5);
    constexpr uint32_t kOut = 0x80000000u;                      // an offset past every buffer: reads zero

    // copy plan: copy u of wave w moves rows (NW u + w) * 8 .. + 7 of two K
    // steps (64 bytes a row and step) into 1 KB of LDS laid out as the first
    // step's eight 64-byte rows, then the second's; lane l takes slot l & 3
    // of row (l >> 2) & 7 of step l >> 5, which holds that step's global
    // chunk (l & 3) ^ ((row >> 1) & 3).  Activation rows are row-major (one
    // 128-byte piece a row); weight rows sit in 1 KB tiles of 16 rows x one
    // step, so a weight copy reads two 512-byte halves of consecutive tiles.
    // The E8M0 copies give lane l of wave w the 16 bytes of row (w % 4) * 64
    // + l for four steps (activations: a row-major row piece; weights: the
    // row's 16 bytes in its block's 256-byte group).  Offsets past a buffer's
    // end (rows past M or N) read as zero.
    const int lr = (lane >> 2) & 7, lh = lane >> 5, gw = w & 3;
    const uint32_t lchunk = (uint32_t)(((lane & 3) ^ ((lr >> 1) & 3)) * 16);
    uint32_t va[UA], vw[UW];
#pragma unroll
    for (int u = 0; u < UA; ++u) va[u] = (uint32_t)(m0 + (NW * u + w) * 8 + lr) * ld + lh * 64 + lchunk;
#pragma unroll
    for (int u = 0; u < UW; ++u) {
        const uint32_t n = (uint32_t)(n0 + (NW * u + w) * 8 + lr);
        vw[u] = ((n >> 4) * (uint32_t)KT + lh) * 1024 + (n & 15) * 64 + lchunk;
    }
    const uint32_t sn = (uint32_t)(n0 + gw * 64 + lane), kg4 = (uint32_t)(KT / 4);
    const uint32_t vsa = (uint32_t)(m0 + gw * 64 + lane) * s_ld;
    const uint32_t vsw = gw * 64 + lane < BN ? ((sn >> 4) * kg4 * 16 + (sn & 15)) * 16 : kOut;
    const rsrc_t ra = make_rsrc(xq, (size_t)M * ld), rw = make_rsrc(wq, (size_t)N * ld);
    const rsrc_t rsa = make_rsrc(xe, (size_t)M * s_ld), rsw = make_rsrc(we, (size_t)N * kg4 * 16);

    // steps 2 p and 2 p + 1 into stage stg; into stage 0 (p even but for the
    // clamped copies past the last pair) also the E8M0 bytes of steps 2 p ..
    // 2 p + 3, first
    auto dma = [&](auto SI, uint8_t *stg, int p) {
        if constexpr (decltype(SI)::value == 0) {
            const int q = p >> 1;   // the four-step group
            if (NW == 4 || w < 4)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, SERQ_LDS_PTR(stg + L::GA + gw * 1024), 16, (int)vsa, q * 16,
                                                         0, 0);
            if (NW == 4 || w >= 4)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, SERQ_LDS_PTR(stg + L::GW + gw * 1024), 16, (int)vsw,
                                                         q * 256, 0, 0);
        }
        // the pair's byte offsets within an activation row and within a block
        // of weight tiles (never decide a bound)
        const int ka = p * 128, kw = p * 2048;
#pragma unroll
        for (int u = 0; u < UA; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, SERQ_LDS_PTR(stg + (NW * u + w) * 1024), 16, (int)va[u], ka, 0, 0);
#pragma unroll
        for (int u = 0; u < UW; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, SERQ_LDS_PTR(stg + L::A + (NW * u + w) * 1024), 16, (int)vw[u], kw,
                                                     0, 0);
    };
    auto barrier = [&]() {
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;

    // prologue: Q(R) (one K step: its tiles are 64-byte rows in channel
    // order; the step's E8M0 bytes lead each row's 16-byte group), then steps
    // 0 .. 3 into the two stages
    const bool has_r = r_pad > 0;
    if (has_r) {
        const rsrc_t rr = make_rsrc(rq, (size_t)N * 64), rsr = make_rsrc(re, (size_t)N * 16);
        const int qrow = lane >> 2, qcol = (lane & 3) ^ ((qrow >> 1) & 3);
        if constexpr (TQ) {
            for (int c = w; c < L::QW / 1024; c += NW) {
                const int row = c * 16 + qrow;
                const uint32_t v = row < BN ? (uint32_t)(n0 + row) * 64 + qcol * 16 : kOut;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, SERQ_LDS_PTR(qr + c * 1024), 16, (int)v, 0, 0, 0);
            }
            // Q(T): 256 token rows of 64 bytes (row-major [M][64]) in the same
            // swizzled layout, then their four E8M0 bytes each
            const rsrc_t rt = make_rsrc(tq, (size_t)M * 64), rts = make_rsrc(te, (size_t)M * 4);
            for (int c = w; c < L_BM / 16; c += NW) {
                const int row = c * 16 + qrow;
                const uint32_t v = (uint32_t)(m0 + row) * 64 + qcol * 16;   // rows past M read as zero
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, SERQ_LDS_PTR(tqs + c * 1024), 16, (int)v, 0, 0, 0);
            }
            if (w < 4)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rts, SERQ_LDS_PTR(tqs + L::TT + w * 256), 4,
                                                         (int)((uint32_t)(m0 + w * 64 + lane) * 4), 0, 0, 0);
        } else {
#pragma unroll
            for (int u = 0; u < L::QW / (1024 * NW); ++u) {
                const int row = (u * NW + w) * 16 + qrow;
                const uint32_t v = row < BN ? (uint32_t)(n0 + row) * 64 + qcol * 16 : kOut;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, SERQ_LDS_PTR(qr + (u * NW + w) * 1024), 16, (int)v, 0, 0,
                                                         0);
            }
        }
        if (w < 4) {
            const uint32_t v = w * 64 + lane < BN ? (uint32_t)(n0 + w * 64 + lane) * 16 : kOut;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsr, SERQ_LDS_PTR(qr + L::QW + w * 256), 4, (int)v, 0, 0, 0);
        }
    }
    dma(S0{}, st0, 0);
    dma(S1{}, st1, min(1, KT / 2 - 1));

    // Per-lane fragment offsets: blocks of 16 rows sit 2048 bytes (256 bytes
    // of E8M0) apart, a pair's second step 512 bytes after its first, and
    // rows 16 apart share the swizzle, so one base per region serves every
    // block through the instruction's offset field.  The empty asm keeps the
    // compiler from re-deriving each block's address.
    const uint32_t swz = (uint32_t)((i & 7) * 64 + ((g ^ ((i >> 1) & 3)) * 16));
    uint32_t oa = (uint32_t)((wm * (WR / 8) + (i >> 3)) * 1024) + swz;
    uint32_t ow = (uint32_t)(L::A + (wn * (WC / 8) + (i >> 3)) * 1024) + swz;
    uint32_t oq = (uint32_t)((wn * WC + i) * 64 + ((g ^ ((i >> 1) & 3)) * 16));
    uint32_t oga = (uint32_t)(L::GA + (wm * WR + i) * 16), ogw = (uint32_t)(L::GW + (wn * WC + i) * 16);
    uint32_t oqs = (uint32_t)(L::QW + (wn * WC + i) * 4 + g);
    __asm__ volatile("" : "+v"(oa), "+v"(ow), "+v"(oq), "+v"(oga), "+v"(ogw), "+v"(oqs));
    // byte g of each of a row's four E8M0 dwords (steps 0 .. 3), packed
    const uint32_t sel = (uint32_t)g | ((uint32_t)(g + 4) << 8) | 0x0c0c0000u;
    auto pack = [&](const u32x4 &d) {
        const uint32_t lo = __builtin_amdgcn_perm(d.y, d.x, sel), hi = __builtin_amdgcn_perm(d.w, d.z, sel);
        return (int)__builtin_amdgcn_perm(hi, lo, 0x05040100u);
    };

    struct Frag {
        u32x4 a[MB], b[NB];
    };
    struct Scales {
        int a[MB], b[NB];
    };
    struct RawScales {
        u32x4 a[MB], b[NB];
    };
    // fragments of the step in half h of a stage
    auto read = [&](const uint8_t *stg, int h, Frag &F) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) F.a[mb] = lds16(stg + oa + h * 512 + mb * 2048);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) F.b[nb] = lds16(stg + ow + h * 512 + nb * 2048);
    };
    auto read_scales = [&](RawScales &R) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) R.a[mb] = lds16(st0 + oga + mb * 256);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) R.b[nb] = lds16(st0 + ogw + nb * 256);
    };
    auto pack_scales = [&](const RawScales &R, Scales &S) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) S.a[mb] = pack(R.a[mb]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) S.b[nb] = pack(R.b[nb]);
    };
    v4f acc[NB][MB];
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
        for (int b = 0; b < MB; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};
    // step s (0 .. 3) of a four-step group: the scales' byte s
    auto step = [&](auto SI, const Frag &F, const Scales &S) {
        constexpr int s = decltype(SI)::value;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const v8i bf = v8i{(int)F.b[nb].x, (int)F.b[nb].y, (int)F.b[nb].z, (int)F.b[nb].w, 0, 0, 0, 0};
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const v8i af = v8i{(int)F.a[mb].x, (int)F.a[mb].y, (int)F.a[mb].z, (int)F.a[mb].w, 0, 0, 0, 0};
                acc[nb][mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af, acc[nb][mb], 4, 4, s, S.b[nb], s,
                                                                                S.a[mb]);
            }
        }
    };
    auto residual = [&](const Frag &F, const Scales &S) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const u32x4 p = lds16(qr + oq + nb * 1024);
            const int sr = qr[oqs + nb * 64];
            const v8i rf = v8i{(int)p.x, (int)p.y, (int)p.z, (int)p.w, 0, 0, 0, 0};
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const v8i af = v8i{(int)F.a[mb].x, (int)F.a[mb].y, (int)F.a[mb].z, (int)F.a[mb].w, 0, 0, 0, 0};
                acc[nb][mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(rf, af, acc[nb][mb], 4, 4, 0, sr, 0,
                                                                                S.a[mb]);
            }
        }
    };

    // TQ: the residual is Q(T) . L2 (the L2QER comparator), the Q(T) tile
    // from LDS against L2 in Q(R)'s place
    auto residual_tq = [&]() {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const u32x4 p = lds16(qr + oq + nb * 1024);
            const int sr = qr[oqs + nb * 64];
            const v8i rf = v8i{(int)p.x, (int)p.y, (int)p.z, (int)p.w, 0, 0, 0, 0};
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int row = wm * WR + mb * 16 + i;
                const u32x4 a = lds16(tqs + row * 64 + ((g ^ ((row >> 1) & 3)) * 16));
                const int sa = tqs[L::TT + row * 4 + g];
                const v8i af = v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
                acc[nb][mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(rf, af, acc[nb][mb], 4, 4, 0, sr, 0, sa);
            }
        }
    };

    // steps 0 and 1, their E8M0 group and Q(R) landed; steps 2 and 3 may
    // still be in flight
    Frag F0, F1;
    Scales Sc;
    RawScales Rn;
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(ND, 15));
    barrier();
    read(st0, 0, F0);
    read_scales(Rn);
    pack_scales(Rn, Sc);
    if constexpr (TQ) {
        if (has_r) residual_tq();
    } else {
        if (has_r) residual(F0, Sc);   // Q(R) against the first 128 input channels
    }

    // One step j (s = j % 4; stage 0 holds steps 4q, 4q + 1, stage 1 steps
    // 4q + 2, 4q + 3).  The fragments of step j are in registers; the reads of
    // step j + 1 go out ahead of step j's MFMAs.  Where step j + 1 lies in the
    // other stage (s = 1, 3) every wave first waits for that stage's copies
    // (vmcnt: none other is in flight) and for its own reads of the stage it
    // leaves (lgkmcnt), then, after the barrier, refills the stage it left
    // with the pair two ahead -- which has two steps of MFMAs to land.  At
    // s = 3 the reads also take the next E8M0 group (it came into stage 0 with
    // steps 4q + 4 and 4q + 5), packed after the MFMAs.  Past the last step the
    // copies re-read the last pair and the reads take a stale stage, unused.
    auto iter = [&](auto SI, int j) {
        constexpr int s = decltype(SI)::value;
        Frag &Fc = (s & 1) ? F1 : F0;
        Frag &Fn = (s & 1) ? F0 : F1;
        if constexpr (s == 1 || s == 3) {
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
            barrier();
            if constexpr (s == 1) dma(S0{}, st0, min(j / 2 + 2, KT / 2 - 1));
            else dma(S1{}, st1, min(j / 2 + 2, KT / 2 - 1));
        }
        if constexpr (s == 0) read(st0, 1, Fn);
        if constexpr (s == 1) read(st1, 0, Fn);
        if constexpr (s == 2) read(st1, 1, Fn);
        if constexpr (s == 3) read(st0, 0, Fn);
        if constexpr (s == 3) read_scales(Rn);
        step(SI, Fc, Sc);
        // the copies spread over the step's MFMAs, fragment reads one between
        // consecutive MFMAs from the first (with the copies bunched at the
        // start of the step: 142 vs 136 us on the LLaMA-3-8B gate|up)
        constexpr int nd = s == 1 ? ND + NG : s == 3 ? ND : 0, nr = (s == 3 ? 2 : 1) * (MB + NB);
        if constexpr (nd + nr <= MB * NB) sched_spread<0, MB * NB, nd, nr>();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (s == 3) pack_scales(Rn, Sc);
    };
    for (int j = 0; j < KT; j += 4) {
        iter(S0{}, j);
        iter(S1{}, j + 1);
        iter(S2{}, j + 2);
        iter(S3{}, j + 3);
    }

    // every copy (the clamped ones past the last step too) has landed and
    // every wave is done with the stages before they take Y
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    barrier();
    // Y rows of YP bytes (16 NB channels padded to a power of two), 16 token
    // rows per wave at a time, chunk q of row tl at q ^ tl
    constexpr int YP = NB <= 4 ? 256 : 512, QPR = YP / 16, RPI = 64 / QPR;
    uint8_t *const ybuf = st0 + w * (16 * YP);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int q = nb * 4 + g;
            *reinterpret_cast<v4f *>(ybuf + i * YP + ((q ^ i) * 16)) = acc[nb][mb];
        }
        if constexpr (SQ) {
            // SwiGLU into the next layer's MXFP4 input: the wave's WC columns
            // are WC / 2 (gate, up) pairs, H[j] = silu(g) u / s_next[j] for
            // its H channels jw .. jw + WC / 2 - 1 -- whole MX blocks.  Eight
            // lanes take one token's block, lane c its chunk of four H values
            // (eight Y columns), and encode it as the activation quantizer
            // does.
            constexpr int HB = WC / 64;                           // MX blocks of H per token row
            const int dn = N >> 1, jw = (n0 + wn * WC) >> 1;
#pragma unroll
            for (int it = 0; it < 2 * HB; ++it) {
                const int task = it * 64 + lane, bi = task >> 3, c = task & 7;
                const int tl = bi / HB, blk = bi % HB, q0 = blk * 16 + 2 * c;
                const float4 y0 = *reinterpret_cast<const float4 *>(ybuf + tl * YP + ((q0 ^ tl) * 16));
                const float4 y1 = *reinterpret_cast<const float4 *>(ybuf + tl * YP + (((q0 + 1) ^ tl) * 16));
                const int row = m0 + wm * WR + mb * 16 + tl, j = jw + blk * 32 + 4 * c;
                if (row < M && j < dn) {   // the same for the block's eight lanes
                    const float4 sn = *reinterpret_cast<const float4 *>(s_next + j);
                    float4 h;
                    h.x = ((y0.x / (1.0f + exp32(-y0.x))) * y0.y) / sn.x;
                    h.y = ((y0.z / (1.0f + exp32(-y0.z))) * y0.w) / sn.y;
                    h.z = ((y1.x / (1.0f + exp32(-y1.x))) * y1.y) / sn.z;
                    h.w = ((y1.z / (1.0f + exp32(-y1.z))) * y1.w) / sn.w;
                    mx_encode_chunk<false>(h, j >> 2, xqn + (size_t)row * (size_t)(dn >> 1),
                                           xen + (size_t)row * (size_t)(dn >> 5));
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < 16 / RPI; ++k) {
                const int tl = k * RPI + lane / QPR, q = lane % QPR;
                const float4 y = *reinterpret_cast<const float4 *>(ybuf + tl * YP + ((q ^ tl) * 16));
                const int row = m0 + wm * WR + mb * 16 + tl, col = n0 + wn * WC + q * 4;
                if (q < NB * 4 && row < M && col < N) store_y(Y + (size_t)row * (size_t)N + col, y);
            }
        }
    }
}

// ===========================================================================
// Wide MX W4A8 kernel with LDS-direct copies (r_pad <= 128, d_in % 512 == 0):
// the FP8-activation counterpart of k_gemm_mxd.  A step's activation rows
// are 128 bytes (whole L2 lines), its weight rows 64; two one-step stages
// (an FP8 step has twice the MFMA time of an FP4 one to cover a copy), the
// E8M0 bytes in groups of four steps with stage 0 as in k_gemm_mxd.  An FP8
// fragment is 32 bytes a lane, so the activation fragments of the next step
// are read block by block right after each block's last MFMA of this step
// (one set of them instead of two); the weight fragments are read for the
// next step ahead of this step's MFMAs.  128-byte activation rows keep the
// swizzle of k_gemm_mx8 (16-byte chunk c of row r at c ^ (r & 7)).
// ===========================================================================
template <int NB>
struct MxDma8 {
    static constexpr int BN = 32 * NB;
    static constexpr int WI = (BN * 64 + 4095) / 4096; // weight copies per thread and step
    static constexpr int A = L_BM * 128;               // activation rows: 256 x 128 bytes
    static constexpr int STAGE = A + WI * 4096;        // + weight rows: WI x 64 rows x 64 bytes
    static constexpr int GA = STAGE, GW = GA + 4096;   // stage 0 only: E8M0 of four steps, 256 x 16 bytes each
    static constexpr int STAGE0 = GW + 4096;
    static constexpr int QW = WI * 4096, QR = QW + 256 * 4;
    static constexpr int ND = 8 + WI;                  // LDS-direct loads per thread and step (+ 2 into stage 0)
};

template <int NB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_mxd8(
    const uint8_t *__restrict__ xq, const uint8_t *__restrict__ xe, int M,
    const uint8_t *__restrict__ wq, const uint8_t *__restrict__ we,
    const uint8_t *__restrict__ rq, const uint8_t *__restrict__ re,
    int N, int K, int r_pad, float *__restrict__ Y, int gm) {
    using L = MxDma8<NB>;
    constexpr int WR = 128, WC = NB * 16, MB = WR / 16, BN = L::BN, WI = L::WI, ND = L::ND;
    __shared__ __attribute__((aligned(16))) uint8_t st0[L::STAGE0], st1[L::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t qr[L::QR];
    const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int i = lane & 15, g = lane >> 4;
    const int wm = w >> 1, wn = w & 1;
    int tm, tn;
    tile_coords((M + L_BM - 1) / L_BM, (N + BN - 1) / BN, gm, tm, tn);
    const int m0 = tm * L_BM, n0 = tn * BN;
    const int KT = K >> 7;
    const uint32_t a_ld = (uint32_t)K, w_ld = (uint32_t)(K >> 1), s_ld = (uint32_t)(K >> 5);
    constexpr uint32_t kOut = 0x80000000u;                      // an offset past every buffer: reads zero

    // copy plan.  Activations: copy u of wave w moves rows (4 u + w) * 8 .. + 7
    // (128 bytes each); lane l takes slot l & 7 of row l >> 3, which holds
    // global chunk (l & 7) ^ (row & 7).  Weights: copy u fills rows u * 64 +
    // w * 16 .. + 15 (64 bytes each) -- one 16-row block, so one whole 1 KB
    // tile of the step; lane l takes slot l & 3 of row l >> 2, global chunk
    // (l & 3) ^ ((row >> 1) & 3).  E8M0: lane l of wave w the 16 bytes of row
    // w * 64 + l for four steps (activations: a row-major row piece; weights:
    // the row's 16 bytes in its block's 256-byte group).  Offsets past a
    // buffer's end read as zero.
    const int ar = lane >> 3, ac = (lane & 7) ^ (ar & 7);
    const int lr = lane >> 2, lc = (lane & 3) ^ ((lr >> 1) & 3);
    uint32_t va[8], vw[WI];
#pragma unroll
    for (int u = 0; u < 8; ++u) va[u] = (uint32_t)(m0 + (4 * u + w) * 8 + ar) * a_ld + ac * 16;
#pragma unroll
    for (int u = 0; u < WI; ++u) {
        const int row = u * 64 + w * 16 + lr;
        vw[u] = row < BN ? (uint32_t)((n0 + row) >> 4) * (uint32_t)KT * 1024 + lr % 16 * 64 + lc * 16 : kOut;
    }
    const uint32_t sn = (uint32_t)(n0 + w * 64 + lane), kg4 = (uint32_t)(KT / 4);
    const uint32_t vsa = (uint32_t)(m0 + w * 64 + lane) * s_ld;
    const uint32_t vsw = w * 64 + lane < BN ? ((sn >> 4) * kg4 * 16 + (sn & 15)) * 16 : kOut;
    const rsrc_t ra = make_rsrc(xq, (size_t)M * a_ld), rw = make_rsrc(wq, (size_t)N * w_ld);
    const rsrc_t rsa = make_rsrc(xe, (size_t)M * s_ld), rsw = make_rsrc(we, (size_t)N * kg4 * 16);

    // step kt into stage stg; with grp (kt % 4 == 0, but for the clamped
    // copies past the last step, which re-read the last group's bytes into
    // stage 0 after they are in registers) also the E8M0 bytes of steps kt ..
    // kt + 3, first
    auto dma = [&](uint8_t *stg, int kt, bool grp) {
        if (grp) {
            const int q = kt >> 2;   // the four-step group
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, SERQ_LDS_PTR(stg + L::GA + w * 1024), 16, (int)vsa, q * 16, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, SERQ_LDS_PTR(stg + L::GW + w * 1024), 16, (int)vsw, q * 256, 0,
                                                     0);
        }
        // the step's byte offsets within an activation row and within a block
        // of weight tiles (never decide a bound)
        const int ka = kt * 128, kw = kt * 1024;
#pragma unroll
        for (int u = 0; u < 8; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, SERQ_LDS_PTR(stg + (4 * u + w) * 1024), 16, (int)va[u], ka, 0, 0);
#pragma unroll
        for (int u = 0; u < WI; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, SERQ_LDS_PTR(stg + L::A + u * 4096 + w * 1024), 16, (int)vw[u], kw,
                                                     0, 0);
    };
    auto barrier = [&]() {
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;

    const bool has_r = r_pad > 0;
    if (has_r) {   // Q(R), one K step: 64-byte rows in channel order; its E8M0 bytes lead each 16-byte group
        const rsrc_t rr = make_rsrc(rq, (size_t)N * 64), rsr = make_rsrc(re, (size_t)N * 16);
#pragma unroll
        for (int u = 0; u < WI; ++u) {
            const int row = u * 64 + w * 16 + lr;
            const uint32_t v = row < BN ? (uint32_t)(n0 + row) * 64 + lc * 16 : kOut;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, SERQ_LDS_PTR(qr + u * 4096 + w * 1024), 16, (int)v, 0, 0, 0);
        }
        const uint32_t v = w * 64 + lane < BN ? (uint32_t)(n0 + w * 64 + lane) * 16 : kOut;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsr, SERQ_LDS_PTR(qr + L::QW + w * 256), 4, (int)v, 0, 0, 0);
    }
    dma(st0, 0, true);
    dma(st1, min(1, KT - 1), false);

    // per-lane fragment offsets (blocks of 16 rows: 2048 bytes of activation
    // rows, 1024 of weight rows, 256 of E8M0 groups)
    // (an FP8 fragment is 16-byte chunks g and g + 4 of the row's step, as
    // the MX FP8 activation layout places a lane group's 32-element block)
    uint32_t oal = (uint32_t)((wm * WR + i) * 128 + ((g ^ (i & 7)) * 16));
    uint32_t oah = (uint32_t)((wm * WR + i) * 128 + (((g + 4) ^ (i & 7)) * 16));
    uint32_t ow = (uint32_t)(L::A + (wn * WC + i) * 64 + ((g ^ ((i >> 1) & 3)) * 16));
    uint32_t oq = (uint32_t)((wn * WC + i) * 64 + ((g ^ ((i >> 1) & 3)) * 16));
    uint32_t oga = (uint32_t)(L::GA + (wm * WR + i) * 16), ogw = (uint32_t)(L::GW + (wn * WC + i) * 16);
    uint32_t oqs = (uint32_t)(L::QW + (wn * WC + i) * 4 + g);
    __asm__ volatile("" : "+v"(oal), "+v"(oah), "+v"(ow), "+v"(oq), "+v"(oga), "+v"(ogw), "+v"(oqs));
    const uint32_t sel = (uint32_t)g | ((uint32_t)(g + 4) << 8) | 0x0c0c0000u;
    auto pack = [&](const u32x4 &d) {
        const uint32_t lo = __builtin_amdgcn_perm(d.y, d.x, sel), hi = __builtin_amdgcn_perm(d.w, d.z, sel);
        return (int)__builtin_amdgcn_perm(hi, lo, 0x05040100u);
    };
    struct Scales {
        int a[MB], b[NB];
    };
    struct RawScales {
        u32x4 a[MB], b[NB];
    };
    auto read_a = [&](const uint8_t *stg, int mb) {
        const u32x4 lo = lds16(stg + oal + mb * 2048), hi = lds16(stg + oah + mb * 2048);
        return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
    auto read_scales = [&](RawScales &R) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) R.a[mb] = lds16(st0 + oga + mb * 256);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) R.b[nb] = lds16(st0 + ogw + nb * 256);
    };
    auto pack_scales = [&](const RawScales &R, Scales &S) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) S.a[mb] = pack(R.a[mb]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) S.b[nb] = pack(R.b[nb]);
    };
    v4f acc[NB][MB];
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
        for (int b = 0; b < MB; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};

    v8i A[MB];
    u32x4 W0[NB], W1[NB];
    Scales Sc;
    RawScales Rn;
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(ND, 15));   // step 0, its E8M0 group and Q(R)
    barrier();
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) A[mb] = read_a(st0, mb);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) W0[nb] = lds16(st0 + ow + nb * 1024);
    read_scales(Rn);
    pack_scales(Rn, Sc);
    if (has_r) {   // Q(R) against the first 128 input channels
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const u32x4 p = lds16(qr + oq + nb * 1024);
            const int sr = qr[oqs + nb * 64];
            const v8i rf = v8i{(int)p.x, (int)p.y, (int)p.z, (int)p.w, 0, 0, 0, 0};
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                acc[nb][mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(rf, A[mb], acc[nb][mb], 4, 0, 0, sr, 0,
                                                                                Sc.a[mb]);
        }
    }

    // One step j (s = j % 4, stage j % 2): every wave holds step j's
    // fragments (lgkmcnt) and step j + 1 has landed (vmcnt: nothing later is
    // in flight); after the barrier stage j % 2 takes step j + 2.  Then the
    // next step's weight fragments are read, and each activation block of the
    // next step right after its last MFMA of this one; at s = 3 the next E8M0
    // group (it came into stage 0 with step j + 1) is read too, packed after
    // the MFMAs.  Past the last step the copies re-read it and the reads take
    // a stale stage, unused.
    auto iter = [&](auto SI, int j) {
        constexpr int s = decltype(SI)::value;
        uint8_t *const cur = (s & 1) ? st1 : st0;
        const uint8_t *const nxt = (s & 1) ? st0 : st1;
        u32x4 *Wc = (s & 1) ? W1 : W0;
        u32x4 *Wn = (s & 1) ? W0 : W1;
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
        barrier();
        dma(cur, min(j + 2, KT - 1), s == 2);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) Wn[nb] = lds16(nxt + ow + nb * 1024);
        if constexpr (s == 3) read_scales(Rn);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const v8i bf = v8i{(int)Wc[nb].x, (int)Wc[nb].y, (int)Wc[nb].z, (int)Wc[nb].w, 0, 0, 0, 0};
                acc[nb][mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, A[mb], acc[nb][mb], 4, 0, s, Sc.b[nb],
                                                                                s, Sc.a[mb]);
            }
            A[mb] = read_a(nxt, mb);
        }
        {   // one copy or fragment read between consecutive MFMAs
            constexpr int nd = ND + (s == 2 ? 2 : 0), nr = NB + 2 * MB + (s == 3 ? MB + NB : 0);
#pragma unroll
            for (int k = 0; k < nd; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            }
#pragma unroll
            for (int k = 0; k < nr; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, MB * NB - nd - nr, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (s == 3) pack_scales(Rn, Sc);
    };
    for (int j = 0; j < KT; j += 4) {
        iter(S0{}, j);
        iter(S1{}, j + 1);
        iter(S2{}, j + 2);
        iter(S3{}, j + 3);
    }

    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    barrier();
    uint8_t *const ybuf = st0 + w * 8192;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int q = nb * 4 + g;
            *reinterpret_cast<v4f *>(ybuf + i * 512 + ((q ^ i) * 16)) = acc[nb][mb];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int tl = k * 2 + (lane >> 5), q = lane & 31;
            const float4 y = *reinterpret_cast<const float4 *>(ybuf + tl * 512 + ((q ^ tl) * 16));
            const int row = m0 + wm * WR + mb * 16 + tl, col = n0 + wn * WC + q * 4;
            if (q < NB * 4 && row < M && col < N) store_y(Y + (size_t)row * (size_t)N + col, y);
        }
    }
}

// ===========================================================================
// MX decode kernel (MXFP4 / MX W4A8 with M <= 16 tokens: bandwidth-bound).
// The schedule of the INT4 decode kernel below: a workgroup owns NB blocks
// of 16 output channels; the K steps of What_q (d_in / 128) followed by the
// r_pad / 128 steps of Q(R) form one sequence of T steps cut into KS
// contiguous ranges; the NW waves form NW / KS groups of KS, each group
// taking NB KS / NW of the blocks and each wave of it one range, which it
// streams through a ring of D register buffers (the loads of step v + D go
// out as soon as step v is consumed; positions past the range re-load its
// last step, so no load is conditional).  A step's operands go from HBM
// (weights: one 1 KB tile of 16 channels x 128 elements per block, a
// 16-byte piece per lane; their E8M0 words: 16 words of the block's 256-byte
// group) and L2 (activations, shared by the workgroup's blocks) straight into
// the scaled MFMA.  A lane holds token i and channels 4 g .. 4 g + 3 of a
// block.  MX keeps main and residual in one fp32 sum per block: the KS
// waves' partial sums meet in LDS and are added in wave order.  The step
// index is wave-uniform (the wave index goes through readfirstlane), so
// every test on it is a scalar branch: an MFMA under an EXEC mask would
// still write its accumulator.
// ===========================================================================
template <bool A8, int NB, int NW, int D, int KS, bool SL = true>
__global__ __launch_bounds__(64 * NW) void k_decode_mx(
    const uint8_t *__restrict__ xq, const uint8_t *__restrict__ xe, int M,
    const uint8_t *__restrict__ wq, const uint8_t *__restrict__ we,
    const uint8_t *__restrict__ rq, const uint8_t *__restrict__ re,
    int N, int K, int r_pad, float *__restrict__ Y) {
    static_assert(NW % KS == 0 && NB % (NW / KS) == 0, "wave split");
    constexpr int NBW = NB / (NW / KS);
    constexpr uint32_t kOut = 0x80000000u;                      // an offset past every buffer: reads zero
    const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int kw = w % KS, b0 = (w / KS) * NBW;                 // this wave's part of K and first block
    const int i = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * NB * 16;
    const int KT = K >> 7, RT = r_pad >> 7, T = KT + RT;
    const uint32_t KG = (uint32_t)((KT + 3) / 4), RG = (uint32_t)((RT + 3) / 4);   // E8M0 groups a row
    const int lo = (T * kw) / KS, hi = (T * (kw + 1)) / KS;
    const uint32_t s_ld = (uint32_t)(K >> 5), a_ld = (uint32_t)(A8 ? K : K >> 1);
    const rsrc_t rw = make_rsrc(wq, (size_t)N * (size_t)(K >> 1)), rsw = make_rsrc(we, (size_t)N * KG * 16);
    const rsrc_t ra = make_rsrc(xq, (size_t)M * a_ld), rsa = make_rsrc(xe, (size_t)M * s_ld);
    const rsrc_t rr = make_rsrc(rq, (size_t)N * (size_t)(r_pad > 0 ? r_pad >> 1 : 1));
    const rsrc_t rsr = make_rsrc(re, (size_t)N * (RG > 0 ? RG * 16 : 1));
    // per-lane offsets: the tiles and E8M0 groups of this wave's blocks (a
    // block past N re-reads the last one; its results are not stored), token
    // rows (tokens past M read as zero)
    uint32_t wro[NBW], wso[NBW], rro[NBW], rso[NBW];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
        const uint32_t blk = (uint32_t)min(n0 / 16 + b0 + nb, N / 16 - 1);
        wro[nb] = blk * (uint32_t)KT * 1024 + i * 64 + g * 16;
        rro[nb] = blk * (uint32_t)RT * 1024 + i * 64 + g * 16;
        wso[nb] = blk * KG * 256 + i * 16;
        rso[nb] = blk * RG * 256 + i * 16;
    }
    const uint32_t aro = i < M ? (uint32_t)i * a_ld : kOut, aso = i < M ? (uint32_t)i * s_ld : kOut;

    // SL: every E8M0 byte the workgroup uses -- its blocks' groups of What_q
    // and of Q(R) (each a contiguous run of NB groups rows) and the 16 token
    // rows of the activations' -- goes into LDS once, by LDS-direct copies of
    // 1 KB a wave instruction, so that a step reads its scale words from LDS
    // instead of from 16 separate rows of memory.  Bytes past a buffer (the
    // last workgroup's blocks past N, tokens past M) read as zero.
    extern __shared__ __attribute__((aligned(16))) uint8_t sl[];
    const uint32_t wsb = (uint32_t)NB * KG * 256, rsb = (uint32_t)NB * RG * 256, asb = 16 * s_ld;
    const uint32_t lw = 0, lr = (wsb + 1023) & ~1023u, la = lr + ((rsb + 1023) & ~1023u);
    if constexpr (SL) {
        const uint32_t gw0 = (uint32_t)(n0 / 16) * KG * 256, gr0 = (uint32_t)(n0 / 16) * RG * 256;
        for (uint32_t c = (uint32_t)w * 1024; c < wsb; c += 1024u * NW)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, SERQ_LDS_PTR(sl + lw + c), 16, (int)(gw0 + c + lane * 16), 0, 0, 0);
        for (uint32_t c = (uint32_t)w * 1024; c < rsb; c += 1024u * NW)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsr, SERQ_LDS_PTR(sl + lr + c), 16, (int)(gr0 + c + lane * 16), 0, 0, 0);
        for (uint32_t c = (uint32_t)w * 1024; c < asb; c += 1024u * NW)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, SERQ_LDS_PTR(sl + la + c), 16, (int)(c + lane * 16), 0, 0, 0);
    }

    v4f acc[NBW];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) acc[nb] = v4f{0.f, 0.f, 0.f, 0.f};

    u32x4 wf[D][NBW], xa[D], xb[D];
    uint32_t swv[D][NBW], sxv[D];
    const int len = hi - lo;
    const int rot = len > 0 ? (int)((blockIdx.x * 11u + (unsigned)w * 5u) % (unsigned)len) : 0;
    auto rotv = [&](int v) {   // v in [lo, hi) -> the step taken at that position
        int x = v - lo + rot;
        if (x >= len) x -= len;
        return lo + x;
    };
    auto issue = [&](int j, int v) {
        v = rotv(min(v, hi - 1));
        const bool res = v >= KT;
        const int k = res ? v - KT : v;                          // the K step of the activations
        const uint32_t gs = (uint32_t)(k >> 2) * 256 + (uint32_t)(k & 3) * 4;   // the step's word in its group
        // the same loads for a main and a residual step (only the buffer and
        // offsets differ), so that the waits for a slot stay partial
        const rsrc_t rb = res ? rr : rw, rbs = res ? rsr : rsw;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            wf[j][nb] = bld16(rb, (res ? rro[nb] : wro[nb]) + (uint32_t)k * 1024);
            if constexpr (!SL)
                swv[j][nb] = __builtin_amdgcn_raw_buffer_load_b32(rbs, (int)((res ? rso[nb] : wso[nb]) + gs), 0, 0);
        }
        if constexpr (A8) {   // chunks g and g + 4 of the token's 128-byte step row
            xa[j] = bld16(ra, aro + (uint32_t)k * 128 + g * 16);
            xb[j] = bld16(ra, aro + (uint32_t)k * 128 + (g + 4) * 16);
        } else {
            xa[j] = bld16(ra, aro + (uint32_t)k * 64 + g * 16);
        }
        if constexpr (!SL) sxv[j] = __builtin_amdgcn_raw_buffer_load_b32(rsa, (int)(aso + (uint32_t)k * 4), 0, 0);
    };
    // SL: the scale words of step v from LDS (blocks local to the workgroup)
    auto lds_scales = [&](int j, int v) {
        const bool res = v >= KT;
        const int k = res ? v - KT : v;
        const uint32_t gs = (uint32_t)(k >> 2) * 256 + (uint32_t)(k & 3) * 4 + i * 16;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
            swv[j][nb] = *reinterpret_cast<const uint32_t *>(sl + (res ? lr + (uint32_t)(b0 + nb) * RG * 256
                                                                       : lw + (uint32_t)(b0 + nb) * KG * 256) + gs);
        sxv[j] = *reinterpret_cast<const uint32_t *>(sl + la + (uint32_t)i * s_ld + (uint32_t)k * 4);
    };
    auto consume = [&](int j) {
        const v8i af = A8 ? v8i{(int)xa[j].x, (int)xa[j].y, (int)xa[j].z, (int)xa[j].w,
                                (int)xb[j].x, (int)xb[j].y, (int)xb[j].z, (int)xb[j].w}
                          : v8i{(int)xa[j].x, (int)xa[j].y, (int)xa[j].z, (int)xa[j].w, 0, 0, 0, 0};
        const int s_x = (int)((sxv[j] >> (8 * g)) & 255u);      // lane group g's block of the step
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            const v8i bf = v8i{(int)wf[j][nb].x, (int)wf[j][nb].y, (int)wf[j][nb].z, (int)wf[j][nb].w, 0, 0, 0, 0};
            const int s_w = (int)((swv[j][nb] >> (8 * g)) & 255u);
            acc[nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af, acc[nb], 4, A8 ? 0 : 4, 0, s_w, 0,
                                                                       s_x);
        }
    };
    if (lo < hi) {
#pragma unroll
        for (int j = 0; j < D; ++j) issue(j, lo + j);
    }
    if constexpr (SL) {
        // the scale copies, issued before the ring's first loads, have landed
        // in every wave (loads complete in order: at most the ring's loads
        // may still be in flight)
        constexpr int ring = D * (NBW + (A8 ? 2 : 1));
        if (lo < hi) __builtin_amdgcn_s_waitcnt(waitcnt_imm(ring, 15));
        else __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
        // a bare barrier: __syncthreads() would also wait for the ring's loads
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
    }
    if (lo < hi) {
        // steady state: D steps consumed and D issued a round, unconditionally
        // (so that a slot's wait leaves the later slots' loads in flight);
        // then the last rounds issue nothing past the range (re-reading its
        // last step there cost 11-13 % of the kernel at 8-9 steps a wave)
        int base = lo;
        for (; base + 2 * D <= hi; base += D) {
#pragma unroll
            for (int j = 0; j < D; ++j) {
                if constexpr (SL) lds_scales(j, rotv(base + j));
                consume(j);
                issue(j, base + j + D);
            }
        }
        for (; base < hi; base += D) {
#pragma unroll
            for (int j = 0; j < D; ++j) {
                if (base + j < hi) {
                    if constexpr (SL) lds_scales(j, rotv(base + j));
                    consume(j);
                }
                if (base + j + D < hi) issue(j, base + j + D);
            }
        }
    }
    // the KS waves' partial sums of each block, added in wave order
    __shared__ v4f red[KS][NB][64];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) red[kw][b0 + nb][lane] = acc[nb];
    __syncthreads();
    for (int idx = t; idx < NB * 64; idx += 64 * NW) {
        const int nb = idx >> 6, l = idx & 63;
        v4f y = red[0][nb][l];
#pragma unroll
        for (int ww = 1; ww < KS; ++ww) y += red[ww][nb][l];
        const int tok = l & 15, col = n0 + nb * 16 + 4 * (l >> 4);
        if (tok < M && col < N) *reinterpret_cast<v4f *>(Y + (size_t)tok * (size_t)N + col) = y;
    }
}

// ===========================================================================
// Decode INT4 / W4A8 kernel (M <= 16 tokens: bandwidth-bound).  A workgroup
// owns NB blocks of 16 output channels.  The K steps of What_q and the
// r_pad/128 steps of Q(R) are split over KS waves: as whole steps in KS
// contiguous ranges, or, where that leaves a longer critical path, as whole
// main steps and Q(R) half steps (see the kernel).  The NW waves form NW / KS
// groups of KS, each group taking NB KS / NW of the blocks and each wave of it
// one share of the steps; the waves' int32 partial sums meet in LDS.  (A
// rank-r sequence of 34 steps splits 17 / 17 two ways against 16 / 16 at
// rank 0 -- the ratio of the bytes -- and 8.5 each four ways with halves.)
// Each wave streams its share through a ring of D register buffers: the loads
// of step v + D (weights straight from HBM, one 1024-byte tile per block of
// 16 channels) are issued as soon as step v has been consumed, so D steps
// stay in flight (none past the end of the share).  Each wave starts its
// share at a step rotated by its workgroup and wave index (the int32 sums do
// not depend on the order), so that the waves of the grid do not all read the
// same offsets of their weight blocks at once.  The epilogue terms of the
// outputs a thread stores are loaded first and arrive while the weights
// stream.
// ===========================================================================
template <bool A8, int NB, int NW, int D, int KS>
__global__ __launch_bounds__(64 * NW) void k_decode_int(IntArgs args) {
    // KS waves split the step sequence of a block; the NW / KS groups of them
    // take NBW blocks each
    static_assert(NW % KS == 0 && NB % (NW / KS) == 0, "wave split");
    constexpr int NBW = NB / (NW / KS);
    const int M = args.M, N = args.N, K = args.K, r_pad = args.r_pad;
    __shared__ int red[KS][2][NB][4][64];
    // The wave index goes through readfirstlane so that the step range, and
    // every branch on it, is scalar: an MFMA placed under an EXEC mask still
    // writes its accumulator, so MFMAs must never sit behind a branch the
    // compiler may lower to lane masking.
    const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int kw = w % KS, b0 = (w / KS) * NBW;       // this wave's part of K and first block
    const int i = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * NB * 16;
    // The wave's work is a list of K steps: nm main steps from mlo on, nf
    // whole residual steps from flo on, then nh residual half steps (64 of a
    // step's 128 elements) from rlo on.  With whole steps the KT + RT steps
    // split evenly over the KS waves.  Where that leaves a longer critical
    // path than half steps do, the main steps go KT / KS to a wave (one more
    // to the last KT % KS waves) and the 2 RT halves fill the waves in order
    // up to Lu units each (a step two, a half one): a rank-256 down
    // projection (112 + 2 steps over 16 waves) so runs 7.5 steps on its
    // longest wave instead of 8.
    const int KT = K >> 7, RT = r_pad >> 7, H = 2 * RT, T = KT + RT;
    const int q = KT / KS, full = KS - KT % KS;
    const int Lu = (2 * KT + H + KS - 1) / KS;
    const bool halves = max(Lu, 2 * (q + (full < KS ? 1 : 0))) < 2 * ((T + KS - 1) / KS);
    int mlo, nm, flo = 0, nf = 0, rlo = 0, nh = 0;
    if (halves) {
        mlo = kw * q + max(0, kw - full);
        nm = q + (kw >= full ? 1 : 0);
        const int c0 = max(0, Lu - 2 * q), c1 = max(0, Lu - 2 * q - 2);
        rlo = min(H, min(kw, full) * c0 + max(0, kw - full) * c1);
        nh = min(H, min(kw + 1, full) * c0 + max(0, kw + 1 - full) * c1) - rlo;
    } else {
        const int lo = (T * kw) / KS, hi = (T * (kw + 1)) / KS;
        mlo = lo;
        nm = max(0, min(hi, KT) - lo);
        flo = max(lo, KT) - KT;
        nf = max(0, hi - max(lo, KT));
    }
    const bool live = i < M;
    constexpr int AB = A8 ? 2 : 1;   // 16-byte activation loads per step
    const uint8_t *a_row = args.xq + (size_t)min(i, M - 1) * (A8 ? (size_t)K : (size_t)(K >> 1)) + g * 16 * AB;
    // What_q / Q(R) tiles of 16 channels x 128 elements: lane (i, g) reads
    // bytes 16 g .. 16 g + 15 of channel i, the wave the whole 1024-byte tile.
    // In half step h of a Q(R) tile the lane's 8 bytes are 32 h + 8 g ..
    // 32 h + 8 g + 7 of its row (and of the activation row the bytes holding
    // the same elements); it loads the aligned 16 bytes around them, so that a
    // half step issues the loads of a main step into the same registers.
    const uint8_t *w_row[NBW], *r_row[NBW];
    const int wh = ((g >> 1) - g) * 16, ah = A8 ? -g * 16 : wh;   // half-step offsets from a lane's step piece
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
        const size_t blk = (size_t)min(n0 / 16 + b0 + nb, N / 16 - 1);
        w_row[nb] = args.wq + blk * (size_t)KT * 1024 + i * 64 + g * 16;
        r_row[nb] = args.rq + blk * (size_t)RT * 1024 + i * 64 + g * 16;
    }
    // all ones where the lane's half-step bytes are the upper 8 of the 16 it
    // loads (INT4 activations, weights)
    const uint32_t odd = (g & 1) ? ~0u : 0u;
    auto pick = [&](uint32_t lo, uint32_t hi) { return (hi & odd) | (lo & ~odd); };
    // outputs this thread stores after the reduction, and their terms
    constexpr int E = (NB * 256 + 64 * NW - 1) / (64 * NW);
    const int ev = (t >> 6) & 3, el = t & 63;   // the same for all E outputs, as NW % 4 == 0
    const int row = 4 * (el >> 4) + ev;
    IntRow rrow;
    IntCol rcol[E];
    rrow.load(args, A8, row);
#pragma unroll
    for (int e = 0; e < E; ++e) rcol[e].load(args, A8, n0 + ((t + e * 64 * NW) >> 8) * 16 + (el & 15));

    v4i accm[NBW], accr[NBW];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) accm[nb] = accr[nb] = v4i{0, 0, 0, 0};

    u32x4 wv[D][NBW], av[D][AB];
    // Position x of the ring takes item v = (x + rot) mod len of the list:
    // main step mlo + v (v < nm), residual step flo + v - nm (v < nm + nf),
    // else residual half rlo + v - nm - nf
    const int len = nm + nf + nh;
    const int rot = len > 0 ? (int)((blockIdx.x * 11u + (unsigned)w * 5u) % (unsigned)len) : 0;
    auto rotv = [&](int x) {
        x += rot;
        return x >= len ? x - len : x;
    };
    // Every slot takes the same loads (only their addresses depend on the
    // kind of step), so that the waits for a slot stay partial.
    auto issue = [&](int j, int x) {
        const int v = rotv(x);
        const bool ms = v < nm, hs = v >= nm + nf;
        const int hv = rlo + v - nm - nf;
        const size_t kt = (size_t)(ms ? mlo + v : hs ? hv >> 1 : flo + v - nm);
        const int hw = hs ? wh + (hv & 1) * 32 : 0, ha = hs ? ah + (hv & 1) * 32 * AB : 0;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) wv[j][nb] = gld16((ms ? w_row[nb] : r_row[nb]) + hw + kt * 1024);
#pragma unroll
        for (int u = 0; u < AB; ++u) av[j][u] = gld16(a_row + (hs ? ha : u * 16) + kt * 64 * AB);
    };
    // a whole step into acc (main or residual)
    auto step = [&](int j, v4i *acc) {
        v4i a0, a1;
        if constexpr (A8) {
            a0 = reorder16(av[j][0]);
            a1 = reorder16(av[j][1]);
        } else {
            split_hi_lo(av[j][0], a0, a1);
        }
        // token rows past M take zero operands; their results are not stored
        if (!live) a0 = a1 = v4i{0, 0, 0, 0};
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
            v4i b0, b1;
            if constexpr (A8) unpack32(wv[j][nb], b0, b1);
            else split_hi_lo(wv[j][nb], b1, b0);   // weight low nibbles pair with activation high ones
            acc[nb] = mfma_i8(a0, b0, acc[nb]);
            acc[nb] = mfma_i8(a1, b1, acc[nb]);
        }
    };
    auto consume = [&](int j, int x) {
        const int v = rotv(x);
        if (v < nm) {
            step(j, accm);
        } else if (v < nm + nf) {
            step(j, accr);
        } else {
            // a half step: one MFMA over the lane's 8 bytes (16 elements), in
            // the byte pairing of a whole step
            v4i a;
            if constexpr (A8) {
                a = reorder16(av[j][0]);
            } else {
                const uint32_t x0 = pick(av[j][0].x, av[j][0].z), x1 = pick(av[j][0].y, av[j][0].w);
                a = v4i{(int)(x0 & NIB_HI), (int)(x1 & NIB_HI), (int)(x0 & NIB_LO), (int)(x1 & NIB_LO)};
            }
            if (!live) a = v4i{0, 0, 0, 0};
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const uint32_t w0 = pick(wv[j][nb].x, wv[j][nb].z), w1 = pick(wv[j][nb].y, wv[j][nb].w);
                v4i b;
                if constexpr (A8) b = v4i{nib_lo(w0), nib_hi(w0), nib_lo(w1), nib_hi(w1)};
                else b = v4i{(int)(w0 & NIB_LO), (int)(w1 & NIB_LO), (int)(w0 & NIB_HI), (int)(w1 & NIB_HI)};
                accr[nb] = mfma_i8(a, b, accr[nb]);
            }
        }
    };
    if (len > 0) {
        // the first D loads unconditional (a list shorter than D re-loads its
        // last item, never consumed): with every slot loaded on entry the
        // compiler's waits in the loop stay partial
#pragma unroll
        for (int j = 0; j < D; ++j) issue(j, min(j, len - 1));
        // steady state: D items consumed and D issued a round, unconditionally
        // (so that a slot's wait leaves the later slots' loads in flight);
        // then the last rounds issue nothing past the list
        int base = 0;
        for (; base + 2 * D <= len; base += D) {
#pragma unroll
            for (int j = 0; j < D; ++j) {
                consume(j, base + j);
                issue(j, base + j + D);
            }
        }
        for (; base < len; base += D) {
#pragma unroll
            for (int j = 0; j < D; ++j) {
                if (base + j < len) consume(j, base + j);
                if (base + j + D < len) issue(j, base + j + D);
            }
        }
    }
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            red[kw][0][b0 + nb][v][lane] = accm[nb][v];
            red[kw][1][b0 + nb][v][lane] = accr[nb][v];
        }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int idx = t + e * 64 * NW;
        if (idx >= NB * 256) break;
        const int nb = idx >> 8;
        int sm = 0, sr = 0;
#pragma unroll
        for (int ww = 0; ww < KS; ++ww) {
            sm += red[ww][0][nb][ev][el];
            sr += red[ww][1][nb][ev][el];
        }
        const int col = n0 + nb * 16 + (el & 15);
        if (row < M && col < N) int_store<A8>(args, row, col, sm, sr, rrow, rcol[e]);
    }
}

// ===========================================================================
// Host-side launch helpers
// ===========================================================================

serq_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return SERQ_OK;
    return fail(SERQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Compute units of the current device (cached per device).
int cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Fewer tokens than compute units: each token's workgroup has a compute unit
// to itself, so it takes 1024 threads and every thread a quarter of the work.
bool few_tokens(int32_t M) { return M < cu_count(); }

template <int Q, bool BF16, int NT>
void launch_quant_int_nt(const void *X, int32_t M, int32_t d_in, uint8_t *xq, float *sx, int *xsum, hipStream_t st) {
    constexpr int MAXCH = qa_maxch<NT>();
    const dim3 grid((unsigned)M), block(NT);
    const int ch = (d_in / 4 + NT - 1) / NT;   // register chunks the row needs
    if (ch <= 1) hipLaunchKernelGGL((k_quant_int<Q, BF16, 1, NT>), grid, block, 0, st, X, d_in, xq, sx, xsum);
    else if (ch <= 2) hipLaunchKernelGGL((k_quant_int<Q, BF16, 2, NT>), grid, block, 0, st, X, d_in, xq, sx, xsum);
    else if constexpr (MAXCH <= 4)
        hipLaunchKernelGGL((k_quant_int<Q, BF16, 4, NT>), grid, block, 0, st, X, d_in, xq, sx, xsum);
    else if (ch <= 4) hipLaunchKernelGGL((k_quant_int<Q, BF16, 4, NT>), grid, block, 0, st, X, d_in, xq, sx, xsum);
    else if (ch <= 8) hipLaunchKernelGGL((k_quant_int<Q, BF16, 8, NT>), grid, block, 0, st, X, d_in, xq, sx, xsum);
    else hipLaunchKernelGGL((k_quant_int<Q, BF16, MAXCH, NT>), grid, block, 0, st, X, d_in, xq, sx, xsum);
}

template <int Q, bool BF16>
void launch_quant_int(const void *X, int32_t M, int32_t d_in, uint8_t *xq, float *sx, int *xsum, hipStream_t st) {
    if (few_tokens(M)) launch_quant_int_nt<Q, BF16, QA_THREADS_FEW>(X, M, d_in, xq, sx, xsum, st);
    else launch_quant_int_nt<Q, BF16, QA_THREADS>(X, M, d_in, xq, sx, xsum, st);
}

template <bool FP8, int NT>
void launch_quant_mx_nt(const void *X, bool bf, int32_t M, int32_t d_in, uint8_t *xq, uint8_t *xe, hipStream_t st) {
    const dim3 grid((unsigned)M), block(NT);
    if (bf) hipLaunchKernelGGL((k_quant_mx<true, FP8, NT>), grid, block, 0, st, X, d_in, xq, xe);
    else hipLaunchKernelGGL((k_quant_mx<false, FP8, NT>), grid, block, 0, st, X, d_in, xq, xe);
}

serq_status launch_quant(const void *X, int32_t xdt, int32_t M, int32_t d_in, int32_t fmt,
                         uint8_t *xq, void *xscale, hipStream_t st) {
    const bool bf = xdt == SERQ_DT_BF16;
    float *sx = (float *)xscale;
    int *xsum = (int *)((uint8_t *)xscale + sizeof(float) * (size_t)M);   // INT4 only
    if (fmt == SERQ_FMT_INT4) {
        if (bf) launch_quant_int<7, true>(X, M, d_in, xq, sx, xsum, st);
        else launch_quant_int<7, false>(X, M, d_in, xq, sx, xsum, st);
    } else if (fmt == SERQ_FMT_W4A8) {
        if (bf) launch_quant_int<127, true>(X, M, d_in, xq, sx, nullptr, st);
        else launch_quant_int<127, false>(X, M, d_in, xq, sx, nullptr, st);
    } else {
        uint8_t *xe = (uint8_t *)xscale;
        const bool few = few_tokens(M);
        if (fmt == SERQ_FMT_MXFP4) {
            if (few) launch_quant_mx_nt<false, QA_THREADS_FEW>(X, bf, M, d_in, xq, xe, st);
            else launch_quant_mx_nt<false, QA_THREADS>(X, bf, M, d_in, xq, xe, st);
        } else {
            if (few) launch_quant_mx_nt<true, QA_THREADS_FEW>(X, bf, M, d_in, xq, xe, st);
            else launch_quant_mx_nt<true, QA_THREADS>(X, bf, M, d_in, xq, xe, st);
        }
    }
    return hip_status(hipGetLastError(), "quant_act launch");
}

// Producer kernels: one workgroup per token, the producer's row (d fp32) in
// dynamic LDS.  Q = 7 / 127 / 0 / 1 selects INT4 / W4A8 / MXFP4 / MX W4A8.
struct ProducerArgs {
    int mode;                  // 0 RMSNorm, 1 SwiGLU
    const void *in;
    int M, d;
    const float *gamma;
    float eps;
    const int32_t *perm;
    const float *s;
    uint8_t *xq;
    void *xscale;
};

template <int Q, bool BF16, int CH, int NT>
hipError_t launch_producer_ch(const ProducerArgs &a, hipStream_t st) {
    const size_t lds = sizeof(float) * (size_t)a.d;
    static hipError_t attr[2] = {
        hipFuncSetAttribute(reinterpret_cast<const void *>(&k_rmsnorm_quant<Q, BF16, CH, NT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)(sizeof(float) * kQuantMaxInReg)),
        hipFuncSetAttribute(reinterpret_cast<const void *>(&k_swiglu_quant<Q, BF16, CH, NT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)(sizeof(float) * kQuantMaxInReg))};
    const dim3 grid((unsigned)a.M), block(NT);
    if (a.mode == 1 && a.perm == nullptr) {   // permutation folded into the producer: no LDS row
        hipLaunchKernelGGL((k_swiglu_quant_folded<Q, BF16, CH, NT>), grid, block, 0, st, a.in, a.M, a.d, a.s, a.xq,
                           a.xscale);
        return hipGetLastError();
    }
    if (attr[a.mode] != hipSuccess) return attr[a.mode];
    if (a.mode == 0)
        hipLaunchKernelGGL((k_rmsnorm_quant<Q, BF16, CH, NT>), grid, block, lds, st, a.in, a.M, a.d, a.gamma, a.eps,
                           a.perm, a.s, a.xq, a.xscale);
    else
        hipLaunchKernelGGL((k_swiglu_quant<Q, BF16, CH, NT>), grid, block, lds, st, a.in, a.M, a.d, a.perm, a.s,
                           a.xq, a.xscale);
    return hipGetLastError();
}

template <int Q, bool BF16, int NT>
hipError_t launch_producer_nt(const ProducerArgs &a, hipStream_t st) {
    constexpr int MAXCH = qa_maxch<NT>();
    if constexpr (Q == 0 || Q == 1) {
        return launch_producer_ch<Q, BF16, 1, NT>(a, st);
    } else {
        const int ch = (a.d / 4 + NT - 1) / NT;   // register chunks the row needs
        if (ch <= 1) return launch_producer_ch<Q, BF16, 1, NT>(a, st);
        if (ch <= 2) return launch_producer_ch<Q, BF16, 2, NT>(a, st);
        if constexpr (MAXCH <= 4) {
            return launch_producer_ch<Q, BF16, 4, NT>(a, st);
        } else {
            if (ch <= 4) return launch_producer_ch<Q, BF16, 4, NT>(a, st);
            if (ch <= 8) return launch_producer_ch<Q, BF16, 8, NT>(a, st);
            return launch_producer_ch<Q, BF16, MAXCH, NT>(a, st);
        }
    }
}

template <int Q, bool BF16>
hipError_t launch_producer_q(const ProducerArgs &a, hipStream_t st) {
    if (few_tokens(a.M)) return launch_producer_nt<Q, BF16, QA_THREADS_FEW>(a, st);
    return launch_producer_nt<Q, BF16, QA_THREADS>(a, st);
}

serq_status launch_producer(const ProducerArgs &a, int32_t xdt, int32_t fmt, hipStream_t st) {
    const bool bf = xdt == SERQ_DT_BF16;
    hipError_t e;
    if (fmt == SERQ_FMT_INT4) e = bf ? launch_producer_q<7, true>(a, st) : launch_producer_q<7, false>(a, st);
    else if (fmt == SERQ_FMT_W4A8) e = bf ? launch_producer_q<127, true>(a, st) : launch_producer_q<127, false>(a, st);
    else if (fmt == SERQ_FMT_MXFP4) e = bf ? launch_producer_q<0, true>(a, st) : launch_producer_q<0, false>(a, st);
    else e = bf ? launch_producer_q<1, true>(a, st) : launch_producer_q<1, false>(a, st);
    return hip_status(e, a.mode == 0 ? "rmsnorm_quant launch" : "swiglu_quant launch");
}

template <bool A8, int NB, int NW, int D, int KS = NW>
void launch_decode(const IntArgs &a, hipStream_t st) {
    static_assert(NW % 4 == 0, "epilogue thread mapping");
    const int cols = NB * 16;
    const dim3 grid((unsigned)((a.N + cols - 1) / cols)), block(64 * NW);
    hipLaunchKernelGGL((k_decode_int<A8, NB, NW, D, KS>), grid, block, 0, st, a);
}

// Dynamic LDS of the large-tile kernel: two stages (activation + weight
// tiles of one 256-element K step), the kept activation tile and Q(R).
constexpr size_t kBigLds = 2 * (L_BM * 128 + L_BN * 128) + L_BM * 128 + L_BN * 128 + 16 * (L_BM + L_BN);

// Token tiles per group in the large-tile tile order: the group size whose
// window of 32 concurrent tiles (one XCD's CUs) touches the fewest activation
// and weight bytes.
int pick_gm(int M, int N) {
    const int tiles_m = (M + L_BM - 1) / L_BM, tiles_n = (N + L_BN - 1) / L_BN;
    const int window = min(32, tiles_m * tiles_n);
    int best = tiles_m, best_cost = 1 << 30;
    for (int gm = 1; gm <= tiles_m; gm *= 2) {
        const int rows = min(gm, window), cols = min(tiles_n, (window + rows - 1) / rows);
        const int cost = rows * L_BM + cols * L_BN;
        if (cost < best_cost) best = gm, best_cost = cost;
    }
    if (tiles_m < best) best = tiles_m;
    return best;
}

// Wave grid of the large-tile kernel: 4 x 2 waves (2 per SIMD), 64 x 64 each.
constexpr int L_WGM = 4, L_WGN = 2;
constexpr bool kIntPipelined = true;

serq_status launch_big(const IntArgs &a, hipStream_t st) {
    auto kern = &k_gemm_int_big<L_WGM, L_WGN, kIntPipelined>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kBigLds);
    if (attr != hipSuccess) return hip_status(attr, "gemm_int_big LDS attribute");
    const unsigned tiles = (unsigned)(((a.M + L_BM - 1) / L_BM) * ((a.N + L_BN - 1) / L_BN));
    IntArgs b = a;
    b.direct_y = tiles <= (unsigned)cu_count();   // one round of tiles: every epilogue exposed
    hipLaunchKernelGGL(kern, dim3(tiles), dim3(64 * L_WGM * L_WGN), kBigLds, st, b);
    return hip_status(hipGetLastError(), "gemm_int_big launch");
}

// Channel blocks per wave of the wide LDS-direct MX kernels: of the tile
// widths 32 * 8, 32 * 7 and 32 * 6 (up to 32 * max_nb), the one with the
// least work in whole rounds of workgroups (rounds of one workgroup per CU,
// times the tile width), ties to the wider.
int mx_wide_nb(int M, int N, int max_nb = 8) {
    const int cus = cu_count(), mt = (M + L_BM - 1) / L_BM;
    int best = max_nb;
    long best_cost = -1;
    for (int nb = max_nb; nb >= 6; --nb) {
        const int bn = 32 * nb;
        const long tiles = (long)mt * ((N + bn - 1) / bn);
        const long cost = (tiles + cus - 1) / cus * bn;
        if (best_cost < 0 || cost < best_cost) {
            best = nb;
            best_cost = cost;
        }
    }
    return best;
}

// the LDS-direct form of the wide MXFP4 kernel (r_pad <= 128, d_in % 512 == 0; static LDS)
template <int NB, int NW = 4>
serq_status launch_mx_dma_nb(const uint8_t *xq, const uint8_t *xe, int M, const uint8_t *wq, const uint8_t *we,
                             const uint8_t *rq, const uint8_t *re, int N, int K, int rp, float *Y, hipStream_t st) {
    const int bn = 32 * NB;
    const unsigned tiles = (unsigned)(((M + L_BM - 1) / L_BM) * ((N + bn - 1) / bn));
    hipLaunchKernelGGL((k_gemm_mxd<NB, NW>), dim3(tiles), dim3(64 * NW), 0, st, xq, xe, M, wq, we, rq, re, N, K, rp, Y,
                       pick_gm(M, N));
    return hip_status(hipGetLastError(), "gemm_mx wide (LDS-direct) launch");
}

// the LDS-direct form of the wide MX W4A8 kernel (r_pad <= 128, d_in % 512 == 0; static LDS)
template <int NB>
serq_status launch_mx_dma8_nb(const uint8_t *xq, const uint8_t *xe, int M, const uint8_t *wq, const uint8_t *we,
                              const uint8_t *rq, const uint8_t *re, int N, int K, int rp, float *Y, hipStream_t st) {
    const int bn = 32 * NB;
    const unsigned tiles = (unsigned)(((M + L_BM - 1) / L_BM) * ((N + bn - 1) / bn));
    hipLaunchKernelGGL((k_gemm_mxd8<NB>), dim3(tiles), dim3(256), 0, st, xq, xe, M, wq, we, rq, re, N, K, rp, Y,
                       pick_gm(M, N));
    return hip_status(hipGetLastError(), "gemm_mx8 wide (LDS-direct) launch");
}

// LDS bytes of the MX decode kernel's scale copies (NB blocks).
size_t decode_mx_lds(int NB, int K, int rp) {
    const size_t KT = (size_t)K / 128, RT = (size_t)rp / 128;
    auto kb = [](size_t b) { return (b + 1023) & ~(size_t)1023; };
    return kb(NB * ((KT + 3) / 4) * 256) + kb(NB * ((RT + 3) / 4) * 256) + kb(16 * (size_t)K / 32);
}

template <bool A8, int NB, int NW, int D, int KS>
serq_status launch_decode_mx_cfg(const uint8_t *xq, const uint8_t *xe, int M, const uint8_t *wq, const uint8_t *we,
                                 const uint8_t *rq, const uint8_t *re, int N, int K, int rp, float *Y, hipStream_t st) {
    const dim3 grid((unsigned)((N / 16 + NB - 1) / NB)), block(64 * NW);
    const size_t lds = decode_mx_lds(NB, K, rp);
    if (lds <= 64 * 1024)   // scales staged in LDS (every layer shape here)
        hipLaunchKernelGGL((k_decode_mx<A8, NB, NW, D, KS, true>), grid, block, lds, st, xq, xe, M, wq, we, rq, re, N,
                           K, rp, Y);
    else
        hipLaunchKernelGGL((k_decode_mx<A8, NB, NW, D, KS, false>), grid, block, 0, st, xq, xe, M, wq, we, rq, re, N,
                           K, rp, Y);
    return hip_status(hipGetLastError(), "decode_mx launch");
}

// MX decode (M <= 16): wide layers 4 blocks per workgroup, two steps in
// flight, MXFP4 with the waves in two pairs that each split K for two of
// the blocks (a rank-r sequence of 34 steps splits 17 / 17 against 16 / 16
// at rank 0, the ratio of the bytes; four ways it would be 9 / 8 / 9 / 8 --
// the two ran equally fast), MX W4A8, whose activation loads are twice as
// large, with all four waves on K for all four blocks (faster there);
// narrow layers one block and twelve waves on K, one step in flight, so that
// the grid still covers the CUs (a rank-256 down projection, 114 steps,
// splits 10 / 9 against 10 / 9 at rank 0; MXFP4 7.3 against 7.8 us with
// eight waves and 7.5 with sixteen)
template <bool A8>
serq_status launch_decode_mx(const uint8_t *xq, const uint8_t *xe, int M, const uint8_t *wq, const uint8_t *we,
                             const uint8_t *rq, const uint8_t *re, int N, int K, int rp, float *Y, hipStream_t st) {
    if (N / 64 >= cu_count()) {
        if constexpr (A8) return launch_decode_mx_cfg<A8, 4, 4, 2, 4>(xq, xe, M, wq, we, rq, re, N, K, rp, Y, st);
        else return launch_decode_mx_cfg<A8, 4, 4, 2, 2>(xq, xe, M, wq, we, rq, re, N, K, rp, Y, st);
    }
    return launch_decode_mx_cfg<A8, 1, 12, 1, 12>(xq, xe, M, wq, we, rq, re, N, K, rp, Y, st);
}

// The wide LDS-direct MX kernel (A8: FP8 activations, whose 256-channel
// form needs more registers than it has: widths 224 and 192 only).
template <bool A8>
serq_status launch_mx_wide(const uint8_t *xq, const uint8_t *xe, int M, const uint8_t *wq, const uint8_t *we,
                           const uint8_t *rq, const uint8_t *re, int N, int K, int rp, float *Y, hipStream_t st) {
    switch (mx_wide_nb(M, N, A8 ? 7 : 8)) {
    case 6: return A8 ? launch_mx_dma8_nb<6>(xq, xe, M, wq, we, rq, re, N, K, rp, Y, st)
                      : launch_mx_dma_nb<6>(xq, xe, M, wq, we, rq, re, N, K, rp, Y, st);
    case 7: return A8 ? launch_mx_dma8_nb<7>(xq, xe, M, wq, we, rq, re, N, K, rp, Y, st)
                      : launch_mx_dma_nb<7>(xq, xe, M, wq, we, rq, re, N, K, rp, Y, st);
    default: return launch_mx_dma_nb<8>(xq, xe, M, wq, we, rq, re, N, K, rp, Y, st);
    }
}

// The wide kernel (widths up to 32 max_nb) when its whole rounds of
// workgroups (one per CU) carry no more channels than those of the
// 128-channel tiles -- per channel the two run at about the same rate, so the
// rounds decide.
bool mx_wide_fits(int M, int N, int max_nb) {
    const long cus = cu_count(), mt = (M + L_BM - 1) / L_BM, bn = 32 * mx_wide_nb(M, N, max_nb);
    const long wide = (mt * ((N + bn - 1) / bn) + cus - 1) / cus * bn;
    const long narrow = (mt * ((N + L_BN - 1) / L_BN) + cus - 1) / cus * L_BN;
    return wide <= narrow;
}

// Shapes the LDS-direct MX kernels take: d_in a multiple of four K steps,
// Q(R) within one K step, more tokens than the decode kernel takes.
bool mx_lds_direct(int M, int K, int rp) { return M > 16 && K % 512 == 0 && rp <= 128; }

// Largest buffer (bytes) the buffer-resource kernels address: their byte
// offsets are 32-bit, rows past the end (up to a tile more) must not wrap, and
// the offset 2^31 that their out-of-range lanes use must lie past every buffer.
constexpr uint64_t kBufLimit = 1ull << 31;

serq_status launch_mx8(const uint8_t *xq, const uint8_t *xe, int M, const uint8_t *wq, const uint8_t *we,
                       const uint8_t *rq, const uint8_t *re, int N, int K, int rp, float *Y, hipStream_t st) {
    if ((size_t)N * (size_t)K >= kBufLimit || (size_t)M * (size_t)K >= kBufLimit)
        return fail(SERQ_ERR_UNSUPPORTED, "MX W4A8 buffers must stay below 2 GiB (32-bit offsets)");
    if (M <= 16) return launch_decode_mx<true>(xq, xe, M, wq, we, rq, re, N, K, rp, Y, st);
    if (mx_lds_direct(M, K, rp)) {
        if (mx_wide_fits(M, N, 7)) return launch_mx_wide<true>(xq, xe, M, wq, we, rq, re, N, K, rp, Y, st);
        return launch_mx_dma8_nb<4>(xq, xe, M, wq, we, rq, re, N, K, rp, Y, st);   // 256 x 128 tiles
    }
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_gemm_mx8),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMx8Lds);
    if (attr != hipSuccess) return hip_status(attr, "gemm_mx8 LDS attribute");
    const unsigned tiles = (unsigned)(((M + L_BM - 1) / L_BM) * ((N + L_BN - 1) / L_BN));
    hipLaunchKernelGGL(k_gemm_mx8, dim3(tiles), dim3(256), kMx8Lds, st, xq, xe, M, wq, we, rq, re, N, K, rp, Y,
                       pick_gm(M, N));
    return hip_status(hipGetLastError(), "gemm_mx8 launch");
}

// Tokens up to which the bandwidth-bound decode kernel is used.
constexpr int kDecodeMaxM = 16;

serq_status launch_linear(const serq_layout *L, const uint8_t *xq, const void *xscale, int32_t M,
                          const uint8_t *wq, const void *wscale, const uint8_t *rq, const void *rscale,
                          float *Y, int32_t *am, int32_t *ar, hipStream_t st) {
    const int N = L->d_out, K = L->d_in, rp = L->r_pad;
    if (rp == 0) {
        // no residual steps run; keep the (never dereferenced) R pointer valid
        rq = wq;
        if (!rscale) rscale = wscale;
    }
    if (L->fmt == SERQ_FMT_MXW4A8)
        return launch_mx8(xq, (const uint8_t *)xscale, M, wq, (const uint8_t *)wscale, rq, (const uint8_t *)rscale, N, K,
                          rp, Y, st);
    if (L->fmt == SERQ_FMT_MXFP4) {
        const uint8_t *xe = (const uint8_t *)xscale, *we = (const uint8_t *)wscale, *re = (const uint8_t *)rscale;
        if (M <= 16 && (size_t)N * (size_t)(K / 2) < kBufLimit)
            return launch_decode_mx<false>(xq, xe, M, wq, we, rq, re, N, K, rp, Y, st);
        const bool small_bufs = L->wq_bytes < kBufLimit && (size_t)M * (size_t)(K / 2) < kBufLimit;
        if (small_bufs && mx_lds_direct(M, K, rp)) {
            if (mx_wide_fits(M, N, 8)) return launch_mx_wide<false>(xq, xe, M, wq, we, rq, re, N, K, rp, Y, st);
            if (M > G_BM) return launch_mx_dma_nb<4, 8>(xq, xe, M, wq, we, rq, re, N, K, rp, Y, st);   // 256 x 128, 8 waves
        }
        const dim3 grid((unsigned)((N + G_BN - 1) / G_BN), (unsigned)((M + G_BM - 1) / G_BM));
        hipLaunchKernelGGL(k_gemm_mx, grid, dim3(G_THREADS), 0, st, xq, xe, M, wq, we, rq, re, N, K, rp, Y);
        return hip_status(hipGetLastError(), "gemm_mx launch");
    }
    const bool a8 = L->fmt == SERQ_FMT_W4A8;
    IntArgs a;
    a.xq = xq;
    a.sx = (const float *)xscale;
    a.xsum = a8 ? nullptr : (const int *)((const uint8_t *)xscale + sizeof(float) * (size_t)M);
    a.wq = wq;
    a.sw = (const float *)wscale;
    a.wsum = a8 ? nullptr : (const int *)((const uint8_t *)wscale + sizeof(float) * (size_t)N);
    a.rq = rq;
    a.sR = (const float *)rscale;
    a.rsum = a8 ? nullptr : (const int *)((const uint8_t *)rscale + sizeof(float) * (size_t)N);
    a.Y = Y;
    a.acc_main = am;
    a.acc_res = ar;
    a.M = M;
    a.N = N;
    a.K = K;
    a.r_pad = rp;
    a.gm = pick_gm(M, N);
    if (M <= kDecodeMaxM) {
        // wide layers: 4 column blocks per workgroup (INT4: two pairs of
        // waves, each pair splitting K for 2 blocks, two steps in flight;
        // W4A8, whose activation loads are twice as large, 8 waves on K for
        // all 4 blocks, one step in flight: 14.5 against 15.5 us with 4
        // waves and two steps on the 16-token gate|up); narrow ones: 1 block
        // and 16 waves on K (one step in flight each) so that the grid still
        // covers every CU
        const bool wide = N / 64 >= 256;
        if (a8) {
            if (wide) launch_decode<true, 4, 8, 1, 8>(a, st);
            else launch_decode<true, 1, 16, 1>(a, st);
        } else {
            if (wide) launch_decode<false, 4, 4, 2, 2>(a, st);
            else launch_decode<false, 1, 16, 1>(a, st);
        }
        return hip_status(hipGetLastError(), "decode launch");
    }
    // INT4 with M > 128, K a multiple of 256 and r_pad <= 256: large tiles
    // (its byte offsets are 32-bit: weight and activation buffers below 2 GiB)
    const bool small_bufs = L->wq_bytes < kBufLimit && (size_t)M * (size_t)(K / 2) < kBufLimit;
    if (!a8 && M > G_BM && K % 256 == 0 && rp <= 256 && small_bufs) return launch_big(a, st);
    const dim3 grid((unsigned)((N + G_BN - 1) / G_BN), (unsigned)((M + G_BM - 1) / G_BM));
    if (a8) hipLaunchKernelGGL((k_gemm_int<true>), grid, dim3(G_THREADS), 0, st, a);
    else hipLaunchKernelGGL((k_gemm_int<false>), grid, dim3(G_THREADS), 0, st, a);
    return hip_status(hipGetLastError(), "gemm_int launch");
}

// ---------------------------------------------------------------------------
// L2QER comparator plumbing.  k columns of the intermediate, padded to
// k_pad = round_up(k, 128): INT4 layers k <= 256, MXFP4 layers k a multiple
// of 32 up to 128 (one K step of the output GEMM's residual).
// ---------------------------------------------------------------------------
int l2qer_kpad(int k) { return (k + 127) / 128 * 128; }

serq_status check_l2qer(const serq_layout *L, int32_t k) {
    serq_status st = check_layout(L);
    if (st) return st;
    if (L->fmt == SERQ_FMT_MXFP4) {
        if (k < 32 || k > L2X_KP || k % 32)
            return fail(SERQ_ERR_SHAPE, "MXFP4: k=%d must be a multiple of 32 in [32, %d]", k, L2X_KP);
        return SERQ_OK;
    }
    if (L->fmt != SERQ_FMT_INT4)
        return fail(SERQ_ERR_UNSUPPORTED, "the L2QER comparator is built for INT4 and MXFP4 layers");
    if (k < 1 || k > 256) return fail(SERQ_ERR_SHAPE, "k=%d must be in [1, 256]", k);
    return SERQ_OK;
}

// workspace pieces of the whole L2QER layer: xq, xscale, tq, tscale (MXFP4:
// Q(T) as E2M1 rows of k_pad / 2 bytes and their E8M0 bytes)
void l2qer_ws_parts(const serq_layout *L, int32_t M, int32_t k, size_t part[4]) {
    const int kp = l2qer_kpad(k);
    size_t b0 = 0, b1 = 0;
    act_bytes(M, L->d_in, L->fmt, &b0, &b1);
    part[0] = align256(b0);
    part[1] = align256(b1);
    part[2] = align256((size_t)M * (size_t)(kp / 2));
    part[3] = L->fmt == SERQ_FMT_MXFP4 ? align256((size_t)M * (size_t)(kp / 32))
                                       : align256((size_t)M * (sizeof(float) + sizeof(int32_t) * (size_t)(kp / 128)));
}

serq_status launch_l2qer_t(const serq_layout *L, int32_t k, const uint8_t *xq, const void *xscale, int32_t M,
                           const uint8_t *l1q, const void *l1scale, float *T, uint8_t *tq, void *tscale,
                           hipStream_t st) {
    const int K = L->d_in, kp = l2qer_kpad(k);
    if (L->fmt == SERQ_FMT_MXFP4) {
        if ((size_t)M * (size_t)(K / 2) >= kBufLimit)
            return fail(SERQ_ERR_UNSUPPORTED, "MXFP4 L2QER activations must stay below 2 GiB (32-bit offsets)");
        const unsigned tb8 = (unsigned)((M + 127) / 128);   // token blocks in whole rounds of the 8 XCDs
        hipLaunchKernelGGL(k_l2qer_mx, dim3(tb8 * 8 * (L2X_KP / L2X_CG)), dim3(64 * L2X_KS), 0, st, xq,
                           (const uint8_t *)xscale, M, K, l1q, (const uint8_t *)l1scale, T, tq, (uint8_t *)tscale);
        return hip_status(hipGetLastError(), "l2qer (MXFP4) launch");
    }
    const float *sx = (const float *)xscale;
    const int *xsum = (const int *)((const uint8_t *)xscale + sizeof(float) * (size_t)M);
    const float *sl1 = (const float *)l1scale;
    const int *l1sum = (const int *)((const uint8_t *)l1scale + sizeof(float) * (size_t)kp);
    float *stp = (float *)tscale;
    int *tsum = (int *)((uint8_t *)tscale + sizeof(float) * (size_t)M);
    const dim3 grid((unsigned)((M + 15) / 16));
    const size_t lds = (size_t)L2Q_NW * 16 * kp * sizeof(int);
    if (kp == 128) {
        static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_l2qer<8>),
                                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (attr != hipSuccess) return hip_status(attr, "l2qer LDS attribute");
        hipLaunchKernelGGL((k_l2qer<8>), grid, dim3(64 * L2Q_NW), lds, st, xq, sx, xsum, M, K, l1q, sl1, l1sum, T, tq,
                           stp, tsum);
    } else {
        static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_l2qer<16>),
                                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (attr != hipSuccess) return hip_status(attr, "l2qer LDS attribute");
        hipLaunchKernelGGL((k_l2qer<16>), grid, dim3(64 * L2Q_NW), lds, st, xq, sx, xsum, M, K, l1q, sl1, l1sum, T,
                           tq, stp, tsum);
    }
    return hip_status(hipGetLastError(), "l2qer launch");
}

// the MXFP4 comparator's output GEMM: the wide LDS-direct kernel with Q(T) . L2
// in the residual's place (NB <= 7: Q(T)'s LDS tile takes the rest)
template <int NB, int NW = 4>
serq_status launch_l2qer_mx_nb(const uint8_t *xq, const uint8_t *xe, int M, const uint8_t *wq, const uint8_t *we,
                               const uint8_t *tq, const uint8_t *te, const uint8_t *l2q, const uint8_t *l2e, int N,
                               int K, float *Y, hipStream_t st) {
    const int bn = 32 * NB;
    const unsigned tiles = (unsigned)(((M + L_BM - 1) / L_BM) * ((N + bn - 1) / bn));
    hipLaunchKernelGGL((k_gemm_mxd<NB, NW, true>), dim3(tiles), dim3(64 * NW), 0, st, xq, xe, M, wq, we, l2q, l2e, N,
                       K, L2X_KP, Y, pick_gm(M, N), tq, te);
    return hip_status(hipGetLastError(), "l2qer (MXFP4) GEMM launch");
}

serq_status launch_l2qer_linear(const serq_layout *L, int32_t k, const uint8_t *xq, const void *xscale, int32_t M,
                                const uint8_t *wq, const void *wscale, const uint8_t *tq, const void *tscale,
                                const uint8_t *l2q, const void *l2scale, float *Y, hipStream_t st) {
    const int N = L->d_out, K = L->d_in, kp = l2qer_kpad(k);
    const bool small_bufs = L->wq_bytes < kBufLimit && (size_t)M * (size_t)(K / 2) < kBufLimit;
    if (L->fmt == SERQ_FMT_MXFP4) {
        if (!(M > kDecodeMaxM && K % 512 == 0 && small_bufs))
            return fail(SERQ_ERR_UNSUPPORTED, "the MXFP4 L2QER comparator runs on the LDS-direct kernel only "
                                              "(M > %d, d_in a multiple of 512), got M=%d d_in=%d", kDecodeMaxM, M, K);
        const uint8_t *xe = (const uint8_t *)xscale, *we = (const uint8_t *)wscale, *te = (const uint8_t *)tscale,
                      *l2e = (const uint8_t *)l2scale;
        // the tiles SERQ's own launch would take (widths up to 224 here)
        if (M > G_BM && !mx_wide_fits(M, N, 7))   // 256 x 128 tiles, 8 waves
            return launch_l2qer_mx_nb<4, 8>(xq, xe, M, wq, we, tq, te, l2q, l2e, N, K, Y, st);
        if (mx_wide_nb(M, N, 7) == 6) return launch_l2qer_mx_nb<6>(xq, xe, M, wq, we, tq, te, l2q, l2e, N, K, Y, st);
        return launch_l2qer_mx_nb<7>(xq, xe, M, wq, we, tq, te, l2q, l2e, N, K, Y, st);
    }
    if (!(M > G_BM && K % 256 == 0 && small_bufs))
        return fail(SERQ_ERR_UNSUPPORTED, "the L2QER comparator runs on the large-tile kernel only "
                                          "(M > %d, d_in a multiple of 256), got M=%d d_in=%d", G_BM, M, K);
    IntArgs a;
    a.tq = tq;
    a.st = (const float *)tscale;
    a.tsum = (const int *)((const uint8_t *)tscale + sizeof(float) * (size_t)M);
    a.xq = xq;
    a.sx = (const float *)xscale;
    a.xsum = (const int *)((const uint8_t *)xscale + sizeof(float) * (size_t)M);
    a.wq = wq;
    a.sw = (const float *)wscale;
    a.wsum = (const int *)((const uint8_t *)wscale + sizeof(float) * (size_t)N);
    a.rq = l2q;
    a.sR = (const float *)l2scale;
    a.rsum = (const int *)((const uint8_t *)l2scale + sizeof(float) * (size_t)N);
    a.Y = Y;
    a.acc_main = nullptr;
    a.acc_res = nullptr;
    a.M = M;
    a.N = N;
    a.K = K;
    a.r_pad = kp;
    a.gm = pick_gm(M, N);
    return launch_big(a, st);
}

// The MXFP4 gate|up GEMM with the SwiGLU into the next layer's MXFP4 input:
// tile widths whose waves hold whole MX blocks of H (256 channels with four
// waves, 128 with eight), the one whose whole rounds of workgroups carry
// fewer channels.
template <int NB, int NW>
serq_status launch_swiglu_mx_nb(const uint8_t *xq, const uint8_t *xe, int M, const uint8_t *wq, const uint8_t *we,
                                const uint8_t *rq, const uint8_t *re, int N, int K, int rp, const float *s_next,
                                uint8_t *xqn, uint8_t *xen, hipStream_t st) {
    const int bn = 32 * NB;
    const unsigned tiles = (unsigned)(((M + L_BM - 1) / L_BM) * ((N + bn - 1) / bn));
    hipLaunchKernelGGL((k_gemm_mxd<NB, NW, false, true>), dim3(tiles), dim3(64 * NW), 0, st, xq, xe, M, wq, we, rq, re,
                       N, K, rp, (float *)nullptr, pick_gm(M, N), nullptr, nullptr, s_next, xqn, xen);
    return hip_status(hipGetLastError(), "gate|up SwiGLU (MXFP4) launch");
}

serq_status launch_swiglu_mx(const uint8_t *xq, const uint8_t *xe, int M, const uint8_t *wq, const uint8_t *we,
                             const uint8_t *rq, const uint8_t *re, int N, int K, int rp, const float *s_next,
                             uint8_t *xqn, uint8_t *xen, hipStream_t st) {
    const long cus = cu_count(), mt = (M + L_BM - 1) / L_BM;
    const long wide = (mt * ((N + 255) / 256) + cus - 1) / cus * 256;
    const long narrow = (mt * ((N + 127) / 128) + cus - 1) / cus * 128;
    if (wide <= narrow) return launch_swiglu_mx_nb<8, 4>(xq, xe, M, wq, we, rq, re, N, K, rp, s_next, xqn, xen, st);
    return launch_swiglu_mx_nb<4, 8>(xq, xe, M, wq, we, rq, re, N, K, rp, s_next, xqn, xen, st);
}

// rq (and, for MXFP4, rscale) are empty when r == 0 and may then be NULL.
serq_status check_weights(const serq_layout *L, const uint8_t *wq, const void *wscale, const uint8_t *rq,
                          const void *rscale) {
    const bool need_rq = L->rq_bytes > 0, need_rs = L->rscale_bytes > 0;
    if (!wq || !wscale || (need_rq && !rq) || (need_rs && !rscale))
        return fail(SERQ_ERR_INVALID_ARG, "a weight pointer is NULL");
    if (!aligned16(wq) || !aligned16(wscale) || (rq && !aligned16(rq)) || (rscale && !aligned16(rscale)))
        return fail(SERQ_ERR_INVALID_ARG, "weight buffers must be 16-byte aligned");
    return SERQ_OK;
}

}  // namespace
}  // namespace serq

using namespace serq;

extern "C" {

serq_status serq_quant_act(const void *X, serq_dtype xdt, int32_t M, int32_t d_in, serq_format fmt,
                           uint8_t *xq, void *xscale, void *stream) {
    clear_error();
    if (!X || !xq || !xscale) return fail(SERQ_ERR_INVALID_ARG, "a required pointer is NULL");
    if (xdt != SERQ_DT_F32 && xdt != SERQ_DT_BF16) return fail(SERQ_ERR_INVALID_ARG, "unknown serq_dtype %d", (int)xdt);
    size_t b0, b1;
    serq_status st = act_bytes(M, d_in, (int32_t)fmt, &b0, &b1);
    if (st) return st;
    if (!aligned16(X) || !aligned16(xq) || !aligned16(xscale))
        return fail(SERQ_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
    return launch_quant(X, xdt, M, d_in, fmt, xq, xscale, (hipStream_t)stream);
}

}  // extern "C"

namespace serq {
namespace {
serq_status check_producer(const void *in, serq_dtype xdt, int32_t M, int32_t d, const int32_t *perm, const float *s,
                           serq_format fmt, const uint8_t *xq, const void *xscale, bool perm_optional) {
    if (!in || (!perm && !perm_optional) || !s || !xq || !xscale)
        return fail(SERQ_ERR_INVALID_ARG, "a required pointer is NULL");
    if (xdt != SERQ_DT_F32 && xdt != SERQ_DT_BF16) return fail(SERQ_ERR_INVALID_ARG, "unknown serq_dtype %d", (int)xdt);
    size_t b0, b1;
    serq_status st = act_bytes(M, d, (int32_t)fmt, &b0, &b1);
    if (st) return st;
    if (d > kQuantMaxInReg)
        return fail(SERQ_ERR_UNSUPPORTED, "d=%d: the producer kernels hold a row of at most %d channels", d,
                    kQuantMaxInReg);
    if (!aligned16(in) || (perm && !aligned16(perm)) || !aligned16(s) || !aligned16(xq) || !aligned16(xscale))
        return fail(SERQ_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
    return SERQ_OK;
}
}  // namespace
}  // namespace serq

extern "C" {

serq_status serq_rmsnorm_quant(const void *H, serq_dtype hdt, int32_t M, int32_t d, const float *gamma, float eps,
                               const int32_t *perm, const float *s, serq_format fmt, uint8_t *xq, void *xscale,
                               void *stream) {
    clear_error();
    serq_status st = check_producer(H, hdt, M, d, perm, s, fmt, xq, xscale, false);
    if (st) return st;
    if (!gamma) return fail(SERQ_ERR_INVALID_ARG, "gamma is NULL");
    if (!aligned16(gamma)) return fail(SERQ_ERR_INVALID_ARG, "gamma must be 16-byte aligned");
    if (!(eps >= 0.0f) || eps == __builtin_inff()) return fail(SERQ_ERR_INVALID_ARG, "eps must be finite and >= 0");
    const ProducerArgs a{0, H, M, d, gamma, eps, perm, s, xq, xscale};
    return launch_producer(a, hdt, fmt, (hipStream_t)stream);
}

serq_status serq_swiglu_quant(const void *GU, serq_dtype dt, int32_t M, int32_t d, const int32_t *perm,
                              const float *s, serq_format fmt, uint8_t *xq, void *xscale, void *stream) {
    clear_error();
    serq_status st = check_producer(GU, dt, M, d, perm, s, fmt, xq, xscale, true);
    if (st) return st;
    const ProducerArgs a{1, GU, M, d, nullptr, 0.0f, perm, s, xq, xscale};
    return launch_producer(a, dt, fmt, (hipStream_t)stream);
}

size_t serq_linear_workspace_bytes(const serq_layout *L, int32_t M) {
    if (check_layout(L) != SERQ_OK) return 0;
    size_t b0, b1;
    if (act_bytes(M, L->d_in, L->fmt, &b0, &b1) != SERQ_OK) return 0;
    return align256(b0) + align256(b1);
}

serq_status serq_linear_q(const serq_layout *L, const uint8_t *xq, const void *xscale, int32_t M,
                          const uint8_t *wq, const void *wscale, const uint8_t *rq, const void *rscale,
                          float *Y, int32_t *acc_main, int32_t *acc_res, void *stream) {
    clear_error();
    serq_status st = check_layout(L);
    if (st) return st;
    if (M < 1) return fail(SERQ_ERR_SHAPE, "M=%d must be >= 1", M);
    if (!xq || !xscale || !Y) return fail(SERQ_ERR_INVALID_ARG, "a required pointer is NULL");
    if ((st = check_weights(L, wq, wscale, rq, rscale))) return st;
    if (!aligned16(xq) || !aligned16(xscale) || !aligned16(Y))
        return fail(SERQ_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
    if ((L->fmt == SERQ_FMT_MXFP4 || L->fmt == SERQ_FMT_MXW4A8) && (acc_main || acc_res))
        return fail(SERQ_ERR_INVALID_ARG, "integer accumulators exist only for INT4 and W4A8");
    if ((acc_main == nullptr) != (acc_res == nullptr))
        return fail(SERQ_ERR_INVALID_ARG, "acc_main and acc_res must both be given or both be NULL");
    if ((acc_main && !aligned16(acc_main)) || (acc_res && !aligned16(acc_res)))
        return fail(SERQ_ERR_INVALID_ARG, "accumulator buffers must be 16-byte aligned");
    size_t b0, b1;
    if ((st = act_bytes(M, L->d_in, L->fmt, &b0, &b1))) return st;
    return launch_linear(L, xq, xscale, M, wq, wscale, rq, rscale, Y, acc_main, acc_res, (hipStream_t)stream);
}

serq_status serq_linear(const serq_layout *L, const void *X, serq_dtype xdt, int32_t M, const uint8_t *wq,
                        const void *wscale, const uint8_t *rq, const void *rscale, float *Y,
                        void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    serq_status st = check_layout(L);
    if (st) return st;
    if (!X || !Y || !workspace) return fail(SERQ_ERR_INVALID_ARG, "a required pointer is NULL");
    if (xdt != SERQ_DT_F32 && xdt != SERQ_DT_BF16) return fail(SERQ_ERR_INVALID_ARG, "unknown serq_dtype %d", (int)xdt);
    if ((st = check_weights(L, wq, wscale, rq, rscale))) return st;
    size_t b0, b1;
    if ((st = act_bytes(M, L->d_in, L->fmt, &b0, &b1))) return st;
    const size_t need = align256(b0) + align256(b1);
    if (workspace_bytes < need)
        return fail(SERQ_ERR_BUFFER, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    if (!aligned16(X) || !aligned16(Y) || !aligned16(workspace))
        return fail(SERQ_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
    uint8_t *xq = (uint8_t *)workspace;
    void *xs = (uint8_t *)workspace + align256(b0);
    hipStream_t hs = (hipStream_t)stream;
    if ((st = launch_quant(X, xdt, M, L->d_in, L->fmt, xq, xs, hs))) return st;
    return launch_linear(L, xq, xs, M, wq, wscale, rq, rscale, Y, nullptr, nullptr, hs);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free form of serq_linear: the quantized activations go to a
// file-scope device array instead of a caller workspace.  Each device that
// loads the library holds its own copy of the array until the process ends;
// host code reaches it only through the address hipGetSymbolAddress returns
// for that device (the array's own name is a host-side stand-in).
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[SERQ_NOALLOC_SCRATCH_BYTES];

namespace serq {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices] = {};

// The device the stream belongs to (the current device for the null stream).
serq_status stream_device(hipStream_t st, int *dev) {
    hipError_t e;
    if (st == nullptr) {
        e = hipGetDevice(dev);
    } else {
        hipDevice_t d = 0;
        e = hipStreamGetDevice(st, &d);
        *dev = (int)d;
    }
    if (e != hipSuccess) return hip_status(e, "device of the stream");
    if (*dev < 0 || *dev >= kMaxDevices) return fail(SERQ_ERR_UNSUPPORTED, "device %d is beyond %d", *dev, kMaxDevices);
    return SERQ_OK;
}

// The scratch array's address on `dev`, looked up once per device with that
// device current (and the caller's current device restored).
serq_status scratch_on(int dev, uint8_t **out) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return hip_status(e, "hipGetDevice");
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e, "hipSetDevice");
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t back = hipSetDevice(cur);
            if (e == hipSuccess) e = back;
        }
        if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
        if (!ptr) return fail(SERQ_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_dev[dev] = ptr;
    }
    *out = (uint8_t *)g_scratch_dev[dev];
    return SERQ_OK;
}

}  // namespace
}  // namespace serq

extern "C" {

serq_status serq_linear_noalloc(const serq_layout *L, const void *X, serq_dtype xdt, int32_t M, const uint8_t *wq,
                                const void *wscale, const uint8_t *rq, const void *rscale, float *Y, void *stream) {
    clear_error();
    serq_status st = check_layout(L);
    if (st) return st;
    if (!X || !Y) return fail(SERQ_ERR_INVALID_ARG, "a required pointer is NULL");
    if (xdt != SERQ_DT_F32 && xdt != SERQ_DT_BF16) return fail(SERQ_ERR_INVALID_ARG, "unknown serq_dtype %d", (int)xdt);
    if ((st = check_weights(L, wq, wscale, rq, rscale))) return st;
    size_t b0, b1;
    if ((st = act_bytes(M, L->d_in, L->fmt, &b0, &b1))) return st;
    const size_t need = align256(b0) + align256(b1);
    if (need > (size_t)SERQ_NOALLOC_SCRATCH_BYTES)
        return fail(SERQ_ERR_BUFFER, "M=%d, d_in=%d needs %zu bytes of quantized activations; the allocation-free "
                    "entry point holds at most %zu", M, L->d_in, need, (size_t)SERQ_NOALLOC_SCRATCH_BYTES);
    if (!aligned16(X) || !aligned16(Y)) return fail(SERQ_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
    hipStream_t hs = (hipStream_t)stream;
    int dev = 0;
    if ((st = stream_device(hs, &dev))) return st;
    uint8_t *base = nullptr;
    if ((st = scratch_on(dev, &base))) return st;
    uint8_t *xq = base;
    void *xs = base + align256(b0);
    if ((st = launch_quant(X, xdt, M, L->d_in, L->fmt, xq, xs, hs))) return st;
    return launch_linear(L, xq, xs, M, wq, wscale, rq, rscale, Y, nullptr, nullptr, hs);
}

serq_status serq_linear_swiglu(const serq_layout *L, const void *X, serq_dtype xdt, int32_t M, const uint8_t *wq,
                               const void *wscale, const uint8_t *rq, const void *rscale, const float *s_next,
                               float *H, void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    serq_status st = check_layout(L);
    if (st) return st;
    if (!X || !H || !s_next || !workspace) return fail(SERQ_ERR_INVALID_ARG, "a required pointer is NULL");
    if (xdt != SERQ_DT_F32 && xdt != SERQ_DT_BF16) return fail(SERQ_ERR_INVALID_ARG, "unknown serq_dtype %d", (int)xdt);
    if ((st = check_weights(L, wq, wscale, rq, rscale))) return st;
    size_t b0, b1;
    if ((st = act_bytes(M, L->d_in, L->fmt, &b0, &b1))) return st;
    if (L->fmt != SERQ_FMT_INT4)
        return fail(SERQ_ERR_UNSUPPORTED, "the SwiGLU epilogue is built for INT4 layers");
    const bool small_bufs = L->wq_bytes < kBufLimit && (size_t)M * (size_t)(L->d_in / 2) < kBufLimit;
    if (!(M > G_BM && L->d_in % 256 == 0 && L->r_pad <= 256 && small_bufs))
        return fail(SERQ_ERR_UNSUPPORTED, "the SwiGLU epilogue runs on the large-tile kernel only (M > %d, d_in a "
                    "multiple of 256, r <= 256), got M=%d d_in=%d r=%d", G_BM, M, L->d_in, L->r);
    const size_t need = align256(b0) + align256(b1);
    if (workspace_bytes < need)
        return fail(SERQ_ERR_BUFFER, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    if (!aligned16(X) || !aligned16(H) || !aligned16(s_next) || !aligned16(workspace))
        return fail(SERQ_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
    uint8_t *xq = (uint8_t *)workspace;
    void *xs = (uint8_t *)workspace + align256(b0);
    hipStream_t hs = (hipStream_t)stream;
    if ((st = launch_quant(X, xdt, M, L->d_in, L->fmt, xq, xs, hs))) return st;
    const int N = L->d_out;
    IntArgs a;
    a.xq = xq;
    a.sx = (const float *)xs;
    a.xsum = (const int *)((const uint8_t *)xs + sizeof(float) * (size_t)M);
    a.wq = wq;
    a.sw = (const float *)wscale;
    a.wsum = (const int *)((const uint8_t *)wscale + sizeof(float) * (size_t)N);
    a.rq = L->r_pad > 0 ? rq : wq;
    a.sR = (const float *)(L->r_pad > 0 ? rscale : wscale);
    a.rsum = (const int *)((const uint8_t *)a.sR + sizeof(float) * (size_t)N);
    a.Y = nullptr;
    a.acc_main = nullptr;
    a.acc_res = nullptr;
    a.M = M;
    a.N = N;
    a.K = L->d_in;
    a.r_pad = L->r_pad;
    a.gm = pick_gm(M, N);
    a.sdown = s_next;
    a.H = H;
    return launch_big(a, hs);
}

serq_status serq_linear_swiglu_q(const serq_layout *L, const void *X, serq_dtype xdt, int32_t M, const uint8_t *wq,
                                 const void *wscale, const uint8_t *rq, const void *rscale, const float *s_next,
                                 uint8_t *xq_next, uint8_t *xscale_next, void *workspace, size_t workspace_bytes,
                                 void *stream) {
    clear_error();
    serq_status st = check_layout(L);
    if (st) return st;
    if (!X || !s_next || !xq_next || !xscale_next || !workspace)
        return fail(SERQ_ERR_INVALID_ARG, "a required pointer is NULL");
    if (xdt != SERQ_DT_F32 && xdt != SERQ_DT_BF16) return fail(SERQ_ERR_INVALID_ARG, "unknown serq_dtype %d", (int)xdt);
    if ((st = check_weights(L, wq, wscale, rq, rscale))) return st;
    size_t b0, b1;
    if ((st = act_bytes(M, L->d_in, L->fmt, &b0, &b1))) return st;
    if (L->fmt != SERQ_FMT_MXFP4)
        return fail(SERQ_ERR_UNSUPPORTED, "the quantizing SwiGLU epilogue is built for MXFP4 layers");
    if (L->d_out % 256)
        return fail(SERQ_ERR_SHAPE, "d_out=%d: the next layer's d_in = d_out / 2 must be a multiple of 128", L->d_out);
    const bool small_bufs = L->wq_bytes < kBufLimit && (size_t)M * (size_t)(L->d_in / 2) < kBufLimit;
    if (!(M > kDecodeMaxM && L->d_in % 512 == 0 && L->r_pad <= 128 && small_bufs))
        return fail(SERQ_ERR_UNSUPPORTED, "the quantizing SwiGLU epilogue runs on the LDS-direct kernel only (M > %d, "
                    "d_in a multiple of 512, r <= 128), got M=%d d_in=%d r=%d", kDecodeMaxM, M, L->d_in, L->r);
    const size_t need = align256(b0) + align256(b1);
    if (workspace_bytes < need)
        return fail(SERQ_ERR_BUFFER, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    if (!aligned16(X) || !aligned16(s_next) || !aligned16(xq_next) || !aligned16(xscale_next) || !aligned16(workspace))
        return fail(SERQ_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
    uint8_t *xq = (uint8_t *)workspace;
    uint8_t *xe = (uint8_t *)workspace + align256(b0);
    hipStream_t hs = (hipStream_t)stream;
    if ((st = launch_quant(X, xdt, M, L->d_in, L->fmt, xq, xe, hs))) return st;
    const uint8_t *rqp = L->r_pad > 0 ? rq : wq;
    const uint8_t *rep = (const uint8_t *)(L->r_pad > 0 ? rscale : wscale);
    return launch_swiglu_mx(xq, xe, M, wq, (const uint8_t *)wscale, rqp, rep, L->d_out, L->d_in, L->r_pad, s_next,
                            xq_next, xscale_next, hs);
}

size_t serq_l2qer_workspace_bytes(const serq_layout *L, int32_t M, int32_t k) {
    if (check_l2qer(L, k) != SERQ_OK || M < 1) return 0;
    size_t part[4];
    l2qer_ws_parts(L, M, k, part);
    return part[0] + part[1] + part[2] + part[3];
}

serq_status serq_l2qer_intermediate(const serq_layout *L, int32_t k, const uint8_t *xq, const void *xscale, int32_t M,
                                    const uint8_t *l1q, const void *l1scale, float *T, uint8_t *tq, void *tscale,
                                    void *stream) {
    clear_error();
    serq_status st = check_l2qer(L, k);
    if (st) return st;
    if (M < 1) return fail(SERQ_ERR_SHAPE, "M=%d must be >= 1", M);
    if (!xq || !xscale || !l1q || !l1scale || !tq || !tscale)
        return fail(SERQ_ERR_INVALID_ARG, "a required pointer is NULL");
    if (!aligned16(xq) || !aligned16(xscale) || !aligned16(l1q) || !aligned16(l1scale) || !aligned16(tq) ||
        !aligned16(tscale) || (T && !aligned16(T)))
        return fail(SERQ_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
    return launch_l2qer_t(L, k, xq, xscale, M, l1q, l1scale, T, tq, tscale, (hipStream_t)stream);
}

serq_status serq_l2qer_linear_q(const serq_layout *L, int32_t k, const uint8_t *xq, const void *xscale, int32_t M,
                                const uint8_t *wq, const void *wscale, const uint8_t *tq, const void *tscale,
                                const uint8_t *l2q, const void *l2scale, float *Y, void *stream) {
    clear_error();
    serq_status st = check_l2qer(L, k);
    if (st) return st;
    if (M < 1) return fail(SERQ_ERR_SHAPE, "M=%d must be >= 1", M);
    if (!xq || !xscale || !wq || !wscale || !tq || !tscale || !l2q || !l2scale || !Y)
        return fail(SERQ_ERR_INVALID_ARG, "a required pointer is NULL");
    if (!aligned16(xq) || !aligned16(xscale) || !aligned16(wq) || !aligned16(wscale) || !aligned16(tq) ||
        !aligned16(tscale) || !aligned16(l2q) || !aligned16(l2scale) || !aligned16(Y))
        return fail(SERQ_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
    return launch_l2qer_linear(L, k, xq, xscale, M, wq, wscale, tq, tscale, l2q, l2scale, Y, (hipStream_t)stream);
}

serq_status serq_l2qer_linear(const serq_layout *L, int32_t k, const void *X, serq_dtype xdt, int32_t M,
                              const uint8_t *wq, const void *wscale, const uint8_t *l1q, const void *l1scale,
                              const uint8_t *l2q, const void *l2scale, float *Y, void *workspace,
                              size_t workspace_bytes, void *stream) {
    clear_error();
    serq_status st = check_l2qer(L, k);
    if (st) return st;
    if (M < 1) return fail(SERQ_ERR_SHAPE, "M=%d must be >= 1", M);
    if (xdt != SERQ_DT_F32 && xdt != SERQ_DT_BF16) return fail(SERQ_ERR_INVALID_ARG, "unknown serq_dtype %d", (int)xdt);
    if (!X || !wq || !wscale || !l1q || !l1scale || !l2q || !l2scale || !Y || !workspace)
        return fail(SERQ_ERR_INVALID_ARG, "a required pointer is NULL");
    if (!aligned16(X) || !aligned16(wq) || !aligned16(wscale) || !aligned16(l1q) || !aligned16(l1scale) ||
        !aligned16(l2q) || !aligned16(l2scale) || !aligned16(Y) || !aligned16(workspace))
        return fail(SERQ_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");
    size_t part[4];
    l2qer_ws_parts(L, M, k, part);
    const size_t need = part[0] + part[1] + part[2] + part[3];
    if (workspace_bytes < need) return fail(SERQ_ERR_BUFFER, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    if (L->fmt == SERQ_FMT_MXFP4 ? !(M > kDecodeMaxM && L->d_in % 512 == 0) : !(M > G_BM && L->d_in % 256 == 0))
        return fail(SERQ_ERR_UNSUPPORTED, "the L2QER comparator's envelope: INT4 M > %d and d_in a multiple of 256, "
                                          "MXFP4 M > %d and d_in a multiple of 512; got M=%d d_in=%d",
                    G_BM, kDecodeMaxM, M, L->d_in);
    uint8_t *base = (uint8_t *)workspace;
    uint8_t *xq = base;
    void *xs = base + part[0];
    uint8_t *tq = base + part[0] + part[1];
    void *ts = base + part[0] + part[1] + part[2];
    hipStream_t hs = (hipStream_t)stream;
    if ((st = launch_quant(X, xdt, M, L->d_in, L->fmt, xq, xs, hs))) return st;
    if ((st = launch_l2qer_t(L, k, xq, xs, M, l1q, l1scale, nullptr, tq, ts, hs))) return st;
    return launch_l2qer_linear(L, k, xq, xs, M, wq, wscale, tq, ts, l2q, l2scale, Y, hs);
}

}  // extern "C"
