// Device half of the SERQ library for gfx950 (CDNA4): the on-the-fly
// activation quantizer and the fused linear kernels, plus the runtime entry
// points of serq.h that launch them.
//
// The runtime layer follows the Stage 2 inference equation of the SERQ
// research notes (dihengye.cn):  Y ~= Xhat_q . What_q + Xtilde_{s,q} . Q(R).
// The residual product reuses the first r columns of the same quantized
// activation (no intermediate quantization, gist.science summaries section
// 2.2) and is fused into the main GEMM's K loop: while the K loop walks the
// first r_pad columns it also multiplies the staged activation tile by the
// matching tile of Q(R).
//
// INT4 / W4A8 run on int8 MFMA (v_mfma_i32_16x16x64_i8) with nibbles expanded
// in registers; MXFP4 runs on the block-scaled FP4 MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4), whose 32-element scale blocks are the
// MX blocks.
#include <hip/hip_runtime.h>
#include <stdint.h>

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
// per token; MX blocks per the OCP MX definition).  One workgroup per token.
// Thread t owns the 4-element chunks t, t + 256, t + 512, ... of its row, so
// every load and store instruction of a wave touches one contiguous span.
// ===========================================================================

constexpr int QA_THREADS = 256;
constexpr int QA_MAXCH = kQuantMaxInReg / (4 * QA_THREADS);   // chunks kept in registers

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

// Symmetric RTN code: rne(x / s) with an IEEE fp32 quotient, clipped to +-Q.
template <int Q>
__device__ __forceinline__ int rtn_code(float x, float s) {
    const float q = rintf(x / s);
    return (int)fminf(fmaxf(q, -(float)Q), (float)Q);
}

template <int Q, bool BF16>
__global__ __launch_bounds__(QA_THREADS) void k_quant_int(const void *__restrict__ X, int d_in,
                                                          uint8_t *__restrict__ xq,
                                                          float *__restrict__ sx) {
    const int m = blockIdx.x, t = threadIdx.x;
    const int nch = d_in >> 2;
    const size_t base = (size_t)m * (size_t)d_in;
    const bool inreg = nch <= QA_MAXCH * QA_THREADS;
    float4 v[QA_MAXCH];
    float amax = 0.0f;
    if (inreg) {
#pragma unroll
        for (int c = 0; c < QA_MAXCH; ++c) {
            const int j = t + c * QA_THREADS;
            if (j < nch) {
                v[c] = load4<BF16>(X, base + 4 * (size_t)j);
                amax = fmaxf(amax, amax4(v[c]));
            }
        }
    } else {
        for (int j = t; j < nch; j += QA_THREADS) amax = fmaxf(amax, amax4(load4<BF16>(X, base + 4 * (size_t)j)));
    }
    __shared__ float red[QA_THREADS / 64];
    amax = wave_max(amax);
    if ((t & 63) == 0) red[t >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
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
        if constexpr (Q == 7) {
            const uint32_t b = (uint32_t)(q0 & 15) | ((uint32_t)(q1 & 15) << 4) |
                               ((uint32_t)(q2 & 15) << 8) | ((uint32_t)(q3 & 15) << 12);
            *reinterpret_cast<uint16_t *>(xq + (size_t)m * (size_t)(d_in >> 1) + 2 * (size_t)j) = (uint16_t)b;
        } else {
            const uint32_t b = (uint32_t)(q0 & 255) | ((uint32_t)(q1 & 255) << 8) |
                               ((uint32_t)(q2 & 255) << 16) | ((uint32_t)(q3 & 255) << 24);
            *reinterpret_cast<uint32_t *>(xq + base + 4 * (size_t)j) = b;
        }
    };
    if (inreg) {
#pragma unroll
        for (int c = 0; c < QA_MAXCH; ++c) {
            const int j = t + c * QA_THREADS;
            if (j < nch) encode(v[c], j);
        }
    } else {
        for (int j = t; j < nch; j += QA_THREADS) encode(load4<BF16>(X, base + 4 * (size_t)j), j);
    }
}

// OCP MX shared exponent floor(log2 amax) - 2 from the fp32 exponent field,
// clamped to E8M0's range; 0 for an all-zero block.
__device__ __forceinline__ int mx_exponent(float amax) {
    if (!(amax > 0.0f)) return 0;
    const int e = (int)((__float_as_uint(amax) >> 23) & 0xffu) - 127 - 2;
    return min(127, max(-127, e));
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

template <bool BF16>
__global__ __launch_bounds__(QA_THREADS) void k_quant_mx(const void *__restrict__ X, int d_in,
                                                         uint8_t *__restrict__ xq,
                                                         uint8_t *__restrict__ xe) {
    const int m = blockIdx.x, t = threadIdx.x;
    const int nch = d_in >> 2;   // a multiple of 32: groups of 8 lanes (one MX block) stay whole
    const size_t base = (size_t)m * (size_t)d_in;
    for (int j = t; j < nch; j += QA_THREADS) {
        const float4 u = load4<BF16>(X, base + 4 * (size_t)j);
        float a = amax4(u);
        a = fmaxf(a, __shfl_xor(a, 1));
        a = fmaxf(a, __shfl_xor(a, 2));
        a = fmaxf(a, __shfl_xor(a, 4));
        const int e = mx_exponent(a);
        if ((j & 7) == 0) xe[(size_t)m * (size_t)(d_in >> 5) + (j >> 3)] = (uint8_t)(e + 127);
        const float inv = __uint_as_float((uint32_t)(127 - e) << 23);   // 2^-e, exact
        const uint32_t b = e2m1_code(u.x * inv) | (e2m1_code(u.y * inv) << 4) |
                           (e2m1_code(u.z * inv) << 8) | (e2m1_code(u.w * inv) << 12);
        *reinterpret_cast<uint16_t *>(xq + (size_t)m * (size_t)(d_in >> 1) + 2 * (size_t)j) = (uint16_t)b;
    }
}

// ===========================================================================
// Fused GEMM building blocks
// ===========================================================================

// Nibble expansion: p holds 8 two's-complement nibbles (element k in byte k/2,
// low nibble first).  hi() keeps the odd elements in the high half of each
// byte (int8 value 16*w), lo() moves the even ones there.  Both operands of a
// product are expanded the same way, so every product is 256*x*w (16*x*w for
// W4A8) and the exact int32 sum is shifted back in the epilogue.
__device__ __forceinline__ int nib_hi(uint32_t p) { return (int)(p & 0xF0F0F0F0u); }
__device__ __forceinline__ int nib_lo(uint32_t p) { return (int)((p << 4) & 0xF0F0F0F0u); }

// 16 packed bytes (32 nibbles) -> the two 16x16x64 operands of this lane.
__device__ __forceinline__ void unpack32(u32x4 p, v4i &op0, v4i &op1) {
    op0 = v4i{nib_lo(p.x), nib_hi(p.x), nib_lo(p.y), nib_hi(p.y)};
    op1 = v4i{nib_lo(p.z), nib_hi(p.z), nib_lo(p.w), nib_hi(p.w)};
}

// 32 int8 activations -> the same element order unpack32 produces
// (even elements of each 8-group, then odd ones).
__device__ __forceinline__ v4i reorder16(u32x4 a) {
    const uint32_t E = 0x06040200u, O = 0x07050301u;
    return v4i{(int)__builtin_amdgcn_perm(a.y, a.x, E), (int)__builtin_amdgcn_perm(a.y, a.x, O),
               (int)__builtin_amdgcn_perm(a.w, a.z, E), (int)__builtin_amdgcn_perm(a.w, a.z, O)};
}

// LDS tiles hold rows of 64 (or 128) bytes split into 16-byte columns.  A
// lane group reads one column of 16 consecutive rows; XOR-ing the column with
// these row functions spreads those rows over all banks.
__device__ __forceinline__ int swz4(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }
__device__ __forceinline__ int swz8(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ u32x4 lds16(const uint8_t *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ u32x4 gld16(const uint8_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

constexpr int G_BM = 128, G_BN = 128, G_THREADS = 256;

// ===========================================================================
// Prefill INT4 / W4A8 kernel.  Tile 128 x 128 x (K step 128), 4 waves in a
// 2 x 2 grid, each wave 64 x 64 = 4 x 4 MFMA blocks of 16 x 16.  Two exact
// int32 accumulators per block: A_main over all K, A_res over the first r_pad
// columns (same staged activation tile, Q(R) tile instead of What_q).
// Double-buffered LDS, one barrier per K step.
// ===========================================================================
template <bool A8>
__global__ __launch_bounds__(G_THREADS) void k_gemm_int(
    const uint8_t *__restrict__ xq, const float *__restrict__ sx, int M,
    const uint8_t *__restrict__ wq, const float *__restrict__ sw,
    const uint8_t *__restrict__ rq, const float *__restrict__ sR,
    int N, int K, int r_pad, float *__restrict__ Y,
    int *__restrict__ acc_main, int *__restrict__ acc_res) {
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
    const size_t w_ld = (size_t)(K >> 1), r_ld = (size_t)(r_pad >> 1);

    // global -> LDS copy plan (rows past M or N re-read the last row; their
    // results are never stored)
    const uint8_t *a_src[A_CH];
    int a_dst[A_CH];
#pragma unroll
    for (int u = 0; u < A_CH; ++u) {
        const int c = t + u * G_THREADS, row = c / A_CPR, col = c % A_CPR;
        a_src[u] = xq + (size_t)min(m0 + row, M - 1) * a_ld + col * 16;
        a_dst[u] = row * A_ROWB + (col ^ (A8 ? swz8(row) : swz4(row))) * 16;
    }
    const uint8_t *w_src[2], *r_src[2];
    int b_dst[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int c = t + u * G_THREADS, row = c >> 2, col = c & 3;
        const size_t n = (size_t)min(n0 + row, N - 1);
        w_src[u] = wq + n * w_ld + col * 16;
        r_src[u] = rq + n * r_ld + col * 16;
        b_dst[u] = row * 64 + (col ^ swz4(row)) * 16;
    }
    u32x4 ra[A_CH], rw[2], rr[2];
    auto gload = [&](int kt, bool res) {
#pragma unroll
        for (int u = 0; u < A_CH; ++u) ra[u] = gld16(a_src[u] + (size_t)kt * A_ROWB);
#pragma unroll
        for (int u = 0; u < 2; ++u) rw[u] = gld16(w_src[u] + (size_t)kt * 64);
        if (res) {
#pragma unroll
            for (int u = 0; u < 2; ++u) rr[u] = gld16(r_src[u] + (size_t)kt * 64);
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
        for (int rb = 0; rb < 4; ++rb) {
            const int row = wm * 64 + rb * 16 + i;
            if constexpr (A8) {
                a0[rb] = reorder16(lds16(s + row * 128 + (((2 * g) ^ swz8(row)) * 16)));
                a1[rb] = reorder16(lds16(s + row * 128 + (((2 * g + 1) ^ swz8(row)) * 16)));
            } else {
                unpack32(lds16(s + row * 64 + ((g ^ swz4(row)) * 16)), a0[rb], a1[rb]);
            }
        }
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const int col = wn * 64 + cb * 16 + i;
            v4i b0, b1;
            unpack32(lds16(s + A_BYTES + col * 64 + ((g ^ swz4(col)) * 16)), b0, b1);
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                accm[rb][cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0[rb], b0, accm[rb][cb], 0, 0, 0);
                accm[rb][cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1[rb], b1, accm[rb][cb], 0, 0, 0);
            }
        }
        if (kt < RT) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const int col = wn * 64 + cb * 16 + i;
                v4i b0, b1;
                unpack32(lds16(s + A_BYTES + B_BYTES + col * 64 + ((g ^ swz4(col)) * 16)), b0, b1);
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    accr[rb][cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0[rb], b0, accr[rb][cb], 0, 0, 0);
                    accr[rb][cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1[rb], b1, accr[rb][cb], 0, 0, 0);
                }
            }
        }
        if (nxt) sstore((kt + 1) & 1, kt + 1 < RT);
        __syncthreads();
    }

    // epilogue: Y = sx[m] * (sw[o] * A_main + sR[o] * A_res).  MFMA block
    // layout: lane (g, i) holds rows 4g..4g+3 of column i.
    constexpr int SH = A8 ? 4 : 8;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const int col = n0 + wn * 64 + cb * 16 + i;
        if (col >= N) continue;
        const float swc = sw[col], src = sR[col];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = m0 + wm * 64 + rb * 16 + 4 * g + v;
                if (row >= M) continue;
                const int am = accm[rb][cb][v] >> SH, ar = accr[rb][cb][v] >> SH;
                const size_t o = (size_t)row * (size_t)N + col;
                Y[o] = sx[row] * fmaf(swc, (float)am, src * (float)ar);
                if (acc_main) acc_main[o] = am;
                if (acc_res) acc_res[o] = ar;
            }
        }
    }
}

// ===========================================================================
// Prefill MXFP4 kernel.  Same tiling; one K step of 128 is one scaled MFMA
// per block, each lane group's 16 bytes being one 32-element MX block whose
// E8M0 scale the lane supplies.  The residual blocks are extra K blocks of
// the same fp32 accumulator: Q(R) carries its own block scales, so the
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
    const size_t ld = (size_t)(K >> 1), r_ld = (size_t)(r_pad >> 1);
    const size_t sld = (size_t)(K >> 5), r_sld = (size_t)(r_pad >> 5);

    const uint8_t *a_src[2], *w_src[2], *r_src[2];
    int dst[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int c = t + u * G_THREADS, row = c >> 2, col = c & 3;
        a_src[u] = xq + (size_t)min(m0 + row, M - 1) * ld + col * 16;
        const size_t n = (size_t)min(n0 + row, N - 1);
        w_src[u] = wq + n * ld + col * 16;
        r_src[u] = rq + n * r_ld + col * 16;
        dst[u] = row * 64 + (col ^ swz4(row)) * 16;
    }
    // scale copies: threads 0..127 the activation rows, 128..255 the W and R rows
    const int srow = t & 127;
    const bool s_act = t < 128;
    const uint8_t *s_src = s_act ? xe + (size_t)min(m0 + srow, M - 1) * sld
                                 : we + (size_t)min(n0 + srow, N - 1) * sld;
    const uint8_t *sr_src = re + (size_t)min(n0 + srow, N - 1) * r_sld;

    u32x4 ra[2], rw[2], rr[2];
    uint32_t rs = 0, rsr = 0;
    auto gload = [&](int kt, bool res) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            ra[u] = gld16(a_src[u] + (size_t)kt * 64);
            rw[u] = gld16(w_src[u] + (size_t)kt * 64);
        }
        rs = *reinterpret_cast<const uint32_t *>(s_src + (size_t)kt * 4);
        if (res) {
#pragma unroll
            for (int u = 0; u < 2; ++u) rr[u] = gld16(r_src[u] + (size_t)kt * 64);
            if (!s_act) rsr = *reinterpret_cast<const uint32_t *>(sr_src + (size_t)kt * 4);
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
// Decode INT4 / W4A8 kernel (M <= 16 tokens: bandwidth-bound).  A workgroup
// owns NB blocks of 16 output channels; its NW waves split the K steps (main
// steps followed by the r_pad/128 residual steps) evenly and reduce their
// int32 partial sums in LDS.  Weights stream straight from HBM into
// registers: each lane group reads 16 contiguous bytes of a row per step.
// ===========================================================================
template <bool A8, int NB, int NW>
__global__ __launch_bounds__(64 * NW) void k_decode_int(
    const uint8_t *__restrict__ xq, const float *__restrict__ sx, int M,
    const uint8_t *__restrict__ wq, const float *__restrict__ sw,
    const uint8_t *__restrict__ rq, const float *__restrict__ sR,
    int N, int K, int r_pad, float *__restrict__ Y,
    int *__restrict__ acc_main, int *__restrict__ acc_res) {
    __shared__ int red[NW][2][NB][4][64];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int i = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * NB * 16;
    const int KT = K >> 7, RT = r_pad >> 7, T = KT + RT;
    const int lo = (T * w) / NW, hi = (T * (w + 1)) / NW;
    const bool live = i < M;
    const uint8_t *a_row = xq + (size_t)min(i, M - 1) * (A8 ? (size_t)K : (size_t)(K >> 1));
    const uint8_t *w_row[NB], *r_row[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const size_t n = (size_t)min(n0 + nb * 16 + i, N - 1);
        w_row[nb] = wq + n * (size_t)(K >> 1) + g * 16;
        r_row[nb] = rq + n * (size_t)(r_pad >> 1) + g * 16;
    }
    auto a_frag = [&](int kt, v4i &o0, v4i &o1) {
        if constexpr (A8) {
            o0 = reorder16(gld16(a_row + (size_t)kt * 128 + g * 32));
            o1 = reorder16(gld16(a_row + (size_t)kt * 128 + g * 32 + 16));
        } else {
            unpack32(gld16(a_row + (size_t)kt * 64 + g * 16), o0, o1);
        }
        if (!live) o0 = o1 = v4i{0, 0, 0, 0};
    };
    v4i accm[NB], accr[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) accm[nb] = accr[nb] = v4i{0, 0, 0, 0};

    const int main_hi = min(hi, KT);
#pragma unroll 2
    for (int kt = lo; kt < main_hi; ++kt) {
        u32x4 p[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) p[nb] = gld16(w_row[nb] + (size_t)kt * 64);
        v4i a0, a1;
        a_frag(kt, a0, a1);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            v4i b0, b1;
            unpack32(p[nb], b0, b1);
            accm[nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, accm[nb], 0, 0, 0);
            accm[nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, accm[nb], 0, 0, 0);
        }
    }
    for (int v = max(lo, KT); v < hi; ++v) {
        const int kt = v - KT;
        u32x4 p[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) p[nb] = gld16(r_row[nb] + (size_t)kt * 64);
        v4i a0, a1;
        a_frag(kt, a0, a1);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            v4i b0, b1;
            unpack32(p[nb], b0, b1);
            accr[nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, accr[nb], 0, 0, 0);
            accr[nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, accr[nb], 0, 0, 0);
        }
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            red[w][0][nb][v][lane] = accm[nb][v];
            red[w][1][nb][v][lane] = accr[nb][v];
        }
    __syncthreads();
    constexpr int SH = A8 ? 4 : 8;
    for (int idx = t; idx < NB * 4 * 64; idx += 64 * NW) {
        const int nb = idx >> 8, v = (idx >> 6) & 3, l = idx & 63;
        int sm = 0, sr = 0;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            sm += red[ww][0][nb][v][l];
            sr += red[ww][1][nb][v][l];
        }
        const int row = 4 * (l >> 4) + v, col = n0 + nb * 16 + (l & 15);
        if (row < M && col < N) {
            const int am = sm >> SH, ar = sr >> SH;
            const size_t o = (size_t)row * (size_t)N + col;
            Y[o] = sx[row] * fmaf(sw[col], (float)am, sR[col] * (float)ar);
            if (acc_main) acc_main[o] = am;
            if (acc_res) acc_res[o] = ar;
        }
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

serq_status launch_quant(const void *X, int32_t xdt, int32_t M, int32_t d_in, int32_t fmt,
                         uint8_t *xq, void *xscale, hipStream_t st) {
    const dim3 grid((unsigned)M), block(QA_THREADS);
    const bool bf = xdt == SERQ_DT_BF16;
    if (fmt == SERQ_FMT_INT4) {
        if (bf) hipLaunchKernelGGL((k_quant_int<7, true>), grid, block, 0, st, X, d_in, xq, (float *)xscale);
        else hipLaunchKernelGGL((k_quant_int<7, false>), grid, block, 0, st, X, d_in, xq, (float *)xscale);
    } else if (fmt == SERQ_FMT_W4A8) {
        if (bf) hipLaunchKernelGGL((k_quant_int<127, true>), grid, block, 0, st, X, d_in, xq, (float *)xscale);
        else hipLaunchKernelGGL((k_quant_int<127, false>), grid, block, 0, st, X, d_in, xq, (float *)xscale);
    } else {
        if (bf) hipLaunchKernelGGL((k_quant_mx<true>), grid, block, 0, st, X, d_in, xq, (uint8_t *)xscale);
        else hipLaunchKernelGGL((k_quant_mx<false>), grid, block, 0, st, X, d_in, xq, (uint8_t *)xscale);
    }
    return hip_status(hipGetLastError(), "quant_act launch");
}

template <bool A8, int NB, int NW>
void launch_decode(const serq_layout *L, const uint8_t *xq, const float *sx, int M, const uint8_t *wq,
                   const float *sw, const uint8_t *rq, const float *sR, float *Y, int *am, int *ar,
                   hipStream_t st) {
    const int cols = NB * 16;
    const dim3 grid((unsigned)((L->d_out + cols - 1) / cols)), block(64 * NW);
    hipLaunchKernelGGL((k_decode_int<A8, NB, NW>), grid, block, 0, st, xq, sx, M, wq, sw, rq, sR, L->d_out,
                       L->d_in, L->r_pad, Y, am, ar);
}

// Tokens up to which the bandwidth-bound decode kernel is used.
constexpr int kDecodeMaxM = 16;

serq_status launch_linear(const serq_layout *L, const uint8_t *xq, const void *xscale, int32_t M,
                          const uint8_t *wq, const void *wscale, const uint8_t *rq, const void *rscale,
                          float *Y, int32_t *am, int32_t *ar, hipStream_t st) {
    const int N = L->d_out, K = L->d_in, rp = L->r_pad;
    if (rp == 0) {
        // no residual steps run; keep the (never dereferenced) R pointers valid
        rq = wq;
        if (!rscale) rscale = wscale;
    }
    if (L->fmt == SERQ_FMT_MXFP4) {
        const dim3 grid((unsigned)((N + G_BN - 1) / G_BN), (unsigned)((M + G_BM - 1) / G_BM));
        hipLaunchKernelGGL(k_gemm_mx, grid, dim3(G_THREADS), 0, st, xq, (const uint8_t *)xscale, M, wq,
                           (const uint8_t *)wscale, rq, (const uint8_t *)rscale, N, K, rp, Y);
        return hip_status(hipGetLastError(), "gemm_mx launch");
    }
    const bool a8 = L->fmt == SERQ_FMT_W4A8;
    const float *sx = (const float *)xscale, *sw = (const float *)wscale, *sR = (const float *)rscale;
    if (M <= kDecodeMaxM) {
        // wide layers: 4 column blocks per workgroup; narrow ones: 1 block and
        // 16 waves on K so that the grid still covers every CU
        const bool wide = N / 64 >= 256;
        if (a8) {
            if (wide) launch_decode<true, 4, 4>(L, xq, sx, M, wq, sw, rq, sR, Y, am, ar, st);
            else launch_decode<true, 1, 16>(L, xq, sx, M, wq, sw, rq, sR, Y, am, ar, st);
        } else {
            if (wide) launch_decode<false, 4, 4>(L, xq, sx, M, wq, sw, rq, sR, Y, am, ar, st);
            else launch_decode<false, 1, 16>(L, xq, sx, M, wq, sw, rq, sR, Y, am, ar, st);
        }
        return hip_status(hipGetLastError(), "decode launch");
    }
    const dim3 grid((unsigned)((N + G_BN - 1) / G_BN), (unsigned)((M + G_BM - 1) / G_BM));
    if (a8)
        hipLaunchKernelGGL((k_gemm_int<true>), grid, dim3(G_THREADS), 0, st, xq, sx, M, wq, sw, rq, sR, N, K,
                           rp, Y, am, ar);
    else
        hipLaunchKernelGGL((k_gemm_int<false>), grid, dim3(G_THREADS), 0, st, xq, sx, M, wq, sw, rq, sR, N,
                           K, rp, Y, am, ar);
    return hip_status(hipGetLastError(), "gemm_int launch");
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
    if (L->fmt == SERQ_FMT_MXFP4 && (acc_main || acc_res))
        return fail(SERQ_ERR_INVALID_ARG, "integer accumulators exist only for INT4 and W4A8");
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
