// Sustained-rate probes of the MI355X (gfx950) units the SERQ layer is priced
// against: the int8 MFMA (INT4 / W4A8 GEMMs), the block-scaled FP4 and FP8
// MFMAs (MXFP4 / MX W4A8 GEMMs), and HBM streaming reads and copies (decode,
// activation quantization).  Published peaks assume every SIMD issues one
// MFMA per pipeline slot at the nominal clock; these kernels measure what the
// chip sustains instead, so that a kernel's roofline fraction can be read
// against both.  Each MFMA probe wave runs NACC independent accumulator
// chains of back-to-back MFMAs on register operands (no memory traffic) and
// records the shader-clock cycles and the constant-rate wall clock of its
// loop, from which the host derives the shader clock under that load.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "serq_peaks.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));


// KIND: 0 int8 16x16x64, 1 FP4 x FP4 16x16x128 (scaled), 2 FP8 x FP8, 3 FP4 x FP8.
// One asm block holds the eight MFMAs of an iteration, each accumulating in
// place in its own AGPRs: left to itself the compiler rotates loop-carried
// accumulators between registers with moves every iteration, which would be
// timed instead of the MFMAs.  (MFMAs only: no memory access in the asm.)
#define SERQ_MFMA8(INSN, MODS)                                                                          \
    asm volatile(INSN " %0, %8, %9, %0" MODS "\n\t" INSN " %1, %8, %9, %1" MODS "\n\t"                \
                 INSN " %2, %8, %9, %2" MODS "\n\t" INSN " %3, %8, %9, %3" MODS "\n\t"                \
                 INSN " %4, %8, %9, %4" MODS "\n\t" INSN " %5, %8, %9, %5" MODS "\n\t"                \
                 INSN " %6, %8, %9, %6" MODS "\n\t" INSN " %7, %8, %9, %7" MODS                        \
                 : "+a"(c0), "+a"(c1), "+a"(c2), "+a"(c3), "+a"(c4), "+a"(c5), "+a"(c6), "+a"(c7)      \
                 : "v"(a), "v"(b), "v"(sc))

template <int KIND, int NT>
__global__ __launch_bounds__(NT) void k_mfma_rate(int iters, float *__restrict__ sink, long long *__restrict__ clocks) {
    const int t = threadIdx.x, lane = t & 63;
    const int sc = 127;   // E8M0 scale 2^0 for both operands
    v4f c0 = v4f{}, c1 = v4f{}, c2 = v4f{}, c3 = v4f{}, c4 = v4f{}, c5 = v4f{}, c6 = v4f{}, c7 = v4f{};
    long long k0, k1, w0, w1;
    if constexpr (KIND == 0 || KIND == 1) {   // 16-byte operands: int8 x 16, or FP4 x 32
        const v4i a = v4i{lane, lane * 3 + 1, lane ^ 5, 7}, b = v4i{lane * 5, 3, lane ^ 9, lane + 1};
        k0 = __clock64();
        w0 = wall_clock64();
        for (int it = 0; it < iters; ++it) {
            if constexpr (KIND == 0) SERQ_MFMA8("v_mfma_i32_16x16x64_i8", "");
            else SERQ_MFMA8("v_mfma_scale_f32_16x16x128_f8f6f4", ", %10, %10 op_sel_hi:[0,0,0] cbsz:4 blgp:4");
        }
        k1 = __clock64();
        w1 = wall_clock64();
    } else if constexpr (KIND == 2) {         // FP8 x FP8: 32-byte operands
        const v8i a = v8i{lane, lane * 3 + 1, lane ^ 5, 7, lane * 11, 2, lane + 9, 4};
        const v8i b = v8i{lane * 5, 3, lane ^ 9, lane + 1, 6, lane * 7, 1, lane ^ 2};
        k0 = __clock64();
        w0 = wall_clock64();
        for (int it = 0; it < iters; ++it)
            SERQ_MFMA8("v_mfma_scale_f32_16x16x128_f8f6f4", ", %10, %10 op_sel_hi:[0,0,0] cbsz:0 blgp:0");
        k1 = __clock64();
        w1 = wall_clock64();
    } else {                                  // FP4 (A, 16 bytes) x FP8 (B, 32 bytes)
        const v4i a = v4i{lane, lane * 3 + 1, lane ^ 5, 7};
        const v8i b = v8i{lane * 5, 3, lane ^ 9, lane + 1, 6, lane * 7, 1, lane ^ 2};
        k0 = __clock64();
        w0 = wall_clock64();
        for (int it = 0; it < iters; ++it)
            SERQ_MFMA8("v_mfma_scale_f32_16x16x128_f8f6f4", ", %10, %10 op_sel_hi:[0,0,0] cbsz:4 blgp:0");
        k1 = __clock64();
        w1 = wall_clock64();
    }
    const v4f s = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
    sink[(size_t)blockIdx.x * NT + t] = s[0] + s[1] + s[2] + s[3];
    if (blockIdx.x == 0 && t == 0) {
        clocks[0] = k1 - k0;
        clocks[1] = w1 - w0;
    }
}

// Streaming read: every lane reads 16-byte pieces at a grid stride and keeps
// their XOR (one word per thread is written, so no load is dead).
__global__ __launch_bounds__(256) void k_read(const u32x4 *__restrict__ src, size_t n16, uint32_t *__restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * 256;
    u32x4 x = u32x4{0u, 0u, 0u, 0u};
    for (size_t k = (size_t)blockIdx.x * 256 + threadIdx.x; k < n16; k += stride) x ^= src[k];
    sink[(size_t)blockIdx.x * 256 + threadIdx.x] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

__global__ __launch_bounds__(256) void k_copy(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, size_t n16) {
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t k = (size_t)blockIdx.x * 256 + threadIdx.x; k < n16; k += stride) dst[k] = src[k];
}

int cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
    return n;
}

template <int KIND>
hipError_t launch_mfma(int wps, int iters, float *sink, long long *clocks, hipStream_t st) {
    const dim3 grid((unsigned)cus());
    if (wps == 1) hipLaunchKernelGGL((k_mfma_rate<KIND, 256>), grid, dim3(256), 0, st, iters, sink, clocks);
    else hipLaunchKernelGGL((k_mfma_rate<KIND, 512>), grid, dim3(512), 0, st, iters, sink, clocks);
    return hipGetLastError();
}

}  // namespace

extern "C" {

int serq_peak_sink_floats(int waves_per_simd) { return cus() * 256 * waves_per_simd; }

int serq_peak_wall_khz(void) {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
    return khz;
}

int serq_peak_mfma(int kind, int waves_per_simd, int iters, float *sink, long long *clocks, void *stream) {
    if (kind < 0 || kind > 3 || (waves_per_simd != 1 && waves_per_simd != 2) || iters < 1 || !sink || !clocks)
        return -1;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e;
    switch (kind) {
    case 0: e = launch_mfma<0>(waves_per_simd, iters, sink, clocks, st); break;
    case 1: e = launch_mfma<1>(waves_per_simd, iters, sink, clocks, st); break;
    case 2: e = launch_mfma<2>(waves_per_simd, iters, sink, clocks, st); break;
    default: e = launch_mfma<3>(waves_per_simd, iters, sink, clocks, st); break;
    }
    return e == hipSuccess ? 0 : -5;
}

int serq_peak_read(const void *src, size_t bytes, uint32_t *sink, void *stream) {
    if (!src || !sink || bytes % 16 || ((uintptr_t)src & 15)) return -1;
    hipLaunchKernelGGL(k_read, dim3((unsigned)(cus() * 8)), dim3(256), 0, (hipStream_t)stream,
                       (const u32x4 *)src, bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

int serq_peak_copy(const void *src, void *dst, size_t bytes, void *stream) {
    if (!src || !dst || bytes % 16 || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return -1;
    hipLaunchKernelGGL(k_copy, dim3((unsigned)(cus() * 8)), dim3(256), 0, (hipStream_t)stream, (const u32x4 *)src,
                       (u32x4 *)dst, bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
