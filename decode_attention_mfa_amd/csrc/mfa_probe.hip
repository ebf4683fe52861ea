// mfa_probe.hip -- the matrix-core rate microbenchmark behind the MFMA
// fractions the measurement reports: independent chains of the two MFMA
// shapes the attention runs (v_mfma_f32_16x16x32_bf16 for bf16 operands and
// the unit-scaled v_mfma_f32_16x16x128_f8f6f4 for E4M3 codes) on operands
// held in registers, no memory traffic in the loop, two waves per SIMD. The
// launch's flop count divided by its duration is the rate the chip sustains
// on them, to set beside the dense peaks of the data sheet (2.5 PFLOP/s
// bf16, 5 PFLOP/s FP8).
#include "mfa_device.h"
#include "mfa_internal.h"

namespace mfa {

namespace {

constexpr int kRateChains = 8;   // independent accumulators per wave

// Operands from the lane index, so that nothing is a compile-time constant;
// small values keep the accumulators finite over any iteration count.
template <int KIND>
__global__ __launch_bounds__(256) void mfa_mfma_rate_kernel(int iters, float* sink) {
    const int l = threadIdx.x & 63;
    // eight accumulators as separate variables (an array of them made the
    // register allocator rotate the accumulators between registers inside
    // the loop, a copy per MFMA)
    f32x4 c0{}, c1{}, c2{}, c3{}, c4{}, c5{}, c6{}, c7{};
    if constexpr (KIND == 0) {
        bf16x8 a, b;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            a[i] = (__bf16)(1e-3f * (float)(l + i));
            b[i] = (__bf16)(1e-3f * (float)(64 - l + i));
        }
        // in place, written out: with the builtin the register allocator
        // still moved the accumulators between registers every round. The
        // compiler inserts no wait states after inline asm, so the reads of
        // the results below wait explicitly.
        for (int it = 0; it < iters; it++) {
            asm volatile(
                "v_mfma_f32_16x16x32_bf16 %0, %8, %9, %0\n\t"
                "v_mfma_f32_16x16x32_bf16 %1, %8, %9, %1\n\t"
                "v_mfma_f32_16x16x32_bf16 %2, %8, %9, %2\n\t"
                "v_mfma_f32_16x16x32_bf16 %3, %8, %9, %3\n\t"
                "v_mfma_f32_16x16x32_bf16 %4, %8, %9, %4\n\t"
                "v_mfma_f32_16x16x32_bf16 %5, %8, %9, %5\n\t"
                "v_mfma_f32_16x16x32_bf16 %6, %8, %9, %6\n\t"
                "v_mfma_f32_16x16x32_bf16 %7, %8, %9, %7"
                : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3), "+v"(c4), "+v"(c5), "+v"(c6), "+v"(c7)
                : "v"(a), "v"(b));
        }
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3), "+v"(c4), "+v"(c5), "+v"(c6), "+v"(c7));
    } else {
        i32x8 a, b;
#pragma unroll
        for (int i = 0; i < 8; i++) {   // E4M3 codes of small normal values
            a[i] = (int)(0x20202020u + (uint32_t)((l + i) & 7));
            b[i] = (int)(0x20202020u + (uint32_t)((l + 3 * i) & 7));
        }
        for (int it = 0; it < iters; it++) {
            c0 = mfma16_fp8(a, b, c0); c1 = mfma16_fp8(a, b, c1); c2 = mfma16_fp8(a, b, c2);
            c3 = mfma16_fp8(a, b, c3); c4 = mfma16_fp8(a, b, c4); c5 = mfma16_fp8(a, b, c5);
            c6 = mfma16_fp8(a, b, c6); c7 = mfma16_fp8(a, b, c7);
        }
    }
    const float s = ((c0[0] + c1[0]) + (c2[0] + c3[0])) + ((c4[0] + c5[0]) + (c6[0] + c7[0]));
    // never true for these operands (the sums are positive); keeps the MFMAs
    if (s < 0.f) sink[0] = s;
}

}  // namespace

hipError_t launch_mfma_rate(int kind, int iters, int workgroups, float* sink, const Launch& l) {
    const dim3 grid(workgroups), block(256);
    return kind == 0 ? launch_kernel(mfa_mfma_rate_kernel<0>, grid, block, l, iters, sink)
                     : launch_kernel(mfa_mfma_rate_kernel<1>, grid, block, l, iters, sink);
}

double mfma_rate_flops(int kind, int iters, int workgroups) {
    const double per_mfma = kind == 0 ? 2.0 * 16 * 16 * 32 : 2.0 * 16 * 16 * 128;
    return (double)workgroups * 4 /* waves */ * (double)iters * kRateChains * per_mfma;
}

}  // namespace mfa
