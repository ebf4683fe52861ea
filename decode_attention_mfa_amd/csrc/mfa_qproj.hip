// mfa_qproj.hip -- the low-rank query path of MFA on CDNA4 (gfx950):
// hidden -> 2048-wide bottleneck -> 64 heads x 256 ("Step-3 is Large yet
// Affordable", Key points), with RMSNorm on the bottleneck.
//
//   down   c_part[split] = x . W_qa[k-range]      skinny bf16 MFMA GEMM, fp32
//   norm   chat = bf16(sum_split c_part * rsqrt(mean(c^2) + eps) * gamma)
//   up     q = bf16(chat . W_qb)                   skinny bf16 MFMA GEMM
//
// Both GEMMs have few rows (the batch) and stream a large row-major [in][out]
// weight from HBM once. Each workgroup owns 64 output columns; 64x64 weight
// tiles go HBM -> registers -> LDS and come back transposed with
// ds_read_b64_tr_b16 as MFMA B operands (the contraction index is the
// weight's row). Activation rows are read straight into A-operand registers.
#include "mfa_device.h"
#include "mfa_internal.h"

namespace mfa {

// Weight tile in LDS: 64 rows x 64 bf16 (128 B), 16-byte chunks XOR-swizzled
// per row pair so the transposed reads of 4 rows hit distinct banks.
__device__ __forceinline__ int wswz(int row) { return ((row >> 1) & 3) << 1; }

// Y[m][n] over m < M, n in [64*blockIdx.x, +64), k in split blockIdx.y of
// K/gridDim.y rows, M rows in blocks of 64 (blockIdx.z).
// OUT_BF16: Y is bf16 [M][N]; otherwise fp32 partials [split][M][N].
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void mfa_skinny_gemm_kernel(const uint16_t* __restrict__ X, int ldx,
                                                              const uint16_t* __restrict__ W, int N,
                                                              int K, int M, void* __restrict__ Y) {
    __shared__ __attribute__((aligned(16))) uint8_t wt[2][64 * 128];
    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, lr = l & 15, g = l >> 4;
    const int n0 = 64 * blockIdx.x;
    const int kper = K / gridDim.y;
    const int kbeg = kper * blockIdx.y;
    const int m0 = 64 * blockIdx.z;
    const int mt_n = min(4, (M - m0 + 15) / 16);   // 16-row tiles in this block

    f32x4 acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; mt++) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // thread -> two 16-byte pieces of the 64x64 tile: rows tid/8 and tid/8+32
    const int wr = tid >> 3, wc = tid & 7;
    auto load_tile = [&](int kb, u32x4& r0, u32x4& r1) {
        const uint16_t* src = W + (int64_t)(kb + wr) * N + n0 + 8 * wc;
        r0 = *reinterpret_cast<const u32x4*>(src);
        r1 = *reinterpret_cast<const u32x4*>(src + (int64_t)32 * N);
    };
    auto store_tile = [&](uint8_t* t, const u32x4& r0, const u32x4& r1) {
        *reinterpret_cast<u32x4*>(t + wr * 128 + 16 * (wc ^ wswz(wr))) = r0;
        *reinterpret_cast<u32x4*>(t + (wr + 32) * 128 + 16 * (wc ^ wswz(wr + 32))) = r1;
    };

    const int nkb = kper / 64;
    u32x4 r0, r1;
    load_tile(kbeg, r0, r1);
    store_tile(wt[0], r0, r1);
    __syncthreads();
    for (int kb = 0; kb < nkb; kb++) {
        const uint8_t* t = wt[kb & 1];
        if (kb + 1 < nkb) load_tile(kbeg + 64 * (kb + 1), r0, r1);
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {
            // B operand: W[k = 32ks + 8g + j][n0 + 16w + lr], j = 0..7
            const int ch = 2 * w + ((lr & 3) >> 1);
            const int row0 = 32 * ks + 8 * g + (lr >> 2);
            const int row1 = row0 + 4;
            const i16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4*)(t + row0 * 128 + 16 * (ch ^ wswz(row0)) + 8 * (lr & 1)));
            const i16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4*)(t + row1 * 128 + 16 * (ch ^ wswz(row1)) + 8 * (lr & 1)));
            const u32x2 u0 = bitcast<u32x2>(b0), u1 = bitcast<u32x2>(b1);
            const bf16x8 bop = bitcast<bf16x8>(u32x4{u0.x, u0.y, u1.x, u1.y});
            const int kcol = kbeg + 64 * kb + 32 * ks + 8 * g;
#pragma unroll
            for (int mt = 0; mt < 4; mt++) {
                if (mt < mt_n) {
                    const int row = min(m0 + 16 * mt + lr, M - 1);
                    const bf16x8 aop = *reinterpret_cast<const bf16x8*>(X + (int64_t)row * ldx + kcol);
                    acc[mt] = mfma16(aop, bop, acc[mt]);
                }
            }
        }
        if (kb + 1 < nkb) {
            store_tile(wt[(kb + 1) & 1], r0, r1);
            __syncthreads();
        }
    }

    const int n = n0 + 16 * w + lr;
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
        if (mt >= mt_n) continue;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int m = m0 + 16 * mt + 4 * g + i;
            if (m >= M) continue;
            if constexpr (OUT_BF16) {
                reinterpret_cast<uint16_t*>(Y)[(int64_t)m * N + n] = bitcast<uint16_t>((__bf16)acc[mt][i]);
            } else {
                reinterpret_cast<float*>(Y)[((int64_t)blockIdx.y * M + m) * N + n] = acc[mt][i];
            }
        }
    }
}

// chat[m][j] = bf16(c[m][j] * rsqrt(mean_j c^2 + eps) * gamma[j]),
// c = sum over the K-splits of c_part (fixed order). Block = one row m.
__global__ __launch_bounds__(256) void mfa_rmsnorm_kernel(const float* __restrict__ c_part, int ksplit,
                                                          int M, int rank,
                                                          const uint16_t* __restrict__ gamma, float eps,
                                                          uint16_t* __restrict__ chat) {
    __shared__ float red[4];
    const int m = blockIdx.x;
    float ss = 0.f;
    for (int j = threadIdx.x; j < rank; j += 256) {
        float c = 0.f;
        for (int s = 0; s < ksplit; s++) c += c_part[((int64_t)s * M + m) * rank + j];
        ss += c * c;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    const float r = 1.0f / __builtin_sqrtf(tot / (float)rank + eps);
    for (int j = threadIdx.x; j < rank; j += 256) {
        float c = 0.f;
        for (int s = 0; s < ksplit; s++) c += c_part[((int64_t)s * M + m) * rank + j];
        const float gm = (float)bitcast<__bf16>(gamma[j]);
        chat[(int64_t)m * rank + j] = bitcast<uint16_t>((__bf16)(c * r * gm));
    }
}

hipError_t launch_qproj_down(const QprojArgs& a, const Launch& l) {
    const int mblk = (a.batch + 63) / 64;
    return launch_kernel(mfa_skinny_gemm_kernel<false>, dim3(a.rank / 64, a.ksplit, mblk), dim3(256), l, a.x,
                         a.hidden, a.w_qa, a.rank, a.hidden, a.batch, (void*)a.c_part);
}

hipError_t launch_rmsnorm(const QprojArgs& a, const Launch& l) {
    return launch_kernel(mfa_rmsnorm_kernel, dim3(a.batch), dim3(256), l, (const float*)a.c_part, a.ksplit, a.batch,
                         a.rank, a.rms_w, a.eps, a.chat);
}

hipError_t launch_qproj_up(const QprojArgs& a, const Launch& l) {
    const int mblk = (a.batch + 63) / 64;
    return launch_kernel(mfa_skinny_gemm_kernel<true>, dim3(a.nq / 64, 1, mblk), dim3(256), l,
                         (const uint16_t*)a.chat, a.rank, a.w_qb, a.nq, a.rank, a.batch, (void*)a.q_out);
}

}  // namespace mfa
