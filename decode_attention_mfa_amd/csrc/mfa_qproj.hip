// mfa_qproj.hip -- the low-rank query path of MFA on CDNA4 (gfx950):
// hidden -> 2048-wide bottleneck -> 64 heads x 256 ("Step-3 is Large yet
// Affordable", Key points), with RMSNorm on the bottleneck.
//
//   down   c_part[split] = x . W_qa[k-range]      skinny bf16 MFMA GEMM, fp32
//   norm   chat = bf16(sum_split c_part * rsqrt(mean(c^2) + eps) * gamma)
//   up     q = bf16(chat . W_qb)                   skinny bf16 MFMA GEMM
//
// The same skinny GEMM also computes the new token's key and value rows,
// x . W_k and x . W_v (hidden -> 256 each, one launch for both weights), for
// the KV append.
//
// The GEMMs have few rows (the batch) and read a large row-major [in][out]
// weight from HBM exactly once, so they are bandwidth-bound. Each workgroup
// owns 64 output columns and a range of K; per 64-row K tile, the weight tile
// (64 x 64) and the matching activation tile (64 rows x 64) stream into an
// LDS ring by direct DMA, three tiles deep (48 KB of LDS, so that several
// workgroups share a compute unit: occupancy hides more of the load latency
// than a deeper ring in one workgroup does). The weight tile comes back
// transposed with ds_read_b64_tr_b16 as MFMA B operands (the contraction
// index is the weight's row), the activation tile as A operands.
#include "mfa_device.h"
#include "mfa_internal.h"

namespace mfa {

namespace {

constexpr int kGemmDepth = 3;             // K tiles in the ring
constexpr int kTileBytes = 64 * 128;      // 64 rows x 64 bf16

// 16-byte chunk positions within a 128-byte tile row. Weight rows: swizzled
// per row pair so that the transposed reads of 4 rows hit distinct banks.
// Activation rows: per row, so that 16 rows read at one chunk index spread
// over 8 bank groups.
__device__ __forceinline__ int wswz(int row) { return ((row >> 1) & 3) << 1; }
__device__ __forceinline__ int xswz(int row) { return row & 7; }

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 bytes per lane from global memory into LDS (lane i lands at
// lds_dst + 16*i; lds_dst wave-uniform, through M0). Inline asm so that the
// compiler does not order later LDS accesses behind it; the ring's own waits
// order the reads. Weight tiles are read once: streaming hint (nt). The
// activation tiles are re-read by every column block: default cache policy,
// so they stay in L2.
__device__ __forceinline__ void dma16_stream(const void* sbase, uint32_t voff, uint32_t lds_dst) {
    asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "{m0}"(lds_dst) : "memory");
}
__device__ __forceinline__ void dma16_keep(const void* sbase, uint32_t voff, uint32_t lds_dst) {
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds_dst) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// LDS-only workgroup barrier (does not wait for the DMA still in flight).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ const uint8_t* uniform_ptr(const void* ptr) {
    const uint64_t u = (uint64_t)(uintptr_t)ptr;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

}  // namespace

// Y[m][n] over m in [MR*blockIdx.z, +MR) with m < M, n in [64*bx, +64),
// k in [kper*blockIdx.y, +kper) (kper a multiple of 64), where bx =
// blockIdx.x. A grid of 2 * N/64 columns of blocks computes a second product
// X . W2 into Y2 with the blocks bx >= N/64 (bx - N/64 there).
// MR (32 or 64) rows per block: 32 when the batch fits, so that the
// activation tile carries no repeated rows.
// OUT_BF16: Y is bf16 [M][N]; otherwise fp32 partials [gridDim.y][M][N].
template <bool OUT_BF16, int MR>
__global__ __launch_bounds__(256) void mfa_skinny_gemm_kernel(const uint16_t* __restrict__ X, int ldx,
                                                              const uint16_t* __restrict__ W, int N, int kper,
                                                              int M, void* __restrict__ Y,
                                                              const uint16_t* __restrict__ W2, void* __restrict__ Y2) {
    static_assert(MR == 32 || MR == 64, "rows per block");
    constexpr int MT = MR / 16;            // 16-row MFMA tiles
    constexpr int XI = MR / 32;            // activation DMA instructions per wave and tile
    constexpr int OPS = 2 + XI;            // DMA instructions per wave and tile
    constexpr int kSlot = kTileBytes + MR * 128;
    // slot: weight tile (64 rows x 128 B), then activation tile (MR rows x 128 B)
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kGemmDepth][kSlot];
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, lr = l & 15, g = l >> 4;
    int bx = blockIdx.x;
    if (bx >= N / 64) {
        bx -= N / 64;
        W = W2;
        Y = Y2;
    }
    const int n0 = 64 * bx;
    const int kbeg = kper * blockIdx.y;
    const int m0 = MR * blockIdx.z;
    const int mt_n = min(MT, (M - m0 + 15) / 16);   // 16-row tiles holding real rows
    const int ntiles = kper / 64;

    // DMA lane offsets (loop-invariant). Weight instruction i of wave w fills
    // tile rows 16w + 8i + l/8, activation instruction i rows MR/4*w + 8i +
    // l/8; lane l lands at chunk position l % 8 of its row and fetches the
    // data chunk the swizzle puts there. Activation rows past M repeat row
    // M-1 (in bounds; their products are never stored).
    uint32_t woff[2], xoff[XI];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int r = 16 * w + 8 * i + (l >> 3);
        woff[i] = (uint32_t)(r * N * 2 + 16 * ((l & 7) ^ wswz(r)));
    }
#pragma unroll
    for (int i = 0; i < XI; i++) {
        const int r = MR / 4 * w + 8 * i + (l >> 3);
        const int xr = min(m0 + r, M - 1) - m0;   // row within this block
        xoff[i] = (uint32_t)(xr * ldx * 2 + 16 * ((l & 7) ^ xswz(r)));
    }
    auto issue = [&](int tile) {   // clamped to the last tile
        const int k0 = kbeg + 64 * min(tile, ntiles - 1);
        const uint8_t* wb = uniform_ptr(W + (int64_t)k0 * N + n0);
        const uint8_t* xb = uniform_ptr(X + (int64_t)m0 * ldx + k0);
        const uint32_t slot = lds_addr_of(ring[tile % kGemmDepth]);
        const uint32_t wdst = __builtin_amdgcn_readfirstlane(slot + 2048 * w);
        const uint32_t xdst = __builtin_amdgcn_readfirstlane(slot + kTileBytes + MR * 32 * w);
#pragma unroll
        for (int i = 0; i < 2; i++) dma16_stream(wb, woff[i], wdst + 1024 * i);
#pragma unroll
        for (int i = 0; i < XI; i++) dma16_keep(xb, xoff[i], xdst + 1024 * i);
    };

    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int s = 0; s < kGemmDepth - 1; s++) issue(s);
    for (int tile = 0; tile < ntiles; tile++) {
        // this wave's rows of the tile have landed once at most the younger
        // tiles' loads are in flight; the barrier shows every wave's rows and
        // frees the slot of the previous tile
        wait_vmem<(kGemmDepth - 2) * OPS>();
        lds_barrier();
        issue(tile + kGemmDepth - 1);
        const uint8_t* wt = ring[tile % kGemmDepth];
        const uint8_t* xt = wt + kTileBytes;
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {
            // B operand: W[k = 32ks + 8g + j][n0 + 16w + lr], j = 0..7
            const int ch = 2 * w + ((lr & 3) >> 1);
            const int row0 = 32 * ks + 8 * g + (lr >> 2);
            const int row1 = row0 + 4;
            const i16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4*)(wt + row0 * 128 + 16 * (ch ^ wswz(row0)) + 8 * (lr & 1)));
            const i16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) i16x4*)(wt + row1 * 128 + 16 * (ch ^ wswz(row1)) + 8 * (lr & 1)));
            const u32x2 u0 = bitcast<u32x2>(b0), u1 = bitcast<u32x2>(b1);
            const bf16x8 bop = bitcast<bf16x8>(u32x4{u0.x, u0.y, u1.x, u1.y});
#pragma unroll
            for (int mt = 0; mt < MT; mt++) {
                if (mt < mt_n) {
                    // A operand: X[m0 + 16mt + lr][k = 32ks + 8g + j]
                    const int r = 16 * mt + lr;
                    const bf16x8 aop = *reinterpret_cast<const bf16x8*>(xt + r * 128 + 16 * ((4 * ks + g) ^ xswz(r)));
                    acc[mt] = mfma16(aop, bop, acc[mt]);
                }
            }
        }
    }
    wait_vmem<0>();   // the clamped loads past the last tile

    const int n = n0 + 16 * w + lr;
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
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

// chat[m][j] = bf16(c[m][j] * rsqrt(mean_j c^2 + eps) * gamma[j]), with
// c = the sum of the K-split partials in split order. Block = one row m;
// thread t handles columns 4t + 1024q. Each pass issues the loads of eight
// splits of a column group before summing them.
__global__ __launch_bounds__(256) void mfa_rmsnorm_kernel(const float* __restrict__ c_part, int ksplit, int M,
                                                          int rank, const uint16_t* __restrict__ gamma, float eps,
                                                          uint16_t* __restrict__ chat) {
    __shared__ float red[4];
    const int m = blockIdx.x;
    const f32x4* cp = reinterpret_cast<const f32x4*>(c_part) + (int64_t)m * (rank / 4);
    const int64_t plane = (int64_t)M * (rank / 4);   // f32x4 per split plane
    auto col_sum = [&](int j4) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
        int s = 0;
        for (; s + 8 <= ksplit; s += 8) {
            f32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; u++) v[u] = cp[(s + u) * plane + j4];
#pragma unroll
            for (int u = 0; u < 8; u++) c += v[u];
        }
        for (; s < ksplit; s++) c += cp[s * plane + j4];
        return c;
    };
    float ss = 0.f;
    for (int j4 = threadIdx.x; j4 < rank / 4; j4 += 256) {
        const f32x4 c = col_sum(j4);
        ss += (c[0] * c[0] + c[1] * c[1]) + (c[2] * c[2] + c[3] * c[3]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    const float r = 1.0f / __builtin_sqrtf(tot / (float)rank + eps);
    for (int j4 = threadIdx.x; j4 < rank / 4; j4 += 256) {
        const f32x4 c = col_sum(j4);
        const u32x2 gw = *reinterpret_cast<const u32x2*>(gamma + 4 * j4);
        const float g0 = __builtin_bit_cast(float, gw.x << 16), g1 = __builtin_bit_cast(float, gw.x & 0xffff0000u);
        const float g2 = __builtin_bit_cast(float, gw.y << 16), g3 = __builtin_bit_cast(float, gw.y & 0xffff0000u);
        *reinterpret_cast<u32x2*>(chat + (int64_t)m * rank + 4 * j4) =
            u32x2{pack_bf16x2(c[0] * r * g0, c[1] * r * g1), pack_bf16x2(c[2] * r * g2, c[3] * r * g3)};
    }
}

// Rows per block: 32 when the whole batch fits in one such block, else 64.
template <bool OUT_BF16>
static hipError_t launch_skinny(int gx, int gy, const uint16_t* X, int ldx, const uint16_t* W, int N, int kper,
                                int M, void* Y, const uint16_t* W2, void* Y2, const Launch& l) {
    if (M <= 32)
        return launch_kernel(mfa_skinny_gemm_kernel<OUT_BF16, 32>, dim3(gx, gy, 1), dim3(256), l, X, ldx, W, N,
                             kper, M, Y, W2, Y2);
    return launch_kernel(mfa_skinny_gemm_kernel<OUT_BF16, 64>, dim3(gx, gy, (M + 63) / 64), dim3(256), l, X, ldx,
                         W, N, kper, M, Y, W2, Y2);
}

hipError_t launch_qproj_down(const QprojArgs& a, const Launch& l) {
    return launch_skinny<false>(a.rank / 64, a.ksplit, a.x, a.hidden, a.w_qa, a.rank, a.hidden / a.ksplit, a.batch,
                                (void*)a.c_part, nullptr, nullptr, l);
}

hipError_t launch_rmsnorm(const QprojArgs& a, const Launch& l) {
    return launch_kernel(mfa_rmsnorm_kernel, dim3(a.batch), dim3(256), l, (const float*)a.c_part, a.ksplit, a.batch,
                         a.rank, a.rms_w, a.eps, a.chat);
}

hipError_t launch_qproj_up(const QprojArgs& a, const Launch& l) {
    return launch_skinny<true>(a.nq / 64, 1, a.chat, a.rank, a.w_qb, a.nq, a.rank, a.batch, (void*)a.q_out, nullptr,
                               nullptr, l);
}

hipError_t launch_kv_proj(const KvAppendArgs& a, const Launch& l) {
    float* kp = a.kv_part;
    float* vp = a.kv_part + (int64_t)a.ksplit * a.batch * kHeadDim;
    return launch_skinny<false>(2 * kHeadDim / 64, a.ksplit, a.x, a.hidden, a.w_k, kHeadDim, a.hidden / a.ksplit,
                                a.batch, (void*)kp, a.w_v, (void*)vp, l);
}

}  // namespace mfa
