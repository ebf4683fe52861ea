// mfa_qproj.hip -- the low-rank query path of MFA on CDNA4 (gfx950):
// hidden -> 2048-wide bottleneck -> 64 heads x 256 ("Step-3 is Large yet
// Affordable", Key points), with RMSNorm on the bottleneck.
//
//   down   c_part[split] = x . W_qa[k-range]      skinny bf16 MFMA GEMM, fp32;
//          the last K split to finish a column block sums the partials in
//          split order and writes cg = bf16(c * gamma) and the block's
//          per-row sums of c^2
//   up     q = bf16(rsqrt(mean(c^2) + eps) * (cg . W_qb))   skinny bf16 MFMA
//          GEMM, the RMSNorm factor applied per row to the fp32 result
//
// The same skinny GEMM also computes the new token's key and value rows,
// x . W_k and x . W_v (hidden -> 256 each, one launch for both weights), for
// the KV append.
//
// The GEMMs have few rows (the batch) and read a large row-major [in][out]
// weight from HBM exactly once, so they are bandwidth-bound. Each workgroup
// (eight waves) owns 64 output columns and a range of K; per 64-row K tile,
// the weight tile (64 x 64) and the matching activation tile (32 or 64 rows
// x 64) stream into an LDS ring by direct DMA, four tiles deep, every wave
// issuing part of each tile's DMA. Waves w and w + 4 own the same 16 columns
// and take the two 32-row halves of each K tile; their sums are added
// through LDS after the loop. The weight tile comes back
// transposed with ds_read_b64_tr_b16 as MFMA B operands (the contraction
// index is the weight's row), the activation tile as A operands.
#include "mfa_device.h"
#include "mfa_internal.h"

namespace mfa {

namespace {

constexpr int kGemmDepth = 4;             // K tiles in the ring
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

// Eight device-coherent (sc1, agent scope) 16-byte loads, p[i] -> v[i],
// issued together; the asm block also waits for them, so no output register
// is left pending when it ends.
__device__ __forceinline__ void coherent_load_b128x8(f32x4* v, const f32x4* const* p) {
    asm volatile(
        "global_load_dwordx4 %0, %8, off sc1\n\t"
        "global_load_dwordx4 %1, %9, off sc1\n\t"
        "global_load_dwordx4 %2, %10, off sc1\n\t"
        "global_load_dwordx4 %3, %11, off sc1\n\t"
        "global_load_dwordx4 %4, %12, off sc1\n\t"
        "global_load_dwordx4 %5, %13, off sc1\n\t"
        "global_load_dwordx4 %6, %14, off sc1\n\t"
        "global_load_dwordx4 %7, %15, off sc1\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
        : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5]), "v"(p[6]), "v"(p[7])
        : "memory");
}

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
// EPI selects the output:
//   kEpiPartials  fp32 partials [gridDim.y][M][N] in Y;
//   kEpiBf16      bf16 [M][N] in Y;
//   kEpiNormPrep  partials as kEpiPartials, then the last K split to finish
//                 column block bx (counted in e.counters) sums them in split
//                 order: e.cg[m][n] = bf16(c * gamma[n]) and e.sumsq[m][bx] =
//                 sum over the block's 64 columns of c^2;
//   kEpiBf16RowScale  bf16(acc * r[m]) in Y, r[m] = rsqrt(sum_j e.sumsq[m][j]
//                 / e.rank + e.eps) over the e.rank / 64 column blocks j.
constexpr int kGemmThreads = 512;   // eight waves

template <int EPI, int MR>
__global__ __launch_bounds__(kGemmThreads) void mfa_skinny_gemm_kernel(const uint16_t* __restrict__ X, int ldx,
                                                              const uint16_t* __restrict__ W, int N, int kper,
                                                              int M, void* __restrict__ Y,
                                                              const uint16_t* __restrict__ W2, void* __restrict__ Y2,
                                                              const GemmEpi e) {
    static_assert(MR == 32 || MR == 64, "rows per block");
    constexpr int MT = MR / 16;            // 16-row MFMA tiles
    constexpr int NW = kGemmThreads / 64;  // waves
    constexpr int XW = MR / 8;             // waves that also load 8 activation rows per tile
    constexpr int kSlot = kTileBytes + MR * 128;
    // slot: weight tile (64 rows x 128 B), then activation tile (MR rows x 128 B)
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kGemmDepth][kSlot];
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, lr = l & 15, g = l >> 4;
    const int cw = w & 3;                  // column group: columns 16cw .. 16cw + 15
    const int ks = w >> 2;                 // K half of every tile: rows 32ks .. 32ks + 31
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

    // DMA lane offsets (loop-invariant). Wave w fills weight tile rows
    // 8w + l/8 and, for w < XW, activation rows 8w + l/8; lane l lands at
    // chunk position l % 8 of its row and fetches the data chunk the swizzle
    // puts there. Activation rows past M repeat row M-1 (in bounds; their
    // products are never stored).
    const bool xload = w < XW;
    uint32_t woff, xoff;
    {
        const int r = 8 * w + (l >> 3);
        woff = (uint32_t)(r * N * 2 + 16 * ((l & 7) ^ wswz(r)));
        const int xr = min(m0 + min(r, MR - 1), M - 1) - m0;   // row within this block
        xoff = (uint32_t)(xr * ldx * 2 + 16 * ((l & 7) ^ xswz(r)));
    }
    // kEpiBf16RowScale: the block's rows of e.sumsq ([M][nb] fp32, nb =
    // rank/64 <= kMaxNormBlocks) are copied into LDS by 4-byte DMA ahead of the
    // ring, so they are older than every tile load and the ring's waits cover
    // them; element idx of the copy is row idx / nb (rows past M repeat row
    // M-1, in bounds), column idx % nb.
    __shared__ float ss_lds[EPI == kEpiBf16RowScale ? MR * kMaxNormBlocks : 1];
    if constexpr (EPI == kEpiBf16RowScale) {
        const int nb = e.rank / 64;
        const uint8_t* sb = uniform_ptr(e.sumsq);
        for (int i = w; i * 64 < MR * nb; i += NW) {
            const int idx = 64 * i + l;
            const int r = min(min(idx / nb, MR - 1) + m0, M - 1);
            const uint32_t off = (uint32_t)((r * nb + idx % nb) * 4);
            const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr_of(ss_lds) + 256 * i);
            asm volatile("global_load_lds_dword %0, %1" ::"v"(off), "s"(sb), "{m0}"(dst) : "memory");
        }
    }
    auto issue = [&](int tile) {   // clamped to the last tile
        const int k0 = kbeg + 64 * min(tile, ntiles - 1);
        const uint8_t* wb = uniform_ptr(W + (int64_t)k0 * N + n0);
        const uint8_t* xb = uniform_ptr(X + (int64_t)m0 * ldx + k0);
        const uint32_t slot = lds_addr_of(ring[tile % kGemmDepth]);
        dma16_stream(wb, woff, __builtin_amdgcn_readfirstlane(slot + 1024 * w));
        if (xload) dma16_keep(xb, xoff, __builtin_amdgcn_readfirstlane(slot + kTileBytes + 1024 * w));
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
        if (xload)
            wait_vmem<(kGemmDepth - 2) * 2>();
        else
            wait_vmem<(kGemmDepth - 2) * 1>();
        lds_barrier();
        issue(tile + kGemmDepth - 1);
        const uint8_t* wt = ring[tile % kGemmDepth];
        const uint8_t* xt = wt + kTileBytes;
        {
            // B operand: W[k = 32ks + 8g + j][n0 + 16cw + lr], j = 0..7
            const int ch = 2 * cw + ((lr & 3) >> 1);
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
    // the second K half's sums (waves 4-7) join the first's through LDS,
    // in the ring once every wave is done with it
    __syncthreads();
    f32x4* const red = reinterpret_cast<f32x4*>(&ring[0][0]);
    if (ks == 1) {
#pragma unroll
        for (int mt = 0; mt < MT; mt++) red[(cw * MT + mt) * 64 + l] = acc[mt];
    }
    __syncthreads();
    if (ks == 0) {
#pragma unroll
        for (int mt = 0; mt < MT; mt++) acc[mt] += red[(cw * MT + mt) * 64 + l];
    }

    const int n = n0 + 16 * cw + lr;
    __shared__ float row_scale[MR];
    __shared__ int arrival;
    if constexpr (EPI == kEpiBf16RowScale) {
        // the RMSNorm factor of this block's rows, from the column blocks'
        // sums of squares (every wave's copy has landed: wait above, barrier)
        __syncthreads();
        if (tid < MR) {
            const int nb = e.rank / 64;
            float ss = 0.f;
            for (int j = 0; j < nb; j++) ss += ss_lds[tid * nb + j];
            row_scale[tid] = 1.0f / __builtin_sqrtf(ss / (float)e.rank + e.eps);
        }
        __syncthreads();
    }
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
        if (ks != 0 || mt >= mt_n) continue;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int m = m0 + 16 * mt + 4 * g + i;
            if (m >= M) continue;
            if constexpr (EPI == kEpiBf16) {
                reinterpret_cast<uint16_t*>(Y)[(int64_t)m * N + n] = bitcast<uint16_t>((__bf16)acc[mt][i]);
            } else if constexpr (EPI == kEpiBf16RowScale) {
                const float v = acc[mt][i] * row_scale[m - m0];
                reinterpret_cast<uint16_t*>(Y)[(int64_t)m * N + n] = bitcast<uint16_t>((__bf16)v);
            } else if constexpr (EPI == kEpiPartials) {
                reinterpret_cast<float*>(Y)[((int64_t)blockIdx.y * M + m) * N + n] = acc[mt][i];
            } else {
                // device-coherent: the summing workgroup may run on another XCD
                __hip_atomic_store(reinterpret_cast<float*>(Y) + ((int64_t)blockIdx.y * M + m) * N + n, acc[mt][i],
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    if constexpr (EPI == kEpiNormPrep) {
        // every store of this workgroup is acknowledged before it counts
        wait_vmem<0>();
        __syncthreads();
        int* const ctr = e.counters + blockIdx.z * (N / 64) + bx;
        if (tid == 0) arrival = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (arrival != (int)gridDim.y - 1) return;
        if (tid == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // last split: pass pp, thread t sums columns n0 + 4(t % 16) .. +4 of
        // row m0 + 32 pp + t / 16 over the splits, in split order, eight
        // 16-byte coherent loads at a time
        const int nsplit = gridDim.y;
        const int64_t plane4 = (int64_t)M * N / 4;   // f32x4 per split plane
        const int c4 = tid & 15;
        const int col = n0 + 4 * c4;
        const u32x2 gw = *reinterpret_cast<const u32x2*>(e.gamma + col);
        const float g0 = __builtin_bit_cast(float, gw.x << 16), g1 = __builtin_bit_cast(float, gw.x & 0xffff0000u);
        const float g2 = __builtin_bit_cast(float, gw.y << 16), g3 = __builtin_bit_cast(float, gw.y & 0xffff0000u);
#pragma unroll
        for (int pp = 0; pp < MR / 32; pp++) {
            const int m = m0 + 32 * pp + (tid >> 4);
            const bool live = m < M;
            const f32x4* src = reinterpret_cast<const f32x4*>(Y) + ((int64_t)min(m, M - 1) * N + col) / 4;
            f32x4 c = {0.f, 0.f, 0.f, 0.f};
            for (int s0 = 0; s0 < nsplit; s0 += 8) {
                const f32x4* ptr[8];
#pragma unroll
                for (int u = 0; u < 8; u++) ptr[u] = src + min(s0 + u, nsplit - 1) * plane4;
                f32x4 v[8];
                coherent_load_b128x8(v, ptr);
#pragma unroll
                for (int u = 0; u < 8; u++)
                    if (s0 + u < nsplit) c += v[u];
            }
            if (live)
                *reinterpret_cast<u32x2*>(e.cg + (int64_t)m * N + col) =
                    u32x2{pack_bf16x2(c[0] * g0, c[1] * g1), pack_bf16x2(c[2] * g2, c[3] * g3)};
            // sum of c^2 over the block's 64 columns: the 16 threads of the row
            float ss = (c[0] * c[0] + c[1] * c[1]) + (c[2] * c[2] + c[3] * c[3]);
#pragma unroll
            for (int off = 8; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
            if (live && c4 == 0) e.sumsq[(int64_t)m * (N / 64) + bx] = ss;
        }
    }
}

// Rows per block: 32 when the whole batch fits in one such block, else 64.
template <int EPI>
static hipError_t launch_skinny(int gx, int gy, const uint16_t* X, int ldx, const uint16_t* W, int N, int kper,
                                int M, void* Y, const uint16_t* W2, void* Y2, const GemmEpi& e, const Launch& l) {
    if (M <= 32)
        return launch_kernel(mfa_skinny_gemm_kernel<EPI, 32>, dim3(gx, gy, 1), dim3(kGemmThreads), l, X, ldx, W, N,
                             kper, M, Y, W2, Y2, e);
    return launch_kernel(mfa_skinny_gemm_kernel<EPI, 64>, dim3(gx, gy, (M + 63) / 64), dim3(kGemmThreads), l, X, ldx,
                         W, N, kper, M, Y, W2, Y2, e);
}

hipError_t launch_qproj_down(const QprojArgs& a, const Launch& l) {
    GemmEpi e{};
    e.gamma = a.rms_w;
    e.cg = a.chat;
    e.sumsq = a.sumsq;
    e.counters = a.counters;
    return launch_skinny<kEpiNormPrep>(a.rank / 64, a.ksplit, a.x, a.hidden, a.w_qa, a.rank, a.hidden / a.ksplit,
                                       a.batch, (void*)a.c_part, nullptr, nullptr, e, l);
}

hipError_t launch_qproj_up(const QprojArgs& a, const Launch& l) {
    GemmEpi e{};
    e.sumsq = a.sumsq;
    e.rank = a.rank;
    e.eps = a.eps;
    return launch_skinny<kEpiBf16RowScale>(a.nq / 64, 1, a.chat, a.rank, a.w_qb, a.nq, a.rank, a.batch,
                                           (void*)a.q_out, nullptr, nullptr, e, l);
}

hipError_t launch_kv_proj(const KvAppendArgs& a, const Launch& l) {
    float* kp = a.kv_part;
    float* vp = a.kv_part + (int64_t)a.ksplit * a.batch * kHeadDim;
    return launch_skinny<kEpiPartials>(2 * kHeadDim / 64, a.ksplit, a.x, a.hidden, a.w_k, kHeadDim,
                                       a.hidden / a.ksplit, a.batch, (void*)kp, a.w_v, (void*)vp, GemmEpi{}, l);
}

}  // namespace mfa
