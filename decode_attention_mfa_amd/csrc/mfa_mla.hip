// mfa_mla.hip -- decode attention over a latent KV cache, for the
// head-sharing comparison of the Step-3 summary card (Key points, ablations:
// MFA decodes faster than MLA and GQA).
//
// The latent reading: every token stores one row c_t of kLatent = 512
// elements, which every one of the 64 query heads uses both as its key and as
// its value. The key and value up-projections are taken as absorbed into the
// query (q is given in the latent space, 512 wide per head) and into the
// output projection (the output stays in the latent space), so the attention
// computed here is
//     s_ht = scale * <q_h, c_t>,  out_h = sum_t softmax_t(s_h) c_t,
// multi-query attention with 512-wide heads over one shared row per token.
// With an FP8 latent a token costs the same 512 cache bytes as MFA's K and V
// rows, and twice MFA's matrix work: the comparison isolates the arithmetic.
//
// One workgroup (eight waves) takes 32 of the 64 heads of one (sequence,
// chunk); the two head groups of a (sequence, chunk) get block indices 8
// apart in a group of 16, so that the round-robin dispatch puts them on one
// XCD, where the second reads the latent rows from L2. Per 64-token step the
// latent tile (32 KB of E4M3 codes) streams into a four-slot LDS ring by
// direct DMA; each wave scores 16 tokens against 16 heads (bf16 MFMAs on the
// widened codes, Q held in registers), the softmax keeps a running maximum
// per head and rescales the output accumulators when it rises, and each wave
// then accumulates 64 of the 512 output columns for the 32 heads from the
// transposed tile (the same LDS bytes the scores read). Two barriers per
// step; two waves per SIMD overlap each other's MFMA and VALU work. Pieces are merged by mfa_mla_combine_kernel.
#include "mfa_device.h"
#include "mfa_internal.h"

namespace mfa {

namespace {

constexpr int kRowB = kLatent;          // bytes per FP8 latent row
constexpr int kSlot = kStep * kRowB;    // one step's tile: 32 KB
constexpr int kRing = 4;                // tiles in the ring
constexpr int kHg = 32;                 // heads per workgroup
constexpr int kDmaPerStep = kSlot / (512 * 16);   // 16-byte DMA instructions per thread and step (4)

// 16-byte chunk c of row r of a tile sits at chunk position c ^ (r & 31): the
// score reads (16 rows, one chunk column) and the transposed reads (8 rows)
// then fall in distinct bank groups.
__device__ __forceinline__ int lswz(int r) { return r & 31; }
// P tile: 32 heads x 64 tokens bf16, 128-byte rows
__device__ __forceinline__ int pswz32(int h) { return h & 7; }

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 bytes per lane from global memory into LDS (lane i lands at lds_dst +
// 16 i; lds_dst wave-uniform, through M0); inline asm so that later LDS
// accesses are not ordered behind it (the ring's waits order the reads).
__device__ __forceinline__ void mla_dma(const void* sbase, uint32_t voff, uint32_t lds_dst) {
    asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "{m0}"(lds_dst) : "memory");
}
// The same, first of a step: sbase comes from v_readfirstlane (a VALU write
// of SGPRs), and a memory instruction may read such SGPRs only five wait
// states later, which the compiler does not ensure for an asm block; the
// s_nop inside the block does.
__device__ __forceinline__ void mla_dma_first(const void* sbase, uint32_t voff, uint32_t lds_dst) {
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "{m0}"(lds_dst) : "memory");
}

template <int N>
__device__ __forceinline__ void mla_wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void mla_lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ const uint8_t* mla_uniform(const uint8_t* ptr) {
    const uint64_t u = (uint64_t)(uintptr_t)ptr;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

}  // namespace

// Grid: round_up(batch * n_chunk, 8) * 2 blocks of 512 threads (eight
// waves, two per SIMD, so that one wave's MFMAs run while the other does its
// VALU work or waits). Block x: work item wi = 8 (x / 16) + x % 8 is (row b,
// chunk c) = (wi / n_chunk, wi % n_chunk); head group hg = (x % 16) / 8
// takes heads 32 hg .. 32 hg + 31. Wave v scores tokens 16 (v % 4) .. +15
// of each step against head tile v / 4 (16 heads) and accumulates output
// columns 64 v .. 64 v + 63 of all 32 heads.
template <bool PAGED>
__global__ __launch_bounds__(512) void mfa_mla_kernel(const AttnArgs p) {
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kRing * kSlot];
    __shared__ __attribute__((aligned(16))) uint8_t pbuf[kHg * kStep * 2];
    __shared__ float xmax[4][kHg];   // [token block][head]: the block's maximum
    __shared__ float xsum[4][kHg];   // [token block][head]: the block's share of the sum of P

    const int tid = threadIdx.x;
    const int v = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tw = v & 3, ht = v >> 2;   // score role: token block, head tile
    const int l = tid & 63, lr = l & 15, g = l >> 4;
    const int grp = blockIdx.x >> 4, r16 = blockIdx.x & 15;
    const int wi = grp * 8 + (r16 & 7);
    if (wi >= p.batch * p.n_chunk) return;
    const int hb = kHg * (r16 >> 3);
    const int b = wi / p.n_chunk, c = wi - b * p.n_chunk;
    const int L = seq_len(p.kv, b);
    const int t_begin = c * p.chunk;
    uint16_t* const ob = p.out + ((int64_t)b * kHeads + hb) * kLatent;   // this group's 32 output rows
    if (t_begin >= L) {
        if (c == 0) {   // empty sequence: out = 0, lse = -inf
            for (int i = tid; i < kHg * kLatent / 8; i += 512) reinterpret_cast<u32x4*>(ob)[i] = u32x4{0, 0, 0, 0};
            if (p.lse_out && tid < kHg) p.lse_out[b * kHeads + hb + tid] = -__builtin_inff();
        }
        return;
    }
    const int t_end = min(L, t_begin + p.chunk);
    const int nsteps = (t_end - t_begin + kStep - 1) / kStep;
    const int nparts = (L + p.chunk - 1) / p.chunk;

    // ---- the ring: step s into slot s % kRing; rows past the piece's end
    // repeat its last row (in bounds; their scores are masked). Loads past the
    // last step repeat it, so that every wait sees the same number of younger
    // loads.
    const uint8_t* const kv = mla_uniform(p.kv.k);
    auto issue = [&](int s) {
        const int sl = min(s, nsteps - 1);
        const int t0 = t_begin + sl * kStep;
        int64_t base;
        if constexpr (PAGED) {
            base = (int64_t)p.kv.page_table[(int64_t)b * p.kv.pt_stride + t0 / kPage] * kPage;
        } else {
            base = (int64_t)b * p.kv.kv_stride + t0;
        }
        const uint8_t* src = mla_uniform(kv + base * kRowB);
        const int last = t_end - 1 - t0;
        const uint32_t slot = lds_u32(ring + (s % kRing) * kSlot);
#pragma unroll
        for (int i = 0; i < kDmaPerStep; i++) {
            // instruction i of wave v fills rows 16 i + 2 v + l / 32, chunk position l % 32
            const int row = 16 * i + 2 * v + (l >> 5);
            const int srow = min(row, last);
            const uint32_t voff = (uint32_t)(srow * kRowB + 16 * ((l & 31) ^ lswz(row)));
            const uint32_t dst = __builtin_amdgcn_readfirstlane(slot + 8192 * i + 1024 * v);
            if (i == 0)
                mla_dma_first(src, voff, dst);
            else
                mla_dma(src, voff, dst);
        }
    };

    f32x4 o[2][4];   // O[16 h2 + 4 g + i][64 v + 16 dt + lr]
#pragma unroll
    for (int h2 = 0; h2 < 2; h2++)
#pragma unroll
        for (int dt = 0; dt < 4; dt++) o[h2][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-__builtin_inff(), -__builtin_inff()};   // running maximum of head 16 h2 + lr (base 2)
    float l_run = 0.f;   // this lane's share of the sum of P of head 16 ht + lr

    // Q of head tile ht as MFMA B operands: qop[ks] = q[hb + 16 ht + lr][32 ks + 8 g + 0..7]
    // (loaded before the ring's first DMA: the compiler's waits for them then
    // do not wait for the ring)
    bf16x8 qop[16];
    {
        const uint16_t* qb = p.q + ((int64_t)b * kHeads + hb + 16 * ht + lr) * kLatent;
#pragma unroll
        for (int ks = 0; ks < 16; ks++) qop[ks] = *reinterpret_cast<const bf16x8*>(qb + 32 * ks + 8 * g);
    }
    for (int s = 0; s < kRing - 1; s++) issue(s);
    // tile 0 has landed once at most the two younger tiles' loads are in
    // flight; the barrier shows every thread's part
    mla_wait_vmem<2 * kDmaPerStep>();
    mla_lds_barrier();
    for (int s = 0; s < nsteps; s++) {
        const uint8_t* const tile = ring + (s % kRing) * kSlot;

        // scores of tokens 16 tw + 4 g + i against heads 16 ht + lr
        f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
        {
            const int row = 16 * tw + lr;
#pragma unroll
            for (int ks = 0; ks < 16; ks++) {
                const int ch = 2 * ks + (g >> 1);
                const u32x2 kk = *reinterpret_cast<const u32x2*>(tile + row * kRowB + 16 * (ch ^ lswz(row)) + 8 * (g & 1));
                sc = mfma16(e4m3x8_to_bf16x8(kk.x, kk.y), qop[ks], sc);
            }
        }
        const int tq = t_begin + s * kStep + 16 * tw + 4 * g;   // token of element i = 0
#pragma unroll
        for (int i = 0; i < 4; i++) sc[i] = tq + i < t_end ? sc[i] * p.score_scale : -__builtin_inff();
        {
            float m = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
            m = fmaxf(m, __shfl_xor(m, 16));
            m = fmaxf(m, __shfl_xor(m, 32));
            if (g == 0) xmax[tw][16 * ht + lr] = m;
        }
        // barrier A: every token block's maxima; every wave is done with step
        // s - 1 (its P and its tile slot, which the loads of step s + 3 refill)
        mla_lds_barrier();
        issue(s + kRing - 1);
        float alpha[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; h2++) {
            const int h = 16 * h2 + lr;
            const float ms = fmaxf(fmaxf(xmax[0][h], xmax[1][h]), fmaxf(xmax[2][h], xmax[3][h]));
            const float mn = fmaxf(m_run[h2], ms);
            alpha[h2] = __builtin_amdgcn_exp2f(m_run[h2] - mn);   // 0 on the first step
            m_run[h2] = mn;
        }
        {
            const float mh = ht ? m_run[1] : m_run[0];
            const float ah = ht ? alpha[1] : alpha[0];
            float ps[4];
#pragma unroll
            for (int i = 0; i < 4; i++) ps[i] = __builtin_amdgcn_exp2f(sc[i] - mh);
            l_run = l_run * ah + ((ps[0] + ps[1]) + (ps[2] + ps[3]));
            // P[h][tok] as bf16, tok = 16 tw + 4 g + i: chunk 2 tw + g / 2, elements 4 (g % 2) + i
            const int h = 16 * ht + lr;
            *reinterpret_cast<u32x2*>(pbuf + h * 128 + 16 * ((2 * tw + (g >> 1)) ^ pswz32(h)) + 8 * (g & 1)) =
                u32x2{pack_bf16x2(ps[0], ps[1]), pack_bf16x2(ps[2], ps[3])};
        }
        // the output rows of this lane are heads 16 h2 + 4 g + i: their alpha
        // from the lanes that hold those heads
#pragma unroll
        for (int h2 = 0; h2 < 2; h2++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float a = __shfl(alpha[h2], 4 * g + i);
#pragma unroll
                for (int dt = 0; dt < 4; dt++) o[h2][dt][i] *= a;
            }
        // barrier B: P visible, and tile s + 1 (landed once at most the two
        // younger tiles' loads are in flight) for the next step's scores
        mla_wait_vmem<2 * kDmaPerStep>();
        mla_lds_barrier();

        // O[16 h2 + 4 g + i][64 v + 16 dt + lr] += P . C, the tile read
        // transposed: lane j of a 16-lane group points at row r0 + j / 2,
        // bytes 8 (j % 2) .. +7 of chunk 4 v + dt, and receives column j of
        // that chunk for rows r0 .. r0 + 7
#pragma unroll
        for (int kk = 0; kk < 2; kk++) {
            bf16x8 pa[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; h2++) {
                const int h = 16 * h2 + lr;
                pa[h2] = *reinterpret_cast<const bf16x8*>(pbuf + h * 128 + 16 * ((4 * kk + g) ^ pswz32(h)));
            }
            const int row = 32 * kk + 8 * g + (lr >> 1);
#pragma unroll
            for (int dt = 0; dt < 4; dt++) {
                const uint8_t* a = tile + row * kRowB + 16 * ((4 * v + dt) ^ lswz(row)) + 8 * (lr & 1);
                const i32x2 vr = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(a));
                const bf16x8 vb = e4m3x8_to_bf16x8((uint32_t)vr.x, (uint32_t)vr.y);
                o[0][dt] = mfma16(pa[0], vb, o[0][dt]);
                o[1][dt] = mfma16(pa[1], vb, o[1][dt]);
            }
        }
    }
    mla_wait_vmem<0>();   // the repeated loads past the last step

    // ---- sums of P per head (lanes -> token block -> workgroup), normalisation
    {
        float sv = l_run;
        sv += __shfl_xor(sv, 16);
        sv += __shfl_xor(sv, 32);
        if (g == 0) xsum[tw][16 * ht + lr] = sv;
    }
    __syncthreads();
#pragma unroll
    for (int h2 = 0; h2 < 2; h2++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int h = 16 * h2 + 4 * g + i;
            const float tot = ((xsum[0][h] + xsum[1][h]) + xsum[2][h]) + xsum[3][h];
            const float inv = p.v_scale / tot;
#pragma unroll
            for (int dt = 0; dt < 4; dt++) o[h2][dt][i] *= inv;
        }
    // base-2 log-sum-exp of head 16 h2 + lr (lanes g = 0 of wave 0 write it)
    float lse2[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; h2++) {
        const int h = 16 * h2 + lr;
        const float tot = ((xsum[0][h] + xsum[1][h]) + xsum[2][h]) + xsum[3][h];
        lse2[h2] = m_run[h2] + __builtin_amdgcn_logf(tot);
    }

    // ---- the rows, as bf16, through LDS (ring slot 0, free now): element
    // (h, col) at byte h * 1024 + 2 * (col ^ 16 * ((h >> 2) & 3)) (the XOR
    // spreads the four rows one ds_write_b16 covers over the banks), then
    // 16-byte stores of whole rows: the final output for a one-piece
    // sequence, else this piece's partial slot
    uint8_t* const stage = ring;
#pragma unroll
    for (int h2 = 0; h2 < 2; h2++)
#pragma unroll
        for (int dt = 0; dt < 4; dt++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int h = 16 * h2 + 4 * g + i;
                const int col = 64 * v + 16 * dt + lr;
                *reinterpret_cast<uint16_t*>(stage + h * 1024 + 2 * (col ^ (16 * ((h >> 2) & 3)))) =
                    bitcast<uint16_t>((__bf16)o[h2][dt][i]);
            }
    __syncthreads();
    const bool single = nparts == 1;
    const int64_t pidx = (int64_t)b * p.n_chunk + c;
    uint16_t* const dst = single ? ob : reinterpret_cast<uint16_t*>(p.part_o) + (pidx * kHeads + hb) * kLatent;
#pragma unroll
    for (int rr = 0; rr < kHg * kLatent / 8 / 512; rr++) {
        const int k = tid + 512 * rr, row = k >> 6, c8 = 8 * (k & 63);
        const u32x4 val = *reinterpret_cast<const u32x4*>(stage + row * 1024 + 2 * (c8 ^ (16 * ((row >> 2) & 3))));
        __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(dst + row * kLatent + c8));
    }
    if (v == 0 && g == 0) {
#pragma unroll
        for (int h2 = 0; h2 < 2; h2++) {
            const int h = hb + 16 * h2 + lr;
            if (single) {
                if (p.lse_out) p.lse_out[b * kHeads + h] = lse2[h2] * kLn2;
            } else {
                p.part_lse[pidx * kHeads + h] = lse2[h2];
            }
        }
    }
}

// Merge of the pieces of every sequence with more than one: one wave per
// (row, head), lane t owning columns 8 t .. 8 t + 7; pieces in index order:
//   M = max_c lse2_c, W_c = 2^(lse2_c - M), out = sum_c W_c o_c / sum_c W_c,
//   lse = (M + log2 sum_c W_c) ln 2.
__global__ __launch_bounds__(64) void mfa_mla_combine_kernel(const AttnArgs p) {
    const int b = blockIdx.x / kHeads, h = blockIdx.x % kHeads;
    const int L = seq_len(p.kv, b);
    const int nc = (L + p.chunk - 1) / p.chunk;
    if (nc <= 1) return;   // written by the attention kernel
    const int t = threadIdx.x;
    const int64_t base = (int64_t)b * p.n_chunk;
    float M = -__builtin_inff();
    for (int cc = 0; cc < nc; cc++) M = fmaxf(M, p.part_lse[(base + cc) * kHeads + h]);
    f32x4 a0 = f32x4{0.f, 0.f, 0.f, 0.f}, a1 = a0;
    float s = 0.f;
    for (int cc = 0; cc < nc; cc++) {
        const float wc = __builtin_amdgcn_exp2f(p.part_lse[(base + cc) * kHeads + h] - M);
        const u32x4 d = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.part_o) +
                                                        ((base + cc) * kHeads + h) * kLatent + 8 * t);
        const f32x4 v0 = f32x4{__builtin_bit_cast(float, d.x << 16), __builtin_bit_cast(float, d.x & 0xffff0000u),
                               __builtin_bit_cast(float, d.y << 16), __builtin_bit_cast(float, d.y & 0xffff0000u)};
        const f32x4 v1 = f32x4{__builtin_bit_cast(float, d.z << 16), __builtin_bit_cast(float, d.z & 0xffff0000u),
                               __builtin_bit_cast(float, d.w << 16), __builtin_bit_cast(float, d.w & 0xffff0000u)};
        s += wc;
        a0 += wc * v0;
        a1 += wc * v1;
    }
    const float inv = 1.f / s;
    const u32x4 out = u32x4{pack_bf16x2(a0[0] * inv, a0[1] * inv), pack_bf16x2(a0[2] * inv, a0[3] * inv),
                            pack_bf16x2(a1[0] * inv, a1[1] * inv), pack_bf16x2(a1[2] * inv, a1[3] * inv)};
    *reinterpret_cast<u32x4*>(p.out + ((int64_t)b * kHeads + h) * kLatent + 8 * t) = out;
    if (p.lse_out && t == 0) p.lse_out[b * kHeads + h] = (M + __builtin_amdgcn_logf(s)) * kLn2;
}

hipError_t launch_mla(const AttnArgs& a, bool paged, const Launch& l) {
    const int items = (a.batch * a.n_chunk + 7) / 8 * 8;
    const dim3 grid(2 * items), block(512);
    return paged ? launch_kernel(mfa_mla_kernel<true>, grid, block, l, a)
                 : launch_kernel(mfa_mla_kernel<false>, grid, block, l, a);
}

hipError_t launch_mla_combine(const AttnArgs& a, const Launch& l) {
    return launch_kernel(mfa_mla_combine_kernel, dim3(a.batch * kHeads), dim3(64), l, a);
}

}  // namespace mfa
