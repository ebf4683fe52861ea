// mfa_attn.hip -- decode attention of Multi-Matrix Factorization Attention
// on CDNA4 (gfx950): 64 query heads against one shared K head and one shared
// V head of dimension 256 ("Step-3 is Large yet Affordable", Key points),
// split into KV chunks whose partial softmax results are merged by the
// log-sum-exp identity (Flash-Decoding, cited by title on the DeepSeek-V4
// references).
//
// One workgroup (4 wave64s) owns one (sequence, chunk). It walks the chunk in
// steps of 64 tokens (= one cache page):
//   QK   wave w scores tokens 16w..16w+15 of the step against all 64 heads:
//        S^T[16 tok x 64 heads] = K[16 x 256] . Q^T, the K rows going straight
//        from HBM into MFMA A-operand registers (FP8 codes converted to bf16
//        in registers; E4M3 values are exact in bf16), Q held in registers as
//        B operands for the whole chunk. Each cached K byte feeds 64 heads.
//   max  per-head step maxima meet in LDS; every wave derives the same new
//        running max, so all rows of P share one reference.
//   P    exp2 of the scaled scores, rounded to bf16, written to LDS.
//   PV   wave w owns output columns 64w..64w+63 of all 64 heads:
//        O[64 x 64] += P[64 x 64 tok] . V[64 tok x 64]; its V slice goes
//        HBM -> registers -> LDS and comes back transposed with
//        ds_read_b64_tr_b8 / _b16 as the MFMA B operand.
// The next step's K and V are loaded while the current step computes.
//
// Scores are kept in the base-2 domain: s2 = s * log2(e), exp -> exp2.
// Output of a chunk: if the sequence has one chunk, the final bf16 output and
// lse; otherwise the chunk-normalised output (fp32) and its base-2 lse in the
// workspace, merged by mfa_combine_kernel.
#include <type_traits>

#include "mfa_device.h"
#include "mfa_internal.h"

namespace mfa {

// V slice rows in LDS: 64 tokens x (64 columns * elem) bytes, 16-byte chunks
// XOR-swizzled per row so that the transposed reads hit distinct banks.
__device__ __forceinline__ int vswz_fp8(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int vswz_bf16(int row) { return ((row >> 1) & 3) << 1; }
// P rows in LDS: 64 heads x 64 tokens bf16 (128 B), chunk swizzle by head.
__device__ __forceinline__ int pswz(int h) { return (h >> 1) & 7; }

// K rows of a wave's 16 tokens in LDS: 16-byte chunk c of row t is stored at
// chunk position c ^ (t & 15), so the 16 lanes reading one chunk column of 16
// rows hit 16 distinct bank groups.
__device__ __forceinline__ int kswz(int row) { return row & 15; }

// LDS stores issued as inline asm. The compiler treats any plain LDS store as
// possibly overwriting bytes an LDS DMA is still filling and would wait for
// every load in flight first; these stores go to buffers no DMA touches.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void lds_store_b64(void* p, u32x2 v) {
    asm volatile("ds_write_b64 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_store_b32(void* p, uint32_t v) {
    asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
// Workgroup barrier for LDS traffic only: this wave's LDS operations complete,
// then s_barrier. Unlike __syncthreads() it does not wait for the loads
// still streaming into the LDS ring.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16 bytes per lane from global memory straight into LDS: lane i's bytes land
// at lds_dst + 16*i (lds_dst is wave-uniform, passed in M0). Issued as inline
// asm so that the compiler does not treat every later LDS access as possibly
// overlapping the transfer (it would wait for all loads in flight before each
// one); the ring's own waits (wait_vmem) order the reads instead. No register
// is written, and the "memory" clobber keeps earlier reads of the slot ahead.
__device__ __forceinline__ void dma_b128(const void* gsrc, uint32_t lds_dst) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 ::"v"(gsrc), "s"(lds_dst) : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are in flight.
// The "memory" clobber keeps the compiler from moving LDS reads of the
// DMA-filled ring above the wait.
template <int N>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}


template <bool FP8, bool PAGED>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void mfa_attn_split_kernel(const AttnArgs p) {
    constexpr int ELEM = FP8 ? 1 : 2;
    constexpr int ROWB = kHeadDim * ELEM;          // bytes per cached row
    constexpr int VROWB = 64 * ELEM;               // bytes per row of a wave's V slice
    constexpr int VSLOT = 64 * VROWB;              // one step of a wave's V slice
    constexpr int KSLOT = 16 * ROWB;               // one step of a wave's K rows
    constexpr int NK = KSLOT / 1024;               // 1 KB DMA instructions per step
    constexpr int NV = VSLOT / 1024;
    // vector-memory instructions a wave issues per step (all DMA into LDS)
    constexpr int OPS_PER_STEP = NK + NV;
    // steps in flight (current + prefetched): 3 x 32 KB for FP8, 2 x 64 KB for bf16
    constexpr int RING = FP8 ? 3 : 2;

    // One LDS object per ring slot: the compiler then sees that a read of one
    // slot cannot alias the DMA still filling another, and waits only for the
    // DMA of the slot it reads.
    __shared__ __attribute__((aligned(1024))) uint8_t kr0[4][KSLOT], kr1[4][KSLOT], kr2[4][KSLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t vr0[4][VSLOT], vr1[4][VSLOT], vr2[4][VSLOT];
    __shared__ __attribute__((aligned(16))) uint8_t plds_all[2][kHeads * 64 * 2];
    __shared__ __attribute__((aligned(16))) float xchg[4][kHeads];
    __shared__ __attribute__((aligned(16))) float alpha_lds[kHeads];
    __shared__ int flags_all[2][4];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int lr = l & 15;
    const int g = l >> 4;
    auto kring = [&](auto slot) -> uint8_t* {
        if constexpr (decltype(slot)::value == 0) return kr0[w];
        else if constexpr (decltype(slot)::value == 1) return kr1[w];
        else return kr2[w];
    };
    auto vring = [&](auto slot) -> uint8_t* {
        if constexpr (decltype(slot)::value == 0) return vr0[w];
        else if constexpr (decltype(slot)::value == 1) return vr1[w];
        else return vr2[w];
    };

    const int b = blockIdx.x / p.n_chunk;
    const int c = blockIdx.x - b * p.n_chunk;
    const int L = seq_len(p.kv, b);
    const int t_begin = c * p.chunk;

    if (t_begin >= L) {
        if (c == 0) {  // empty sequence: out = 0, lse = -inf
            uint16_t* ob = p.out + (int64_t)b * kHeads * kHeadDim;
            for (int i = tid; i < kHeads * kHeadDim / 8; i += 256)
                reinterpret_cast<u32x4*>(ob)[i] = u32x4{0, 0, 0, 0};
            if (p.lse_out && tid < kHeads)
                p.lse_out[b * kHeads + tid] = -__builtin_inff();
        }
        return;
    }
    const int t_end = min(L, t_begin + p.chunk);
    const int nsteps = (t_end - t_begin + kStep - 1) / kStep;
    const int last_s = nsteps - 1;
    const bool single = (L + p.chunk - 1) / p.chunk == 1;

    // ---- Q as B operands: qop[ht][ks] holds Q[16ht + lr][d(ks, g, 0..7)] with
    // d(ks, g, j) = 64*(ks/2) + 16*g + 8*(ks%2) + j, the same d order the K
    // A operands use below.
    bf16x8 qop[4][8];
    {
        const uint16_t* qb = p.q + (int64_t)b * kHeads * kHeadDim;
#pragma unroll
        for (int ht = 0; ht < 4; ht++)
#pragma unroll
            for (int ks = 0; ks < 8; ks++) {
                const int d0 = 64 * (ks >> 1) + 16 * g + 8 * (ks & 1);
                qop[ht][ks] = *reinterpret_cast<const bf16x8*>(qb + (16 * ht + lr) * kHeadDim + d0);
            }
    }
    // An empty asm that reads every Q register makes the compiler wait for the
    // Q loads here, where nothing else is in flight; afterwards it has no load
    // of its own outstanding and adds no waits of its own to the ring's.
#pragma unroll
    for (int ht = 0; ht < 4; ht++)
        asm volatile("" ::"v"(qop[ht][0]), "v"(qop[ht][1]), "v"(qop[ht][2]), "v"(qop[ht][3]),
                     "v"(qop[ht][4]), "v"(qop[ht][5]), "v"(qop[ht][6]), "v"(qop[ht][7]));

    // ---- issue the loads of step s (clamped to the last step, whose rows then
    // hit in L2): this wave's 16 K rows and its V columns 64w..64w+63 of all 64
    // tokens, both straight into its LDS ring slot. A DMA instruction writes
    // lane i's 16 bytes at dst + 16*i, so each lane fetches the piece that
    // belongs at that swizzled position.
    auto issue_step = [&](int s, auto slot) {
        const int t0 = t_begin + min(s, last_s) * kStep;
        const int last = t_end - 1 - t0;                 // last valid local token (>= 0)
        const int64_t base = kv_step_base<PAGED>(p.kv, b, t0);
        uint8_t* ks = kring(slot);
#pragma unroll
        for (int i = 0; i < NK; i++) {
            constexpr int RPI = 1024 / ROWB;             // rows per instruction
            const int row = RPI * i + l / (ROWB / 16);
            const int ch = (l % (ROWB / 16)) ^ kswz(row);
            const uint8_t* src = p.kv.k + (base + min(16 * w + row, last)) * ROWB + 16 * ch;
            dma_b128(src, lds_addr(ks + 1024 * i));
        }
        uint8_t* vs = vring(slot);
#pragma unroll
        for (int i = 0; i < NV; i++) {
            int row, ch;
            if constexpr (FP8) {
                row = 16 * i + (l >> 2);
                ch = (l & 3) ^ vswz_fp8(row);
            } else {
                row = 8 * i + (l >> 3);
                ch = (l & 7) ^ vswz_bf16(row);
            }
            const uint8_t* src = p.kv.v + (base + min(row, last)) * ROWB + 64 * w * ELEM + 16 * ch;
            dma_b128(src, lds_addr(vs + 1024 * i));
        }
    };

    // running state (QK layout: heads 16ht + lr)
    float mq[4];        // reference maxima (base 2)
    float lq[4];        // partial softmax denominators
    f32x4 o[4][4];      // O[16ht + 4g + i][64w + 16dt + lr]
#pragma unroll
    for (int ht = 0; ht < 4; ht++) {
        mq[ht] = -__builtin_inff();
        lq[ht] = 0.f;
#pragma unroll
        for (int dt = 0; dt < 4; dt++) o[ht][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    auto compute_step = [&](int s, auto slot) {
        const int t0 = t_begin + s * kStep;
        // K and V of step s have landed once at most the RING-1 younger steps'
        // loads are in flight
        wait_vmem<(RING - 1) * OPS_PER_STEP>();
        // P and the vote flags alternate between two buffers by step parity:
        // with one barrier per step a wave may write step s+1 while another
        // still reads step s.
        uint8_t* plds = plds_all[s & 1];
        int* flags = flags_all[s & 1];
        const uint8_t* vlds = vring(slot);
        const uint8_t* klds = kring(slot) + lr * ROWB;   // this lane's K row
        auto kpiece = [&](int c) {
            return *reinterpret_cast<const u32x4*>(klds + 16 * (c ^ kswz(lr)));
        };
        // (1) scores S^T[token 4g+i][head 16ht+lr] for this wave's 16 tokens
        f32x4 sc[4];
#pragma unroll
        for (int ht = 0; ht < 4; ht++) sc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (FP8) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const u32x4 kr = kpiece(4 * i + g);          // bytes 64i + 16g .. +16
                const bf16x8 a0 = e4m3x8_to_bf16x8(kr.x, kr.y);
                const bf16x8 a1 = e4m3x8_to_bf16x8(kr.z, kr.w);
#pragma unroll
                for (int ht = 0; ht < 4; ht++) {
                    sc[ht] = mfma16(a0, qop[ht][2 * i], sc[ht]);
                    sc[ht] = mfma16(a1, qop[ht][2 * i + 1], sc[ht]);
                }
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < 8; ks++) {
                // bytes 128(ks/2) + 32g + 16(ks%2) .. +16
                const bf16x8 a = bitcast<bf16x8>(kpiece(8 * (ks >> 1) + 2 * g + (ks & 1)));
#pragma unroll
                for (int ht = 0; ht < 4; ht++) sc[ht] = mfma16(a, qop[ht][ks], sc[ht]);
            }
        }
        // (2) mask tokens past the chunk end (last step of a chunk only)
        if (t_end - t0 < kStep) {
            const int valid = t_end - t0 - (16 * w + 4 * g);   // rows i < valid are real tokens
#pragma unroll
            for (int ht = 0; ht < 4; ht++)
#pragma unroll
                for (int i = 0; i < 4; i++)
                    if (i >= valid) sc[ht][i] = -__builtin_inff();
        }
        // (3) optimistic P against the current reference maxima. A reference
        // is kept until some score exceeds it by more than kTau (base 2), so
        // P <= 2^kTau; the wave votes whether that happened.
        bool over = false;
#pragma unroll
        for (int ht = 0; ht < 4; ht++) {
            const float m = fmaxf(fmaxf(sc[ht][0], sc[ht][1]), fmaxf(sc[ht][2], sc[ht][3]));
            over |= m * p.score_scale > mq[ht] + kTau;
        }
        const bool wave_over = __builtin_amdgcn_ballot_w64(over) != 0;
        float lstep[4];
        auto write_p = [&]() {
#pragma unroll
            for (int ht = 0; ht < 4; ht++) {
                float pr[4];
                float sum = 0.f;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    pr[i] = bf16_round(__builtin_amdgcn_exp2f(__builtin_fmaf(sc[ht][i], p.score_scale, -mq[ht])));
                    sum += pr[i];
                }
                lstep[ht] = sum;
                const int h = 16 * ht + lr;
                const int ch = (2 * w + (g >> 1)) ^ pswz(h);
                lds_store_b64(plds + h * 128 + 16 * ch + 8 * (g & 1),
                              u32x2{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])});
            }
        };
        if (!wave_over) write_p();
        if (l == 0) lds_store_b32(&flags[w], wave_over ? 1u : 0u);
        lds_barrier();
        const bool any_over = (flags[0] | flags[1] | flags[2] | flags[3]) != 0;
        if (!any_over) {
#pragma unroll
            for (int ht = 0; ht < 4; ht++) lq[ht] += lstep[ht];
        } else {
            // (4) rare: new references from every wave's maxima; rescale the
            // denominators here and the outputs through alpha_lds; redo P
#pragma unroll
            for (int ht = 0; ht < 4; ht++) {
                float m = fmaxf(fmaxf(sc[ht][0], sc[ht][1]), fmaxf(sc[ht][2], sc[ht][3]));
                m = fmaxf(m, __shfl_xor(m, 16));
                m = fmaxf(m, __shfl_xor(m, 32));
                if (g == 0) lds_store_b32(&xchg[w][16 * ht + lr], __builtin_bit_cast(uint32_t, m * p.score_scale));
            }
            lds_barrier();
#pragma unroll
            for (int ht = 0; ht < 4; ht++) {
                const int h = 16 * ht + lr;
                const float m = fmaxf(mq[ht], fmaxf(fmaxf(xchg[0][h], xchg[1][h]), fmaxf(xchg[2][h], xchg[3][h])));
                const float a = __builtin_amdgcn_exp2f(mq[ht] - m);
                lq[ht] *= a;
                mq[ht] = m;
                if (w == 0 && g == 0) lds_store_b32(&alpha_lds[h], __builtin_bit_cast(uint32_t, a));
            }
            write_p();
#pragma unroll
            for (int ht = 0; ht < 4; ht++) lq[ht] += lstep[ht];
            lds_barrier();
#pragma unroll
            for (int ht = 0; ht < 4; ht++) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(&alpha_lds[16 * ht + 4 * g]);
#pragma unroll
                for (int dt = 0; dt < 4; dt++) o[ht][dt] *= a;
            }
        }
        // (5) O[64 heads][64w..64w+63] += P[64 x 64 tok] . V[64 tok x 64]
#pragma unroll
        for (int kk = 0; kk < 2; kk++) {
            bf16x8 pa[4];
#pragma unroll
            for (int ht = 0; ht < 4; ht++) {
                const int h = 16 * ht + lr;
                pa[ht] = *reinterpret_cast<const bf16x8*>(plds + h * 128 + 16 * ((4 * kk + g) ^ pswz(h)));
            }
#pragma unroll
            for (int dt = 0; dt < 4; dt++) {
                bf16x8 vb;
                if constexpr (FP8) {
                    const int row = 32 * kk + 8 * g + (lr >> 1);
                    const uint8_t* a = vlds + row * VROWB + 16 * (dt ^ vswz_fp8(row)) + 8 * (lr & 1);
                    const i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (__attribute__((address_space(3))) i32x2*)(a));
                    vb = e4m3x8_to_bf16x8((uint32_t)raw.x, (uint32_t)raw.y);
                } else {
                    const int ch = 2 * dt + ((lr & 3) >> 1);
                    const int row0 = 32 * kk + 8 * g + (lr >> 2);
                    const int row1 = row0 + 4;
                    const uint8_t* a0 = vlds + row0 * VROWB + 16 * (ch ^ vswz_bf16(row0)) + 8 * (lr & 1);
                    const uint8_t* a1 = vlds + row1 * VROWB + 16 * (ch ^ vswz_bf16(row1)) + 8 * (lr & 1);
                    const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4*)(a0));
                    const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4*)(a1));
                    const u32x2 u0 = bitcast<u32x2>(r0);
                    const u32x2 u1 = bitcast<u32x2>(r1);
                    vb = bitcast<bf16x8>(u32x4{u0.x, u0.y, u1.x, u1.y});
                }
#pragma unroll
                for (int ht = 0; ht < 4; ht++) o[ht][dt] = mfma16(pa[ht], vb, o[ht][dt]);
            }
        }
    };

    // ---- main loop: kRing steps in flight. Loads are issued unconditionally
    // (past the last step they repeat its rows) so that every wait sees the
    // same number of younger loads.
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    if constexpr (RING == 3) {
        issue_step(0, S0{});
        issue_step(1, S1{});
        for (int s = 0;; s += 3) {
            issue_step(s + 2, S2{});
            compute_step(s, S0{});
            if (s + 1 >= nsteps) break;
            issue_step(s + 3, S0{});
            compute_step(s + 1, S1{});
            if (s + 2 >= nsteps) break;
            issue_step(s + 4, S1{});
            compute_step(s + 2, S2{});
            if (s + 3 >= nsteps) break;
        }
    } else {
        issue_step(0, S0{});
        for (int s = 0;; s += 2) {
            issue_step(s + 1, S1{});
            compute_step(s, S0{});
            if (s + 1 >= nsteps) break;
            issue_step(s + 2, S0{});
            compute_step(s + 1, S1{});
            if (s + 2 >= nsteps) break;
        }
    }
    // drain the repeated loads before the workgroup exits
    wait_vmem<0>();

    // ---- denominators: lanes -> wave (xor over g) -> workgroup (LDS)
#pragma unroll
    for (int ht = 0; ht < 4; ht++) {
        float v = lq[ht];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        lq[ht] = v;
    }
    __syncthreads();   // all waves are done with xchg
    if (g == 0) {
#pragma unroll
        for (int ht = 0; ht < 4; ht++) xchg[w][16 * ht + lr] = lq[ht];
    }
    __syncthreads();

    // log-sum-exp (base 2) per head, from the QK layout of wave 0
    if (w == 0 && g == 0) {
#pragma unroll
        for (int ht = 0; ht < 4; ht++) {
            const int h = 16 * ht + lr;
            const float lsum = ((xchg[0][h] + xchg[1][h]) + xchg[2][h]) + xchg[3][h];
            const float lse2 = mq[ht] + __builtin_amdgcn_logf(lsum);   // v_log_f32 is log2
            if (single) {
                if (p.lse_out) p.lse_out[b * kHeads + h] = lse2 * kLn2;
            } else {
                p.part_lse[((int64_t)b * p.n_chunk + c) * kHeads + h] = lse2;
            }
        }
    }
    const int col = 64 * w + lr;
#pragma unroll
    for (int ht = 0; ht < 4; ht++) {
        const int h0 = 16 * ht + 4 * g;
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(&xchg[0][h0]);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(&xchg[1][h0]);
        const f32x4 l2 = *reinterpret_cast<const f32x4*>(&xchg[2][h0]);
        const f32x4 l3 = *reinterpret_cast<const f32x4*>(&xchg[3][h0]);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int h = h0 + i;
            const float inv = p.v_scale / (((l0[i] + l1[i]) + l2[i]) + l3[i]);
            if (single) {
                uint16_t* orow = p.out + ((int64_t)b * kHeads + h) * kHeadDim + col;
#pragma unroll
                for (int dt = 0; dt < 4; dt++)
                    orow[16 * dt] = bitcast<uint16_t>((__bf16)(o[ht][dt][i] * inv));
            } else {
                const int64_t pidx = (int64_t)b * p.n_chunk + c;
                float* prow = p.part_o + (pidx * kHeads + h) * kHeadDim + col;
#pragma unroll
                for (int dt = 0; dt < 4; dt++) prow[16 * dt] = o[ht][dt][i] * inv;
            }
        }
    }
}

// Merge the chunk partials of every sequence with more than one chunk:
//   M = max_c lse2_c, W_c = 2^(lse2_c - M), out = sum_c W_c o_c / sum_c W_c,
//   lse = (M + log2 sum_c W_c) * ln 2.
// Block (b, head quad); thread -> head 4*hq + tid/64, columns 4*(tid%64)..+3.
__global__ __launch_bounds__(256) void mfa_combine_kernel(const AttnArgs p) {
    const int b = blockIdx.x >> 4;
    const int h = 4 * (blockIdx.x & 15) + (threadIdx.x >> 6);
    const int d = 4 * (threadIdx.x & 63);
    const int L = seq_len(p.kv, b);
    const int nc = (L + p.chunk - 1) / p.chunk;
    if (nc <= 1) return;
    const int64_t base = (int64_t)b * p.n_chunk;
    float M = -__builtin_inff();
    for (int c = 0; c < nc; c++) M = fmaxf(M, p.part_lse[(base + c) * kHeads + h]);
    float sum = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < nc; c++) {
        const float wgt = __builtin_amdgcn_exp2f(p.part_lse[(base + c) * kHeads + h] - M);
        const f32x4 v = *reinterpret_cast<const f32x4*>(p.part_o + ((base + c) * kHeads + h) * kHeadDim + d);
        sum += wgt;
        acc += wgt * v;
    }
    const float inv = 1.f / sum;
    uint16_t* orow = p.out + ((int64_t)b * kHeads + h) * kHeadDim + d;
    *reinterpret_cast<u32x2*>(orow) = u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv),
                                           pack_bf16x2(acc[2] * inv, acc[3] * inv)};
    if (p.lse_out && (threadIdx.x & 63) == 0)
        p.lse_out[b * kHeads + h] = (M + __builtin_amdgcn_logf(sum)) * kLn2;
}

// Copy the logical rows t < L_b of sequence b through the attention kernel's
// own address generation (kv_step_base). Block = one 64-token step.
template <bool PAGED>
__global__ __launch_bounds__(256) void mfa_gather_kernel(const KvView kv, int b, uint8_t* k_dst,
                                                         uint8_t* v_dst) {
    const int L = seq_len(kv, b);
    const int t0 = blockIdx.x * kStep;
    if (t0 >= L) return;
    const int n = min(kStep, L - t0);
    const int64_t base = kv_step_base<PAGED>(kv, b, t0);
    const int per_row = kv.row_bytes / 16;
    for (int i = threadIdx.x; i < n * per_row; i += blockDim.x) {
        const int r = i / per_row, q = i - r * per_row;
        const int64_t src = (base + r) * kv.row_bytes + 16 * q;
        const int64_t dst = (int64_t)(t0 + r) * kv.row_bytes + 16 * q;
        *reinterpret_cast<u32x4*>(k_dst + dst) = *reinterpret_cast<const u32x4*>(kv.k + src);
        *reinterpret_cast<u32x4*>(v_dst + dst) = *reinterpret_cast<const u32x4*>(kv.v + src);
    }
}

hipError_t launch_attn_split(const AttnArgs& a, bool fp8, bool paged, int batch, hipStream_t st) {
    const dim3 grid(batch * a.n_chunk), block(256);
    if (fp8) {
        if (paged) hipLaunchKernelGGL((mfa_attn_split_kernel<true, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((mfa_attn_split_kernel<true, false>), grid, block, 0, st, a);
    } else {
        if (paged) hipLaunchKernelGGL((mfa_attn_split_kernel<false, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((mfa_attn_split_kernel<false, false>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

hipError_t launch_combine(const AttnArgs& a, int batch, hipStream_t st) {
    hipLaunchKernelGGL(mfa_combine_kernel, dim3(batch * 16), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_gather(const KvView& kv, bool paged, int b, int max_seq_len, void* k_dst,
                         void* v_dst, hipStream_t st) {
    const int nblk = (max_seq_len + kStep - 1) / kStep;
    if (nblk == 0) return hipSuccess;
    if (paged)
        hipLaunchKernelGGL(mfa_gather_kernel<true>, dim3(nblk), dim3(256), 0, st, kv, b,
                           (uint8_t*)k_dst, (uint8_t*)v_dst);
    else
        hipLaunchKernelGGL(mfa_gather_kernel<false>, dim3(nblk), dim3(256), 0, st, kv, b,
                           (uint8_t*)k_dst, (uint8_t*)v_dst);
    return hipGetLastError();
}

}  // namespace mfa
