// mfa_attn.hip -- decode attention of Multi-Matrix Factorization Attention
// on CDNA4 (gfx950): 64 query heads against one shared K head and one shared
// V head of dimension 256 ("Step-3 is Large yet Affordable", Key points),
// split into KV chunks whose partial softmax results are merged by the
// log-sum-exp identity (Flash-Decoding, cited by title on the DeepSeek-V4
// references).
//
// One workgroup (4 wave64s) owns one (sequence, chunk). It walks the chunk in
// steps of 64 tokens (= one cache page):
//   load  K and V rows of a step go from HBM straight into an LDS ring slot
//         (global_load_lds_dwordx4, no registers); FP8 keeps 4 steps in
//         flight, bf16 2. Wave w fetches rows 16w..16w+15 of both tensors.
//   QK    wave w scores its 16 tokens against all 64 heads:
//         S^T[16 tok x 64 heads] = K[16 x 256] . Q^T with bf16 MFMA 16x16x32,
//         K rows from LDS as A operands (FP8 codes widened to bf16 in
//         registers; every E4M3 value is exact in bf16), Q held in registers
//         as B operands for the whole chunk. Each cached K byte feeds 64 heads.
//   P     exp2 of the scaled scores against per-head reference maxima that
//         stay fixed for a pass over the chunk (the exact maxima of its first
//         step), rounded to bf16 into LDS. A score above its reference by more
//         than kTau (base 2) makes the waves vote to redo the chunk with a
//         higher reference, so the output is never rescaled inside the loop.
//   PV    wave w owns output columns 64w..64w+63 of all 64 heads:
//         O[64 x 64] += P[64 x 64 tok] . V[64 tok x 64], V read transposed
//         from the shared tile with ds_read_b64_tr_b8 / _b16.
// One workgroup barrier per step orders the ring, P and the vote.
//
// Scores are kept in the base-2 domain: s2 = s * log2(e), exp -> exp2.
// Output of a chunk: for a one-chunk sequence the final bf16 output and lse;
// otherwise the chunk-normalised output (fp32) and its base-2 lse, merged by
// the log-sum-exp identity either here, by the last of the sequence's chunks
// to finish (launches where no sequence has more than two chunks), or by
// mfa_combine_kernel afterwards.
#include <type_traits>

#include "mfa_device.h"
#include "mfa_internal.h"

namespace mfa {

// ---------------------------------------------------------------- LDS layout
// Every 16-byte chunk c of a cached row r is stored at chunk position
// c ^ swz(r) of that row, so that the reads of one chunk column across rows
// spread over distinct bank groups:
//   K (A-operand reads: 16 rows, one chunk each)      kswz(t) = t & 15
//   V (transposed reads: 8 rows fp8 / 4 rows bf16)     vswz(r) = r & 7   (fp8)
//                                                      vswz(r) = (r & 3) << 1 (bf16)
//   P (64 heads x 64 tokens bf16, 128-byte rows)       pswz(h) = (h >> 1) & 7
__device__ __forceinline__ int kswz(int t) { return t & 15; }
template <bool FP8>
__device__ __forceinline__ int vswz(int r) { return FP8 ? (r & 7) : ((r & 3) << 1); }
__device__ __forceinline__ int pswz(int h) { return (h >> 1) & 7; }

// LDS stores issued as inline asm. The compiler treats a plain LDS store as
// possibly overwriting bytes an LDS DMA is still filling and would first wait
// for every load in flight; these stores go to buffers no DMA touches.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void lds_store_b64(void* p, u32x2 v) {
    asm volatile("ds_write_b64 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_store_b128(void* p, u32x4 v) {
    asm volatile("ds_write_b128 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
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

// 16 bytes per lane from global memory straight into LDS: lane i's bytes come
// from sbase + voff and land at lds_dst + 16*i (lds_dst is wave-uniform and
// goes through M0). Issued as inline asm so that the compiler does not treat
// every later LDS access as possibly overlapping the transfer (it would wait
// for all loads in flight before each one); the ring's own waits (wait_vmem)
// order the reads instead. No register is written, and the "memory" clobber
// keeps earlier reads of the slot ahead of it.
__device__ __forceinline__ void dma_b128(const void* sbase, uint32_t voff, uint32_t lds_dst) {
    asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "{m0}"(lds_dst) : "memory");
}

// A pointer every lane of the wave holds, moved to scalar registers.
__device__ __forceinline__ const uint8_t* wave_uniform(const uint8_t* ptr) {
    const uint64_t u = (uint64_t)(uintptr_t)ptr;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Device-coherent (agent scope, sc1) 16-byte store and loads: they bypass the
// per-XCD L2, so a workgroup on another XCD sees the data once the store is
// acknowledged. The loads are issued as one asm block that also waits for
// them, so no output register is left pending when the block ends.
__device__ __forceinline__ void coherent_store_b128(f32x4* ptr, f32x4 v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(ptr), "v"(v) : "memory");
}
__device__ __forceinline__ void coherent_load_b128x8(f32x4* v, const f32x4* src, int stride) {
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
        : "v"(src), "v"(src + stride), "v"(src + 2 * stride), "v"(src + 3 * stride), "v"(src + 4 * stride),
          "v"(src + 5 * stride), "v"(src + 6 * stride), "v"(src + 7 * stride)
        : "memory");
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
    constexpr int CPR = ROWB / 16;                 // 16-byte chunks per row
    constexpr int RPI = 1024 / ROWB;               // rows per 1 KB DMA instruction
    constexpr int KW = 16 * ROWB;                  // a wave's 16 rows of one step
    constexpr int VT = kStep * ROWB;               // the V tile of one step
    constexpr int NDMA = KW / 1024;                // DMA instructions per wave for K (same for V)
    constexpr int OPS = 2 * NDMA;                  // vector-memory instructions per wave per step
    // steps in flight: 4 x 32 KB (FP8) or 2 x 64 KB (bf16) of K + V
    constexpr int RING = FP8 ? 4 : 2;

    // LDS: the ring (slot-major: four waves' K rows, then the V tile), then
    // the two P buffers. Slot RING-1 doubles as the staging area for Q.
    constexpr int SLOT = 4 * KW + VT;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[RING * SLOT + 2 * kHeads * kStep * 2];
    __shared__ __attribute__((aligned(16))) float xchg[4][kHeads];
    __shared__ __attribute__((aligned(16))) float xchg2[4][kHeads];
    __shared__ int flags_all[2][4];
    __shared__ int arrival;
    __shared__ float lse_lds[kHeads];
    auto kring = [&](int slot, int wave) -> uint8_t* { return smem + slot * SLOT + wave * KW; };
    auto vring = [&](int slot) -> uint8_t* { return smem + slot * SLOT + 4 * KW; };
    auto plds_of = [&](int parity) -> uint8_t* { return smem + RING * SLOT + parity * (kHeads * kStep * 2); };

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int lr = l & 15;
    const int g = l >> 4;

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

    // ---- DMA lane offsets (bytes from the step's first row; loop-invariant).
    // Instruction i of wave w fills rows 16w + RPI*i + l/CPR; lane l lands at
    // chunk position l % CPR of its row and so fetches the data chunk that the
    // swizzle puts there.
    uint32_t koff[NDMA], voff[NDMA];
#pragma unroll
    for (int i = 0; i < NDMA; i++) {
        const int t = RPI * i + l / CPR;           // row within the wave's 16
        const int r = 16 * w + t;                  // row within the step
        koff[i] = r * ROWB + 16 * ((l % CPR) ^ kswz(t));
        voff[i] = r * ROWB + 16 * ((l % CPR) ^ vswz<FP8>(r));
    }

    // ---- paged caches: the pages of the chunk's steps, fetched once. Lane j
    // holds the page of step j (pg0) and of step 64 + j (pg1); a step reads
    // its page with v_readlane, so no load (and no wait for one) sits in the
    // loop. Paged chunks have at most kMaxPagedChunkSteps = 128 steps (the
    // host enforces it).
    int32_t pg0 = 0, pg1 = 0;
    if constexpr (PAGED) {
        const int32_t* chunk_pt = p.kv.page_table + (int64_t)b * p.kv.pt_stride + (t_begin >> 6);
        if (l < nsteps) pg0 = chunk_pt[l];
        if (64 + l < nsteps) pg1 = chunk_pt[64 + l];
    }
    // first cache row of step s (s <= last_s)
    auto step_row = [&](int s) -> int64_t {
        if constexpr (PAGED) {
            const int32_t page = s < 64 ? __builtin_amdgcn_readlane(pg0, s) : __builtin_amdgcn_readlane(pg1, s - 64);
            return (int64_t)page * kPage;
        } else {
            return kv_step_base<false>(p.kv, b, t_begin + s * kStep);
        }
    };

    // ---- issue the loads of step s (clamped to the last step, whose rows then
    // hit in L2) into ring slot s % RING: this wave's 16 K rows into its
    // private region, and the same 16 rows of V into the shared V tile.
    auto issue_step = [&](int s) {
        const int t0 = t_begin + min(s, last_s) * kStep;
        const int64_t base = step_row(min(s, last_s));
        const uint8_t* kb = wave_uniform(p.kv.k + base * ROWB);
        const uint8_t* vb = wave_uniform(p.kv.v + base * ROWB);
        const int slot = s % RING;
        const uint32_t kd = __builtin_amdgcn_readfirstlane(lds_addr(kring(slot, w)));
        const uint32_t vd = __builtin_amdgcn_readfirstlane(lds_addr(vring(slot)) + 16 * w * ROWB);
        const int last = t_end - 1 - t0;           // last valid row of the step
        if (last >= kStep - 1) {
#pragma unroll
            for (int i = 0; i < NDMA; i++) {
                dma_b128(kb, koff[i], kd + 1024 * i);
                dma_b128(vb, voff[i], vd + 1024 * i);
            }
        } else {   // partial last step: rows past the chunk end repeat the last row
#pragma unroll
            for (int i = 0; i < NDMA; i++) {
                const int r = 16 * w + RPI * i + l / CPR;
                const uint32_t shift = (uint32_t)((min(r, last) - r) * ROWB);
                dma_b128(kb, koff[i] + shift, kd + 1024 * i);
                dma_b128(vb, voff[i] + shift, vd + 1024 * i);
            }
        }
    };

    // ---- Q, fetched once per workgroup by DMA into the staging area (slot
    // RING-1 of the ring, free until the first step's barrier): 16-byte
    // chunk c of head h at position c ^ (h & 15); wave w copies heads
    // 16w..16w+15. The ring's first steps stream in behind it.
    uint8_t* const qs = smem + (RING - 1) * SLOT;
    {
        const uint8_t* qb = wave_uniform(reinterpret_cast<const uint8_t*>(p.q + (int64_t)b * kHeads * kHeadDim));
        const uint32_t qd = __builtin_amdgcn_readfirstlane(lds_addr(qs + 16 * w * 512));
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int h = 16 * w + 2 * i + (l >> 5);
            dma_b128(qb, (uint32_t)(h * 512 + 16 * ((l & 31) ^ (h & 15))), qd + 1024 * i);
        }
    }
#pragma unroll
    for (int s = 0; s < RING - 1; s++) issue_step(s);

    // Every wave reads its B operands: qop[ht][ks] holds Q[16ht + lr][d(ks,
    // g, 0..7)] with d(ks, g, j) = 64*(ks/2) + 16*g + 8*(ks%2) + j, the same
    // d order the K A operands use below.
    bf16x8 qop[4][8];
    {
        // this wave's Q rows have landed once at most the ring's loads are in
        // flight; the barrier makes every wave's rows visible
        wait_vmem<(RING - 1) * OPS>();
        lds_barrier();
#pragma unroll
        for (int ht = 0; ht < 4; ht++)
#pragma unroll
            for (int ks = 0; ks < 8; ks++) {
                const int h = 16 * ht + lr;
                const int cq = 8 * (ks >> 1) + 2 * g + (ks & 1);
                qop[ht][ks] = *reinterpret_cast<const bf16x8*>(qs + h * 512 + 16 * (cq ^ (h & 15)));
            }
    }

    // ---- per-pass state (QK layout: heads 16ht + lr). The reference maxima
    // are fixed for a whole pass over the chunk: the exact maxima of the
    // first step, raised to m_floor. A later score may exceed its reference
    // by up to kTau (base 2), so unnormalised P <= 2^kTau and the output
    // accumulators are never rescaled inside the loop. A larger excess, voted
    // by any wave, restarts the chunk with the floor raised.
    float mq[4];         // reference maxima (base 2)
    float lq[4];         // partial softmax denominators of the rounded P
    float le[4];         // partial softmax denominators of the unrounded P
    float m_floor[4];    // lower bound for the references (from a restart)
    f32x4 o[4][4];       // O[16ht + 4g + i][64w + 16dt + lr]
#pragma unroll
    for (int ht = 0; ht < 4; ht++) m_floor[ht] = -__builtin_inff();

    auto clear_acc = [&]() {
#pragma unroll
        for (int ht = 0; ht < 4; ht++) {
            lq[ht] = 0.f;
            le[ht] = 0.f;
#pragma unroll
            for (int dt = 0; dt < 4; dt++) o[ht][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };

    // scores S^T[token 4g+i][head 16ht+lr] of this wave's 16 tokens of step s
    // (its K rows have landed), tokens past the chunk end at -inf
    auto qk = [&](int s, f32x4* sc) {
        const int t0 = t_begin + s * kStep;
        const uint8_t* klds = kring(s % RING, w) + lr * ROWB;   // this lane's K row
        u32x4 kp[FP8 ? 4 : 8];
#pragma unroll
        for (int i = 0; i < (FP8 ? 4 : 8); i++) {
            // fp8: piece i = bytes 64i + 16g; bf16: bytes 128(i/2) + 32g + 16(i%2)
            const int cidx = FP8 ? (4 * i + g) : (8 * (i >> 1) + 2 * g + (i & 1));
            kp[i] = *reinterpret_cast<const u32x4*>(klds + 16 * (cidx ^ kswz(lr)));
        }
#pragma unroll
        for (int ht = 0; ht < 4; ht++) sc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (FP8) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const bf16x8 a0 = e4m3x8_to_bf16x8(kp[i].x, kp[i].y);
                const bf16x8 a1 = e4m3x8_to_bf16x8(kp[i].z, kp[i].w);
#pragma unroll
                for (int ht = 0; ht < 4; ht++) {
                    sc[ht] = mfma16(a0, qop[ht][2 * i], sc[ht]);
                    sc[ht] = mfma16(a1, qop[ht][2 * i + 1], sc[ht]);
                }
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < 8; ks++) {
                const bf16x8 a = bitcast<bf16x8>(kp[ks]);
#pragma unroll
                for (int ht = 0; ht < 4; ht++) sc[ht] = mfma16(a, qop[ht][ks], sc[ht]);
            }
        }
        if (t_end - t0 < kStep) {   // last step of the chunk only
            const int valid = t_end - t0 - (16 * w + 4 * g);   // rows i < valid are real tokens
#pragma unroll
            for (int ht = 0; ht < 4; ht++)
#pragma unroll
                for (int i = 0; i < 4; i++)
                    if (i >= valid) sc[ht][i] = -__builtin_inff();
        }
    };

    // per-head maxima (base 2) of this step over all four waves, in QK layout
    auto exchange_max = [&](const f32x4* sc, float* m_out) {
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
            m_out[ht] = fmaxf(fmaxf(xchg[0][h], xchg[1][h]), fmaxf(xchg[2][h], xchg[3][h]));
        }
    };

    // P = exp2(s2 - reference), rounded to bf16, into the step's P buffer.
    // Two partial denominators: of the rounded P (normalises the output, so
    // the weights applied to V sum to one) and of the unrounded P (gives the
    // log-sum-exp to fp32 accuracy instead of bf16's 2^-8).
    auto write_p = [&](int s, const f32x4* sc, float* lr_step, float* le_step) {
        uint8_t* plds = plds_of(s & 1);
#pragma unroll
        for (int ht = 0; ht < 4; ht++) {
            float e[4];
#pragma unroll
            for (int i = 0; i < 4; i++)
                e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[ht][i], p.score_scale, -mq[ht]));
            const uint32_t p01 = pack_bf16x2(e[0], e[1]);
            const uint32_t p23 = pack_bf16x2(e[2], e[3]);
            lr_step[ht] = (__builtin_bit_cast(float, p01 << 16) + __builtin_bit_cast(float, p01 & 0xffff0000u)) +
                          (__builtin_bit_cast(float, p23 << 16) + __builtin_bit_cast(float, p23 & 0xffff0000u));
            le_step[ht] = (e[0] + e[1]) + (e[2] + e[3]);
            const int h = 16 * ht + lr;
            const int ch = (2 * w + (g >> 1)) ^ pswz(h);
            lds_store_b64(plds + h * 128 + 16 * ch + 8 * (g & 1), u32x2{p01, p23});
        }
    };

    // O[64 heads][64w..64w+63] += P[64 x 64 tok] . V[64 tok x 64w..64w+63];
    // all LDS reads of the step are issued before the conversions and MFMAs
    auto pv = [&](int s) {
        const uint8_t* plds = plds_of(s & 1);
        const uint8_t* vt = vring(s % RING);
        bf16x8 pa[2][4];
#pragma unroll
        for (int kk = 0; kk < 2; kk++)
#pragma unroll
            for (int ht = 0; ht < 4; ht++) {
                const int h = 16 * ht + lr;
                pa[kk][ht] = *reinterpret_cast<const bf16x8*>(plds + h * 128 + 16 * ((4 * kk + g) ^ pswz(h)));
            }
        if constexpr (FP8) {
            // lane j of a 16-lane group points at row r0 + j/2, bytes 8(j%2)..+7
            // of chunk 4w + dt; it receives column 64w + 16dt + j of rows r0..r0+7
            i32x2 vr[2][4];
#pragma unroll
            for (int kk = 0; kk < 2; kk++)
#pragma unroll
                for (int dt = 0; dt < 4; dt++) {
                    const int row = 32 * kk + 8 * g + (lr >> 1);
                    const uint8_t* a = vt + row * ROWB + 16 * ((4 * w + dt) ^ vswz<FP8>(row)) + 8 * (lr & 1);
                    vr[kk][dt] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (__attribute__((address_space(3))) i32x2*)(a));
                }
#pragma unroll
            for (int kk = 0; kk < 2; kk++)
#pragma unroll
                for (int dt = 0; dt < 4; dt++) {
                    const bf16x8 vb = e4m3x8_to_bf16x8((uint32_t)vr[kk][dt].x, (uint32_t)vr[kk][dt].y);
#pragma unroll
                    for (int ht = 0; ht < 4; ht++) o[ht][dt] = mfma16(pa[kk][ht], vb, o[ht][dt]);
                }
        } else {
            // two transposed reads of 4 rows each: lane j points at row
            // r0 + j/4, elements 4(j%4)..+3 of the 16-column block
            i16x4 vr[2][4][2];
#pragma unroll
            for (int kk = 0; kk < 2; kk++)
#pragma unroll
                for (int dt = 0; dt < 4; dt++)
#pragma unroll
                    for (int hh = 0; hh < 2; hh++) {
                        const int row = 32 * kk + 8 * g + 4 * hh + (lr >> 2);
                        const int ch = 8 * w + 2 * dt + ((lr & 3) >> 1);
                        const uint8_t* a = vt + row * ROWB + 16 * (ch ^ vswz<FP8>(row)) + 8 * (lr & 1);
                        vr[kk][dt][hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) i16x4*)(a));
                    }
#pragma unroll
            for (int kk = 0; kk < 2; kk++)
#pragma unroll
                for (int dt = 0; dt < 4; dt++) {
                    const u32x2 u0 = bitcast<u32x2>(vr[kk][dt][0]);
                    const u32x2 u1 = bitcast<u32x2>(vr[kk][dt][1]);
                    const bf16x8 vb = bitcast<bf16x8>(u32x4{u0.x, u0.y, u1.x, u1.y});
#pragma unroll
                    for (int ht = 0; ht < 4; ht++) o[ht][dt] = mfma16(pa[kk][ht], vb, o[ht][dt]);
                }
        }
    };

    // Step s > 0 against the fixed references. Returns true (in every wave)
    // when some score exceeded its reference by more than kTau; m_floor then
    // holds the raised bound and the step's P.V is skipped.
    auto step = [&](int s) -> bool {
        // this wave's K and V rows of step s have landed once at most the
        // RING-2 younger steps' loads are in flight
        wait_vmem<(RING - 2) * OPS>();
        f32x4 sc[4];
        qk(s, sc);
        bool over = false;
#pragma unroll
        for (int ht = 0; ht < 4; ht++) {
            const float m = fmaxf(fmaxf(sc[ht][0], sc[ht][1]), fmaxf(sc[ht][2], sc[ht][3]));
            over |= m * p.score_scale > mq[ht] + kTau;
        }
        const bool wave_over = __builtin_amdgcn_ballot_w64(over) != 0;
        float lstep[4], estep[4];
        write_p(s, sc, lstep, estep);
        int* flags = flags_all[s & 1];
        if (l == 0) lds_store_b32(&flags[w], wave_over ? 1u : 0u);
        // after this barrier: P of step s and every wave's V rows of step s
        // are visible, and every wave is done with the P.V of step s-1
        lds_barrier();
        if ((flags[0] | flags[1] | flags[2] | flags[3]) != 0) {
            float m[4];
            exchange_max(sc, m);
#pragma unroll
            for (int ht = 0; ht < 4; ht++) m_floor[ht] = fmaxf(mq[ht], m[ht]);
            lds_barrier();   // everyone has read xchg before it is reused
            // The next pass starts from zero. Clearing here (not at the top
            // of the pass) leaves the accumulators entering this step with a
            // single use, the P.V MFMA, so it can accumulate in place.
            clear_acc();
            return true;
        }
        // ring slot (s-1) % RING is free now: refill it
        issue_step(s + RING - 1);
#pragma unroll
        for (int ht = 0; ht < 4; ht++) {
            lq[ht] += lstep[ht];
            le[ht] += estep[ht];
        }
        pv(s);
        return false;
    };

    clear_acc();
    for (int pass = 0;; pass++) {   // one pass over the chunk; repeated only after a vote
        // Loads are issued unconditionally (past the last step they repeat
        // its rows) so that every wait sees the same number of younger loads.
        if (pass > 0) {
#pragma unroll
            for (int s = 0; s < RING - 1; s++) issue_step(s);
        }
        {   // step 0 sets the references from its exact maxima
            wait_vmem<(RING - 2) * OPS>();
            f32x4 sc[4];
            qk(0, sc);
            float m[4];
            exchange_max(sc, m);
#pragma unroll
            for (int ht = 0; ht < 4; ht++) mq[ht] = fmaxf(m_floor[ht], m[ht]);
            float lstep[4], estep[4];
            write_p(0, sc, lstep, estep);
            lds_barrier();
            issue_step(RING - 1);
#pragma unroll
            for (int ht = 0; ht < 4; ht++) {
                lq[ht] += lstep[ht];
                le[ht] += estep[ht];
            }
            pv(0);
        }
        bool restart = false;
        for (int s = 1; s < nsteps; s++)
            if ((restart = step(s))) break;
        // drain the ring's loads (the repeated ones too) before the next pass
        // or the exit
        wait_vmem<0>();
        if (!restart) break;
        lds_barrier();   // no wave still reads the ring or P of the pass
    }

    // ---- denominators: lanes -> wave (xor over g) -> workgroup (LDS)
#pragma unroll
    for (int ht = 0; ht < 4; ht++) {
        float v = lq[ht], u = le[ht];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        u += __shfl_xor(u, 16);
        u += __shfl_xor(u, 32);
        lq[ht] = v;
        le[ht] = u;
    }
    __syncthreads();   // all waves are done with xchg
    if (g == 0) {
#pragma unroll
        for (int ht = 0; ht < 4; ht++) {
            xchg[w][16 * ht + lr] = lq[ht];
            xchg2[w][16 * ht + lr] = le[ht];
        }
    }
    __syncthreads();

    // log-sum-exp (base 2) per head, from the QK layout of wave 0, shared
    // through LDS
    if (w == 0 && g == 0) {
#pragma unroll
        for (int ht = 0; ht < 4; ht++) {
            const int h = 16 * ht + lr;
            const float lsum = ((xchg2[0][h] + xchg2[1][h]) + xchg2[2][h]) + xchg2[3][h];
            lse_lds[h] = mq[ht] + __builtin_amdgcn_logf(lsum);   // v_log_f32 is log2
        }
    }
    __syncthreads();

    const int col = 64 * w + lr;
    // this chunk's normalised output, PV layout
#pragma unroll
    for (int ht = 0; ht < 4; ht++) {
        const int h0 = 16 * ht + 4 * g;
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(&xchg[0][h0]);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(&xchg[1][h0]);
        const f32x4 l2 = *reinterpret_cast<const f32x4*>(&xchg[2][h0]);
        const f32x4 l3 = *reinterpret_cast<const f32x4*>(&xchg[3][h0]);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float inv = p.v_scale / (((l0[i] + l1[i]) + l2[i]) + l3[i]);
#pragma unroll
            for (int dt = 0; dt < 4; dt++) o[ht][dt][i] *= inv;
        }
    }
    auto store_final = [&](int h, int dt, float v) {
        p.out[((int64_t)b * kHeads + h) * kHeadDim + col + 16 * dt] = bitcast<uint16_t>((__bf16)v);
    };
    if (single) {
#pragma unroll
        for (int ht = 0; ht < 4; ht++)
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int dt = 0; dt < 4; dt++) store_final(16 * ht + 4 * g + i, dt, o[ht][dt][i]);
        if (p.lse_out && tid < kHeads) p.lse_out[b * kHeads + tid] = lse_lds[tid] * kLn2;
        return;
    }

    // several chunks: publish this chunk's partial (normalised output and
    // base-2 log-sum-exp)
    const int64_t pidx = (int64_t)b * p.n_chunk + c;
    const int nc = (L + p.chunk - 1) / p.chunk;
    if (nc > p.fuse_max) {   // mfa_combine_kernel merges these after this kernel
#pragma unroll
        for (int ht = 0; ht < 4; ht++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                float* prow = p.part_o + (pidx * kHeads + 16 * ht + 4 * g + i) * kHeadDim + col;
#pragma unroll
                for (int dt = 0; dt < 4; dt++) prow[16 * dt] = o[ht][dt][i];
            }
        if (tid < kHeads) p.part_lse[pidx * kHeads + tid] = lse_lds[tid];
        return;
    }

    // few chunks: the workgroup that finishes a sequence's chunks last merges
    // them. Each workgroup dumps its registers (thread-major: float4 j of
    // thread tid at (j * 256 + tid), so every instruction writes 4 KB
    // contiguous) with device-coherent stores that bypass the per-XCD L2;
    // they are acknowledged (vmcnt 0) before the arrival count. The merging
    // workgroup reads the other dumps back the same way after seeing the
    // count. No cache-wide writeback or invalidate is needed.
    f32x4* dump = reinterpret_cast<f32x4*>(p.part_o) + pidx * (kHeads * kHeadDim / 4);
#pragma unroll
    for (int j = 0; j < 16; j++) {
        const int ht = j >> 2, i = j & 3;
        coherent_store_b128(dump + j * 256 + tid, f32x4{o[ht][0][i], o[ht][1][i], o[ht][2][i], o[ht][3][i]});
    }
    if (tid < kHeads)
        __hip_atomic_store(p.part_lse + pidx * kHeads + tid, lse_lds[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_vmem<0>();
    __syncthreads();
    if (tid == 0) arrival = __hip_atomic_fetch_add(&p.counters[b], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (arrival != nc - 1) return;
    if (tid == 0) __hip_atomic_store(&p.counters[b], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // chunks in index order whichever workgroup merges, so the result does
    // not depend on which one finished last
    const int64_t base = (int64_t)b * p.n_chunk;
    float M[16], wsum[16];
    f32x4 acc[16];
#pragma unroll
    for (int j = 0; j < 16; j++) {
        M[j] = -__builtin_inff();
        wsum[j] = 0.f;
        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int cc = 0; cc < nc; cc++) {
#pragma unroll
        for (int j = 0; j < 16; j++) {
            const int h = 16 * (j >> 2) + 4 * g + (j & 3);
            M[j] = fmaxf(M[j], __hip_atomic_load(p.part_lse + (base + cc) * kHeads + h, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT));
        }
    }
    for (int cc = 0; cc < nc; cc++) {
        f32x4 v[16];
        if (cc == c) {   // this workgroup's own chunk, still in registers
#pragma unroll
            for (int j = 0; j < 16; j++) {
                const int ht = j >> 2, i = j & 3;
                v[j] = f32x4{o[ht][0][i], o[ht][1][i], o[ht][2][i], o[ht][3][i]};
            }
        } else {
            const f32x4* src = reinterpret_cast<const f32x4*>(p.part_o) + (base + cc) * (kHeads * kHeadDim / 4);
            coherent_load_b128x8(v, src + tid, 256);
            coherent_load_b128x8(v + 8, src + 8 * 256 + tid, 256);
        }
#pragma unroll
        for (int j = 0; j < 16; j++) {
            const int h = 16 * (j >> 2) + 4 * g + (j & 3);
            const float wc = __builtin_amdgcn_exp2f(
                __hip_atomic_load(p.part_lse + (base + cc) * kHeads + h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - M[j]);
            wsum[j] += wc;
            acc[j] += wc * v[j];
        }
    }
#pragma unroll
    for (int j = 0; j < 16; j++) {
        const int h = 16 * (j >> 2) + 4 * g + (j & 3);
        const float inv = 1.f / wsum[j];
#pragma unroll
        for (int dt = 0; dt < 4; dt++) store_final(h, dt, acc[j][dt] * inv);
        if (p.lse_out && w == 0 && lr == 0) p.lse_out[b * kHeads + h] = (M[j] + __builtin_amdgcn_logf(wsum[j])) * kLn2;
    }
}

// Merge the chunk partials of every sequence with more than one chunk:
//   M = max_c lse2_c, W_c = 2^(lse2_c - M), out = sum_c W_c o_c / sum_c W_c,
//   lse = (M + log2 sum_c W_c) * ln 2.
// One wave per (sequence, head); lane t owns columns 4t..4t+3. The chunk
// weights go through LDS; the partial rows (1 KB per chunk, contiguous) are
// read kCombineUnroll at a time so that many loads are in flight. Chunks are
// accumulated in index order.
constexpr int kCombineUnroll = 16;
constexpr int kCombineBlock = 1024;   // chunk weights staged per round
__global__ __launch_bounds__(64) void mfa_combine_kernel(const AttnArgs p) {
    __shared__ float wts[kCombineBlock];
    const int b = blockIdx.x >> 6;
    const int h = blockIdx.x & 63;
    const int t = threadIdx.x;
    const int L = seq_len(p.kv, b);
    const int nc = (L + p.chunk - 1) / p.chunk;
    if (nc <= p.fuse_max) return;   // merged by the attention kernel itself
    const int64_t base = (int64_t)b * p.n_chunk;
    const float* lse = p.part_lse + base * kHeads + h;   // chunk c at lse[c * kHeads]
    constexpr int64_t kRow = kHeads * kHeadDim / 4;      // f32x4 per chunk partial
    const f32x4* po = reinterpret_cast<const f32x4*>(p.part_o) + (base * kHeads + h) * (kHeadDim / 4) + t;

    float M = -__builtin_inff();
    for (int c = t; c < nc; c += 64) M = fmaxf(M, lse[(int64_t)c * kHeads]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));

    float wpart = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < nc; c0 += kCombineBlock) {
        const int n = min(kCombineBlock, nc - c0);
        for (int i = t; i < n; i += 64) {
            const float wv = __builtin_amdgcn_exp2f(lse[(int64_t)(c0 + i) * kHeads] - M);
            wts[i] = wv;
            wpart += wv;
        }
        __syncthreads();
        int i = 0;
        for (; i + kCombineUnroll <= n; i += kCombineUnroll) {
            f32x4 v[kCombineUnroll];
#pragma unroll
            for (int j = 0; j < kCombineUnroll; j++) v[j] = po[(int64_t)(c0 + i + j) * kRow];
#pragma unroll
            for (int j = 0; j < kCombineUnroll; j++) acc += wts[i + j] * v[j];
        }
        for (; i < n; i++) acc += wts[i] * po[(int64_t)(c0 + i) * kRow];
        __syncthreads();
    }
    float wsum = wpart;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) wsum += __shfl_xor(wsum, off);
    const float inv = 1.f / wsum;
    uint16_t* orow = p.out + ((int64_t)b * kHeads + h) * kHeadDim + 4 * t;
    *reinterpret_cast<u32x2*>(orow) = u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv),
                                           pack_bf16x2(acc[2] * inv, acc[3] * inv)};
    if (p.lse_out && t == 0) p.lse_out[b * kHeads + h] = (M + __builtin_amdgcn_logf(wsum)) * kLn2;
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

hipError_t launch_attn_split(const AttnArgs& a, bool fp8, bool paged, int batch, const Launch& l) {
    const dim3 grid(batch * a.n_chunk), block(256);
    if (fp8)
        return paged ? launch_kernel(mfa_attn_split_kernel<true, true>, grid, block, l, a)
                     : launch_kernel(mfa_attn_split_kernel<true, false>, grid, block, l, a);
    return paged ? launch_kernel(mfa_attn_split_kernel<false, true>, grid, block, l, a)
                 : launch_kernel(mfa_attn_split_kernel<false, false>, grid, block, l, a);
}

hipError_t launch_combine(const AttnArgs& a, int batch, const Launch& l) {
    return launch_kernel(mfa_combine_kernel, dim3(batch * kHeads), dim3(64), l, a);
}

hipError_t launch_gather(const KvView& kv, bool paged, int b, int max_seq_len, void* k_dst,
                         void* v_dst, const Launch& l) {
    const int nblk = (max_seq_len + kStep - 1) / kStep;
    if (nblk == 0) return hipSuccess;
    return launch_kernel(paged ? mfa_gather_kernel<true> : mfa_gather_kernel<false>, dim3(nblk), dim3(256), l, kv,
                         b, (uint8_t*)k_dst, (uint8_t*)v_dst);
}

}  // namespace mfa
