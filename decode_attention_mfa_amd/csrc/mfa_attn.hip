// mfa_attn.hip -- decode attention of Multi-Matrix Factorization Attention
// on CDNA4 (gfx950): 64 query heads against one shared K head and one shared
// V head of dimension 256 ("Step-3 is Large yet Affordable", Key points),
// split into KV chunks whose partial softmax results are merged by the
// log-sum-exp identity (Flash-Decoding, cited by title on the DeepSeek-V4
// references).
//
// One workgroup (eight wave64s, two per SIMD) owns a piece of one sequence:
// a chunk (chunked kernel) or the part of its equal range of the batch's
// steps that falls in that sequence (balanced kernel; see the notes before
// the two kernels). The piece body (mfa_attn_ws.inc) walks the piece in
// steps of 64 tokens (= one cache page), with the waves in two roles:
//   score waves 0-3: wave w streams K rows 16w..16w+15 of each step from HBM
//         into its own LDS region (global_load_lds_dwordx4, no registers) and
//         scores them against all heads: S^T[16 tok x heads] = K . Q^T with
//         bf16 MFMA 16x16x32, K rows from LDS as A operands (FP8 codes
//         widened to bf16 in registers; every E4M3 value is exact in bf16), Q
//         held in registers as B operands for the whole piece. Each cached K
//         byte feeds 64 heads. Then P = exp2 of the scaled scores against
//         per-head reference maxima that stay fixed for a pass over the piece
//         (the exact maxima of its first step), rounded to bf16 into LDS. A
//         score above its reference by more than kTau (base 2) makes the
//         waves vote to redo the piece with a higher reference, so the output
//         is never rescaled inside the loop.
//   P.V waves 4-7: wave w streams V rows 16w..16w+15 into the shared V tile
//         and owns output columns 64w..64w+63 of all heads:
//         O[heads x 64] += P[heads x 64 tok] . V[64 tok x 64], V read
//         transposed from the tile with ds_read_b64_tr_b8 / _b16.
//   The roles run one step apart (scores of step s+1 beside the P.V of step
//   s), so one wave's MFMAs overlap the other's VALU work; one workgroup
//   barrier per step orders the ring, P and the vote.
//
// Scores are kept in the base-2 domain: s2 = s * log2(e), exp -> exp2.
// Output of a piece: for a one-piece sequence the final bf16 output and lse;
// otherwise the piece-normalised output (rounded to bf16) and its base-2 lse
// (fp32), merged in fp32 by the log-sum-exp identity either here, by the last
// of the sequence's pieces to finish (balanced launches, and chunked launches
// where no sequence has more than two chunks), or by mfa_combine_kernel
// afterwards.
#include <algorithm>
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
// FP8-MFMA mode: P as E4M3, 64-byte rows (64 tokens), 16-byte chunks
__device__ __forceinline__ int p8swz(int h) { return (h >> 2) & 3; }

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

// Device-coherent (sc1) variants for reading back data that workgroups on
// other XCDs published with device-coherent stores: 16 or 4 bytes per lane.
__device__ __forceinline__ void dma_b128_coherent(const void* sbase, uint32_t voff, uint32_t lds_dst) {
    asm volatile("global_load_lds_dwordx4 %0, %1 sc1" ::"v"(voff), "s"(sbase), "{m0}"(lds_dst) : "memory");
}
__device__ __forceinline__ void dma_b32_coherent(const void* sbase, uint32_t voff, uint32_t lds_dst) {
    asm volatile("global_load_lds_dword %0, %1 sc1" ::"v"(voff), "s"(sbase), "{m0}"(lds_dst) : "memory");
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
// A store of more than 8 bytes still reads its data VGPRs after it issues: a
// VALU write to them must come at least two wait states later on this
// architecture. The compiler keeps that distance after the stores it
// generates but cannot see this one, so the block ends with the wait states.
__device__ __forceinline__ void coherent_store_b128(u32x4* ptr, u32x4 v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" ::"v"(ptr), "v"(v) : "memory");
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

__device__ __forceinline__ void coherent_load_b128x2(f32x4* v, const f32x4* src, int stride) {
    asm volatile(
        "global_load_dwordx4 %0, %2, off sc1\n\t"
        "global_load_dwordx4 %1, %3, off sc1\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1])
        : "v"(src), "v"(src + stride)
        : "memory");
}

__device__ __forceinline__ void coherent_load_b128x4(f32x4* v, const f32x4* src, int stride) {
    asm volatile(
        "global_load_dwordx4 %0, %4, off sc1\n\t"
        "global_load_dwordx4 %1, %5, off sc1\n\t"
        "global_load_dwordx4 %2, %6, off sc1\n\t"
        "global_load_dwordx4 %3, %7, off sc1\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
        : "v"(src), "v"(src + stride), "v"(src + 2 * stride), "v"(src + 3 * stride)
        : "memory");
}

// Rows 2j and 2j + 1 (four columns each) of a bf16 dump group: the low half
// of each word is the first of its two values.
__device__ __forceinline__ void unpack_bf16_rows(u32x4 d, f32x4& r0, f32x4& r1) {
    r0 = f32x4{__builtin_bit_cast(float, d.x << 16), __builtin_bit_cast(float, d.x & 0xffff0000u),
               __builtin_bit_cast(float, d.y << 16), __builtin_bit_cast(float, d.y & 0xffff0000u)};
    r1 = f32x4{__builtin_bit_cast(float, d.z << 16), __builtin_bit_cast(float, d.z & 0xffff0000u),
               __builtin_bit_cast(float, d.w << 16), __builtin_bit_cast(float, d.w & 0xffff0000u)};
}

// Wait until at most N vector-memory operations of this wave are in flight.
// The "memory" clobber keeps the compiler from moving LDS reads of the
// DMA-filled ring above the wait.
template <int N>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}


// ------------------------------------------------------------ the two kernels
// Two ways to cut the work into workgroups:
//   chunks   (mfa_attn_ws_split_kernel): workgroup (b, c) takes tokens
//            [c*chunk, (c+1)*chunk) of sequence b; workgroups past L_b exit.
//   balanced (mfa_attn_balanced_kernel): all sequences, in sequence order,
//            laid end to end as units (a sequence's 64-token steps plus
//            kBalancedPieceCost for its piece's fixed work), are dealt out
//            in equal ranges of `per` units (per = ceil(total / workgroups),
//            at least kMinBalancedSteps, at most kMaxPagedChunkSteps), so
//            every workgroup does about the same work whatever the lengths
//            (the work-centric decomposition of Stream-K, cited by title on
//            the DeepSeek-V4 references, applied to KV steps). A range may hold the end of one
//            sequence and the start of others; each piece is a call of
//            attend_piece, and the last of a sequence's pieces to finish
//            merges them.
// Both run the same piece body (the two .inc files).
//
// Multi-token decode (MTP, chunked kernel only): each cache sequence kvb has
// t = p.qtok query tokens, query rows b = kvb*t + j; token j attends to the
// first L_kvb - (t-1-j) rows (the cache already holds the t new tokens, the
// last at row L - 1). The t workgroups of one (sequence, chunk) get block
// indices 8 apart inside a group of 8t, so that the round-robin dispatch puts
// them on one XCD at about the same time: the KV bytes come from HBM once and
// from that XCD's L2 for the other tokens.

// The chunked kernel: eight waves in two roles (the body in
// mfa_attn_ws.inc). With several workgroups per (sequence, chunk) -- the t
// query tokens of multi-token decode, or p.nh groups of 16 * NHT heads --
// those workgroups get block indices 8 apart inside a group of 8 times their
// number, so that the round-robin dispatch puts them on one XCD at about the
// same time (their shared K/V rows then come from HBM once).
template <bool FP8, bool PAGED, bool MTP, bool F8MMA, int NHT>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void mfa_attn_ws_split_kernel(const AttnArgs p) {
    int b, c, kvb, L, part = 0;
    const int reps = p.qtok * p.nh;
    if (reps == 1) {
        b = blockIdx.x / p.n_chunk;
        c = blockIdx.x - b * p.n_chunk;
        kvb = b;
        L = seq_len(p.kv, b);
    } else {
        const int grp = blockIdx.x / (8 * reps);
        const int r = blockIdx.x - grp * 8 * reps;
        const int wi = grp * 8 + (r & 7);   // (sequence, chunk) work item
        if (wi >= p.batch * p.n_chunk) return;
        kvb = wi / p.n_chunk;
        c = wi - kvb * p.n_chunk;
        const int rep = r >> 3;
        const int j = rep % p.qtok;         // query token
        if constexpr (NHT < 4) part = rep / p.qtok;
        b = kvb * p.qtok + j;
        L = seq_len(p.kv, kvb);
        if constexpr (MTP) L = max(0, L - (p.qtok - 1 - j));
    }
    constexpr int NHW = 16 * NHT;           // heads of this workgroup
    const int hb = NHW * part;
    const int kvg = p.kv_groups > 1 ? part : 0;
    const int t_begin = c * p.chunk;

    if (t_begin >= L) {
        if (c == 0) {  // empty sequence: out = 0, lse = -inf for this workgroup's heads
            uint16_t* ob = p.out + ((int64_t)b * kHeads + hb) * kHeadDim;
            for (int i = threadIdx.x; i < NHW * kHeadDim / 8; i += 512)
                reinterpret_cast<u32x4*>(ob)[i] = u32x4{0, 0, 0, 0};
            if (p.lse_out && threadIdx.x < NHW)
                p.lse_out[b * kHeads + hb + threadIdx.x] = -__builtin_inff();
        }
        return;
    }
    const int t_end = min(L, t_begin + p.chunk);
    const int nsteps = (t_end - t_begin + kStep - 1) / kStep;
    const int last_s = nsteps - 1;
    const bool single = (L + p.chunk - 1) / p.chunk == 1;

#define MFA_PIECE_TID threadIdx.x
#define MFA_PIECE_K c
#define MFA_PIECE_NPARTS ((L + p.chunk - 1) / p.chunk)
#define MFA_PIECE_BASE ((int64_t)b * p.n_chunk)
#include "mfa_attn_ws.inc"
#undef MFA_PIECE_TID
#undef MFA_PIECE_K
#undef MFA_PIECE_NPARTS
#undef MFA_PIECE_BASE
}

// The thread index through an opaque copy: in the balanced kernel's piece
// loop, values derived from it are then computed per piece instead of being
// hoisted out of the loop, where they would stay live across the step loop.
__device__ __forceinline__ int opaque_thread_index() {
    int t;
    asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"((int)threadIdx.x));
    return t;
}

// One piece of the balanced kernel: tokens [t_begin, t_end) of sequence b
// (length L, t_begin < L), the piece_k-th of the sequence's nparts pieces,
// whose partials sit at workspace slots part_base + 0 .. nparts-1.
template <bool FP8, bool PAGED, bool F8MMA>
__device__ __forceinline__ void attend_piece(const AttnArgs& p, const int b, const int L, const int t_begin,
                                                const int t_end, const int piece_k, const int nparts,
                                                const int64_t part_base) {
    constexpr int NHT = 4;
    const int hb = 0, kvg = 0;
    const int kvb = b;
    const int nsteps = (t_end - t_begin + kStep - 1) / kStep;
    const int last_s = nsteps - 1;
    const bool single = nparts == 1;
#define MFA_PIECE_TID opaque_thread_index()
#define MFA_PIECE_K piece_k
#define MFA_PIECE_NPARTS nparts
#define MFA_PIECE_BASE part_base
#include "mfa_attn_ws.inc"
#undef MFA_PIECE_TID
#undef MFA_PIECE_K
#undef MFA_PIECE_NPARTS
#undef MFA_PIECE_BASE
}

// out = 0, lse = -inf for an empty sequence.
__device__ __forceinline__ void write_empty(const AttnArgs& p, int b) {
    uint16_t* ob = p.out + (int64_t)b * kHeads * kHeadDim;
    for (int i = threadIdx.x; i < kHeads * kHeadDim / 8; i += blockDim.x)
        reinterpret_cast<u32x4*>(ob)[i] = u32x4{0, 0, 0, 0};
    if (p.lse_out && threadIdx.x < kHeads) p.lse_out[b * kHeads + threadIdx.x] = -__builtin_inff();
}

template <bool FP8, bool PAGED, bool F8MMA>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void mfa_attn_balanced_kernel(const AttnArgs p) {
    constexpr int NT = 512;               // threads
    constexpr int NW = NT / 64;           // waves
    __shared__ int wave_total[NW];
    __shared__ int first_seq[3];
    __shared__ unsigned empty_mask;   // bit j: sequence blockIdx.x + j*G is empty
    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int w = tid >> 6;
    const int B = p.batch;
    const int G = gridDim.x;
    auto steps_of_len = [](int len) { return (len + kStep - 1) / kStep; };
    // a sequence's share of the ranges: its steps plus kBalancedPieceCost
    // units for the fixed work of its piece (none when it is empty)
    auto units_of_len = [&](int len) {
        const int n = steps_of_len(len);
        return n > 0 ? n + kBalancedPieceCost : 0;
    };

    // prefix of the unit counts over sequences: thread t sums sequences
    // [t*per_t, (t+1)*per_t) (up to four lengths kept in registers, so
    // the lengths are read once), then a scan across the workgroup
    constexpr int kRegLens = 4;
    const int per_t = (B + NT - 1) / NT;
    const int b0 = min(B, tid * per_t), b1 = min(B, b0 + per_t);
    int lens[kRegLens];
    int cnt = 0;
    if (tid == 0) empty_mask = 0;
    __syncthreads();
    // the lengths are read here only: the empty sequences this workgroup
    // clears (b = blockIdx.x + j*G, j < 32) are noted in a mask
    auto note_empty = [&](int bb, int len) {
        if (len == 0 && bb % G == (int)blockIdx.x && bb / G < 32)
            atomicOr(&empty_mask, 1u << (bb / G));
    };
    if (per_t <= kRegLens) {
#pragma unroll
        for (int i = 0; i < kRegLens; i++) {
            lens[i] = b0 + i < b1 ? seq_len(p.kv, b0 + i) : 0;
            cnt += units_of_len(lens[i]);
        }
#pragma unroll
        for (int i = 0; i < kRegLens; i++)
            if (b0 + i < b1) note_empty(b0 + i, lens[i]);
    } else {
        for (int bb = b0; bb < b1; bb++) {
            const int len = seq_len(p.kv, bb);
            cnt += units_of_len(len);
            note_empty(bb, len);
        }
    }
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off);
        if (l >= off) incl += v;
    }
    if (l == 63) wave_total[w] = incl;
    __syncthreads();
    int excl = incl - cnt;
    for (int i = 0; i < w; i++) excl += wave_total[i];
    int total = 0;
#pragma unroll
    for (int i = 0; i < NW; i++) total += wave_total[i];
    const int per = min(kMaxPagedChunkSteps, max(kMinBalancedSteps, (total + G - 1) / G));
    const int s_lo = blockIdx.x * per;
    const int s_hi = min(total, s_lo + per);
    if (s_lo < total) {
        // the sequence holding unit s_lo, its first unit and its length
        if (excl <= s_lo && s_lo < excl + cnt) {
            int P = excl;
            for (int bb = b0; bb < b1; bb++) {
                int len;
                if (per_t <= kRegLens) {   // lens[bb - b0], by selects (no indexed register array)
                    len = lens[0];
#pragma unroll
                    for (int i = 1; i < kRegLens; i++) len = bb - b0 == i ? lens[i] : len;
                } else {
                    len = seq_len(p.kv, bb);
                }
                const int n = units_of_len(len);
                if (s_lo < P + n) {
                    first_seq[0] = bb;
                    first_seq[1] = P;
                    first_seq[2] = len;
                    break;
                }
                P += n;
            }
        }
        __syncthreads();
        int bq = __builtin_amdgcn_readfirstlane(first_seq[0]);
        int Pq = __builtin_amdgcn_readfirstlane(first_seq[1]);
        int L = __builtin_amdgcn_readfirstlane(first_seq[2]);
        // sequence bq takes units [Pq, Pq + units): the piece cost first,
        // then its steps from unit r0 = Pq + kBalancedPieceCost on
        for (;;) {
            const int n = steps_of_len(L);
            if (n > 0) {
                const int r0 = Pq + kBalancedPieceCost;
                const int lo = max(s_lo, r0), hi = min(s_hi, r0 + n);
                if (hi > lo) {
                    const int first = r0 / per, last = (r0 + n - 1) / per;
                    attend_piece<FP8, PAGED, F8MMA>(p, bq, L, (lo - r0) * kStep, min(L, (hi - r0) * kStep),
                                                    (int)blockIdx.x - first, last - first + 1,
                                                    (int64_t)bq * p.part_stride);
                }
                if (r0 + n >= s_hi) break;
                if (hi > lo) __syncthreads();   // the piece is done with the LDS
            }
            Pq += units_of_len(L);
            bq++;
            L = seq_len(p.kv, bq);
        }
    }
    // empty sequences b = blockIdx.x (mod G): out = 0, lse = -inf (from
    // the mask for the first 32, reading the length past that)
    const unsigned em = __builtin_amdgcn_readfirstlane(*(volatile unsigned*)&empty_mask);
    for (int j = 0; j < 32; j++)
        if (em & (1u << j)) write_empty(p, (int)blockIdx.x + j * G);
    for (int bb = (int)blockIdx.x + 32 * G; bb < B; bb += G)
        if (seq_len(p.kv, bb) == 0) write_empty(p, bb);
}


// Merge the chunk partials of every sequence with more than one chunk:
//   M = max_c lse2_c, W_c = 2^(lse2_c - M), out = sum_c W_c o_c / sum_c W_c,
//   lse = (M + log2 sum_c W_c) * ln 2.
// One workgroup per (sequence, head) of up to kCombineWaves waves (one per
// kCombineUnroll chunks of the longest sequence); wave k takes the k-th of
// equal ranges of the chunks, lane t columns 4t..4t+3.
// The first batch of rows is loaded before the maxima are known, so that a
// sequence of few chunks costs one memory round trip; later rows are read
// kCombineUnroll at a time. Each wave accumulates its range in chunk order,
// lane j holding the weight of chunk c0 + j of a 64-chunk block (broadcast
// with readlane); the waves' sums are added in wave order.
constexpr int kCombineWaves = 4;
constexpr int kCombineUnroll = 16;
__global__ __launch_bounds__(64 * kCombineWaves) void mfa_combine_kernel(const AttnArgs p) {
    __shared__ float red_m[kCombineWaves];
    __shared__ float red_w[kCombineWaves];
    __shared__ f32x4 red_acc[kCombineWaves][64];
    const int b = blockIdx.x >> 6;
    const int h = blockIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = blockDim.x >> 6;
    const int t = threadIdx.x & 63;
    // multi-token decode: query row b is token b % qtok of cache sequence b / qtok
    const int L = p.qtok > 1 ? max(0, seq_len(p.kv, b / p.qtok) - (p.qtok - 1 - b % p.qtok)) : seq_len(p.kv, b);
    const int nc = (L + p.chunk - 1) / p.chunk;
    if (nc <= p.fuse_max) return;   // merged by the attention kernel itself
    const int per = (nc + nw - 1) / nw;
    const int c_lo = min(nc, wv * per), c_hi = min(nc, c_lo + per);
    const int64_t base = (int64_t)b * p.n_chunk;
    const float* lse = p.part_lse + base * kHeads + h;   // chunk c at lse[c * kHeads]
    constexpr int64_t kRow = kHeads * kHeadDim / 4;      // 8-byte groups per chunk partial
    const u32x2* po = reinterpret_cast<const u32x2*>(p.part_o) + (base * kHeads + h) * (kHeadDim / 4) + t;
    auto row = [](u32x2 d) {
        return f32x4{__builtin_bit_cast(float, d.x << 16), __builtin_bit_cast(float, d.x & 0xffff0000u),
                     __builtin_bit_cast(float, d.y << 16), __builtin_bit_cast(float, d.y & 0xffff0000u)};
    };
    // rows of chunks c0 .. c0 + kCombineUnroll - 1, clamped into the range
    // (unconditional loads stay in flight together; the clamped ones are not
    // used)
    auto load_rows = [&](int c0, u32x2* v) {
#pragma unroll
        for (int j = 0; j < kCombineUnroll; j++) v[j] = po[(int64_t)min(c0 + j, c_hi - 1) * kRow];
    };

    u32x2 v[kCombineUnroll];
    if (c_lo < c_hi) load_rows(c_lo, v);
    // the maxima: this wave's range (the first 64 values kept), then the workgroup's
    const float l0 = c_lo + t < c_hi ? lse[(int64_t)(c_lo + t) * kHeads] : -__builtin_inff();
    float M = l0;
    for (int c = c_lo + 64 + t; c < c_hi; c += 64) M = fmaxf(M, lse[(int64_t)c * kHeads]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    if (t == 0) red_m[wv] = M;
    __syncthreads();
    M = red_m[0];
    for (int k = 1; k < nw; k++) M = fmaxf(M, red_m[k]);

    float wpart = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = c_lo; c0 < c_hi; c0 += 64) {
        const int n = min(64, c_hi - c0);
        // lane j: the weight of chunk c0 + j (0 past the range)
        const float lv = c0 == c_lo ? l0 : (t < n ? lse[(int64_t)(c0 + t) * kHeads] : -__builtin_inff());
        const float wl = t < n ? __builtin_amdgcn_exp2f(lv - M) : 0.f;
        wpart += wl;
        for (int i = 0; i < n; i += kCombineUnroll) {
            if (c0 != c_lo || i != 0) load_rows(c0 + i, v);
#pragma unroll
            for (int j = 0; j < kCombineUnroll; j++) {
                if (i + j >= n) break;
                const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), i + j));
                acc += wj * row(v[j]);
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) wpart += __shfl_xor(wpart, off);
    red_acc[wv][t] = acc;
    if (t == 0) red_w[wv] = wpart;
    __syncthreads();
    if (wv != 0) return;
    acc = red_acc[0][t];
    float wsum = red_w[0];
    for (int k = 1; k < nw; k++) {
        acc += red_acc[k][t];
        wsum += red_w[k];
    }
    const float inv = 1.f / wsum;
    uint16_t* orow = p.out + ((int64_t)b * kHeads + h) * kHeadDim + 4 * t;
    *reinterpret_cast<u32x2*>(orow) = u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv),
                                           pack_bf16x2(acc[2] * inv, acc[3] * inv)};
    if (p.lse_out && t == 0) p.lse_out[b * kHeads + h] = (M + __builtin_amdgcn_logf(wsum)) * kLn2;
}

// Copy the logical rows t < L_b of sequence b through the attention kernel's
// own address generation (PieceRows, with the page indices of a piece held in
// registers and read back per step). One wave per piece of kMaxPieceSteps
// steps; it copies each step's rows 16 bytes per lane.
template <bool PAGED>
__global__ __launch_bounds__(64) void mfa_gather_kernel(const KvView kv, int b, uint8_t* k_dst, uint8_t* v_dst) {
    const int L = seq_len(kv, b);
    const int t_begin = blockIdx.x * kMaxPieceSteps * kStep;
    if (t_begin >= L) return;
    const int l = threadIdx.x;
    const int t_end = min(L, t_begin + kMaxPieceSteps * kStep);
    const int nsteps = (t_end - t_begin + kStep - 1) / kStep;
    PieceRows<PAGED> rows;
    rows.init(kv, b, t_begin, nsteps, l);
    const int per_row = kv.row_bytes / 16;
    for (int s = 0; s < nsteps; s++) {
        const int64_t base = rows.step_row(kv, 0, s);
        const int t0 = t_begin + s * kStep;
        const int n = min(kStep, L - t0);
        for (int i = l; i < n * per_row; i += 64) {
            const int r = i / per_row, q = i - r * per_row;
            const int64_t src = (base + r) * kv.row_bytes + 16 * q;
            const int64_t dst = (int64_t)(t0 + r) * kv.row_bytes + 16 * q;
            *reinterpret_cast<u32x4*>(k_dst + dst) = *reinterpret_cast<const u32x4*>(kv.k + src);
            *reinterpret_cast<u32x4*>(v_dst + dst) = *reinterpret_cast<const u32x4*>(kv.v + src);
        }
    }
}

// One FP8 MFMA per tile, with the operand layout of the FP8-MFMA attention
// mode (mfma16_fp8): a [n][16][128] and b [n][128][16] E4M3 codes, c and d
// [n][16][16] fp32, row-major; lane l holds row l % 16 of A and column l % 16
// of B over k = 32 (l / 16) .. + 31, and D rows 4 (l / 16) .. + 3 of column
// l % 16.
__global__ __launch_bounds__(64) void mfa_fp8_mfma_kernel(const uint8_t* a, const uint8_t* b, const float* c,
                                                           float* d) {
    const int64_t t = blockIdx.x;
    const int l = threadIdx.x, r = l & 15, kq = l >> 4;
    const uint8_t* at = a + t * 16 * 128 + r * 128 + 32 * kq;
    const uint8_t* bt = b + t * 128 * 16 + (32 * kq) * 16 + r;
    i32x8 av, bv;
#pragma unroll
    for (int j = 0; j < 8; j++) {
        av[j] = *reinterpret_cast<const int*>(at + 4 * j);
        bv[j] = (int)((uint32_t)bt[(4 * j) * 16] | ((uint32_t)bt[(4 * j + 1) * 16] << 8) |
                      ((uint32_t)bt[(4 * j + 2) * 16] << 16) | ((uint32_t)bt[(4 * j + 3) * 16] << 24));
    }
    f32x4 acc;
#pragma unroll
    for (int i = 0; i < 4; i++) acc[i] = c ? c[t * 256 + (4 * kq + i) * 16 + r] : 0.f;
    acc = mfma16_fp8(av, bv, acc);
#pragma unroll
    for (int i = 0; i < 4; i++) d[t * 256 + (4 * kq + i) * 16 + r] = acc[i];
}

hipError_t launch_attn_split(const AttnArgs& a, bool fp8, bool paged, int workgroups, const Launch& l) {
    const dim3 grid(workgroups), block(512);
    if (a.fp8_mma) {   // FP8 cache only (checked by the caller)
        if (a.balanced)
            return paged ? launch_kernel(mfa_attn_balanced_kernel<true, true, true>, grid, block, l, a)
                         : launch_kernel(mfa_attn_balanced_kernel<true, false, true>, grid, block, l, a);
        if (a.nh == 2)
            return paged ? launch_kernel(mfa_attn_ws_split_kernel<true, true, false, true, 2>, grid, block, l, a)
                         : launch_kernel(mfa_attn_ws_split_kernel<true, false, false, true, 2>, grid, block, l, a);
        return paged ? launch_kernel(mfa_attn_ws_split_kernel<true, true, false, true, 4>, grid, block, l, a)
                     : launch_kernel(mfa_attn_ws_split_kernel<true, false, false, true, 4>, grid, block, l, a);
    }
    if (a.balanced) {
        if (fp8)
            return paged ? launch_kernel(mfa_attn_balanced_kernel<true, true, false>, grid, block, l, a)
                         : launch_kernel(mfa_attn_balanced_kernel<true, false, false>, grid, block, l, a);
        return paged ? launch_kernel(mfa_attn_balanced_kernel<false, true, false>, grid, block, l, a)
                     : launch_kernel(mfa_attn_balanced_kernel<false, false, false>, grid, block, l, a);
    }
    if (!fp8) {
        if (a.qtok > 1)
            return paged ? launch_kernel(mfa_attn_ws_split_kernel<false, true, true, false, 4>, grid, block, l, a)
                         : launch_kernel(mfa_attn_ws_split_kernel<false, false, true, false, 4>, grid, block, l, a);
        if (a.nh == 4)   // four head groups of 16 (or four K/V heads)
            return paged ? launch_kernel(mfa_attn_ws_split_kernel<false, true, false, false, 1>, grid, block, l, a)
                         : launch_kernel(mfa_attn_ws_split_kernel<false, false, false, false, 1>, grid, block, l, a);
        if (a.nh == 2)
            return paged ? launch_kernel(mfa_attn_ws_split_kernel<false, true, false, false, 2>, grid, block, l, a)
                         : launch_kernel(mfa_attn_ws_split_kernel<false, false, false, false, 2>, grid, block, l, a);
        return paged ? launch_kernel(mfa_attn_ws_split_kernel<false, true, false, false, 4>, grid, block, l, a)
                     : launch_kernel(mfa_attn_ws_split_kernel<false, false, false, false, 4>, grid, block, l, a);
    }
    if (a.qtok > 1)   // bf16 MFMAs, all 64 heads per workgroup (checked by the caller)
        return paged ? launch_kernel(mfa_attn_ws_split_kernel<true, true, true, false, 4>, grid, block, l, a)
                     : launch_kernel(mfa_attn_ws_split_kernel<true, false, true, false, 4>, grid, block, l, a);
    if (a.nh == 4)    // grouped-query caches with four K/V heads
        return paged ? launch_kernel(mfa_attn_ws_split_kernel<true, true, false, false, 1>, grid, block, l, a)
                     : launch_kernel(mfa_attn_ws_split_kernel<true, false, false, false, 1>, grid, block, l, a);
    if (a.nh == 2)
        return paged ? launch_kernel(mfa_attn_ws_split_kernel<true, true, false, false, 2>, grid, block, l, a)
                     : launch_kernel(mfa_attn_ws_split_kernel<true, false, false, false, 2>, grid, block, l, a);
    return paged ? launch_kernel(mfa_attn_ws_split_kernel<true, true, false, false, 4>, grid, block, l, a)
                 : launch_kernel(mfa_attn_ws_split_kernel<true, false, false, false, 4>, grid, block, l, a);
}

hipError_t launch_combine(const AttnArgs& a, int batch, const Launch& l) {
    const int waves = std::min(kCombineWaves, std::max(1, (a.n_chunk + kCombineUnroll - 1) / kCombineUnroll));
    return launch_kernel(mfa_combine_kernel, dim3(batch * kHeads), dim3(64 * waves), l, a);
}

hipError_t launch_gather(const KvView& kv, bool paged, int b, int max_seq_len, void* k_dst,
                         void* v_dst, const Launch& l) {
    const int nblk = (max_seq_len + kMaxPieceSteps * kStep - 1) / (kMaxPieceSteps * kStep);
    if (nblk == 0) return hipSuccess;
    return launch_kernel(paged ? mfa_gather_kernel<true> : mfa_gather_kernel<false>, dim3(nblk), dim3(64), l, kv,
                         b, (uint8_t*)k_dst, (uint8_t*)v_dst);
}

__global__ __launch_bounds__(256) void mfa_fill_zero_kernel(uint32_t* p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0;
}

hipError_t launch_fill_zero(uint32_t* p, size_t n, const Launch& l) {
    if (n == 0) return hipSuccess;
    const size_t blocks = std::min<size_t>((n + 255) / 256, 1024);
    return launch_kernel(mfa_fill_zero_kernel, dim3((unsigned)blocks), dim3(256), l, p, n);
}

hipError_t launch_fp8_mfma(const uint8_t* a, const uint8_t* b, const float* c, float* d, int n_tiles,
                           const Launch& l) {
    return launch_kernel(mfa_fp8_mfma_kernel, dim3(n_tiles), dim3(64), l, a, b, c, d);
}

}  // namespace mfa
