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
#include "mfa_device.h"
#include "mfa_internal.h"

namespace mfa {

// V slice rows in LDS: 64 tokens x (64 columns * elem) bytes, 16-byte chunks
// XOR-swizzled per row so that the transposed reads hit distinct banks.
__device__ __forceinline__ int vswz_fp8(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int vswz_bf16(int row) { return ((row >> 1) & 3) << 1; }
// P rows in LDS: 64 heads x 64 tokens bf16 (128 B), chunk swizzle by head.
__device__ __forceinline__ int pswz(int h) { return (h >> 1) & 7; }

template <bool FP8>
struct StepRegs {
    static constexpr int NK = FP8 ? 4 : 8;   // 16-byte K pieces per lane
    static constexpr int NV = FP8 ? 4 : 8;   // 16-byte V pieces per lane
    u32x4 k[NK];
    u32x4 v[NV];
};

template <bool FP8, bool PAGED>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void mfa_attn_split_kernel(const AttnArgs p) {
    constexpr int ELEM = FP8 ? 1 : 2;
    constexpr int ROWB = kHeadDim * ELEM;          // bytes per cached row
    constexpr int VROWB = 64 * ELEM;               // bytes per row of a wave's V slice
    constexpr int NK = StepRegs<FP8>::NK;
    constexpr int NV = StepRegs<FP8>::NV;

    __shared__ __attribute__((aligned(16))) uint8_t vlds_all[4 * 64 * VROWB];
    __shared__ __attribute__((aligned(16))) uint8_t plds[kHeads * 64 * 2];
    __shared__ float xchg[4][kHeads];

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

    uint8_t* vlds = vlds_all + w * 64 * VROWB;

    auto load_step = [&](int s, StepRegs<FP8>& r) {
        const int t0 = t_begin + s * kStep;
        const int last = t_end - 1 - t0;                 // last valid local token (>= 0)
        const int64_t base = kv_step_base<PAGED>(p.kv, b, t0);
        {   // K rows of this wave's 16 tokens, MFMA A-operand layout
            const int tl = min(16 * w + lr, last);
            const uint8_t* row = p.kv.k + (base + tl) * ROWB;
#pragma unroll
            for (int i = 0; i < NK; i++) {
                const int off = FP8 ? (64 * i + 16 * g) : (128 * (i >> 1) + 32 * g + 16 * (i & 1));
                r.k[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + off));
            }
        }
#pragma unroll
        for (int i = 0; i < NV; i++) {  // V slice: columns 64w..64w+63 of all 64 tokens
            const int tl = FP8 ? (16 * i + (l >> 2)) : (8 * i + (l >> 3));
            const int ch = FP8 ? (l & 3) : (l & 7);
            const uint8_t* row = p.kv.v + (base + min(tl, last)) * ROWB + 64 * w * ELEM;
            r.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + 16 * ch));
        }
    };

    // running state
    float mq[4];        // running max (base 2) of heads 16ht + lr   (QK layout)
    float lq[4];        // partial softmax denominators, same heads
    float mp[4][4];     // running max of heads 16ht + 4g + i        (PV layout)
    f32x4 o[4][4];      // O[16ht + 4g + i][64w + 16dt + lr]
#pragma unroll
    for (int ht = 0; ht < 4; ht++) {
        mq[ht] = -__builtin_inff();
        lq[ht] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; i++) mp[ht][i] = -__builtin_inff();
#pragma unroll
        for (int dt = 0; dt < 4; dt++) o[ht][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    auto compute_step = [&](int s, const StepRegs<FP8>& r) {
        const int t0 = t_begin + s * kStep;
        // (1) this wave's V slice -> LDS (its own region; program order keeps
        // the previous step's reads ahead of these writes)
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
            *reinterpret_cast<u32x4*>(vlds + row * VROWB + 16 * ch) = r.v[i];
        }
        // (2) scores S^T[token 4g+i][head 16ht+lr] for this wave's 16 tokens
        f32x4 sc[4];
#pragma unroll
        for (int ht = 0; ht < 4; ht++) sc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (FP8) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const bf16x8 a0 = e4m3x8_to_bf16x8(r.k[i].x, r.k[i].y);
                const bf16x8 a1 = e4m3x8_to_bf16x8(r.k[i].z, r.k[i].w);
#pragma unroll
                for (int ht = 0; ht < 4; ht++) {
                    sc[ht] = mfma16(a0, qop[ht][2 * i], sc[ht]);
                    sc[ht] = mfma16(a1, qop[ht][2 * i + 1], sc[ht]);
                }
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < 8; ks++) {
                const bf16x8 a = bitcast<bf16x8>(r.k[ks]);
#pragma unroll
                for (int ht = 0; ht < 4; ht++) sc[ht] = mfma16(a, qop[ht][ks], sc[ht]);
            }
        }
        // (3) mask tokens past the chunk end, per-head max over the wave's tokens
        const int valid = t_end - t0 - (16 * w + 4 * g);   // rows i < valid are real tokens
        float mx[4];
#pragma unroll
        for (int ht = 0; ht < 4; ht++) {
#pragma unroll
            for (int i = 0; i < 4; i++)
                if (i >= valid) sc[ht][i] = -__builtin_inff();
            float m = fmaxf(fmaxf(sc[ht][0], sc[ht][1]), fmaxf(sc[ht][2], sc[ht][3]));
            m = fmaxf(m, __shfl_xor(m, 16));
            m = fmaxf(m, __shfl_xor(m, 32));
            mx[ht] = m * p.score_scale;
        }
        if (g == 0) {
#pragma unroll
            for (int ht = 0; ht < 4; ht++) xchg[w][16 * ht + lr] = mx[ht];
        }
        __syncthreads();
        // (4) new running maxima, identical in every wave
        float mq_new[4], alpha_q[4];
#pragma unroll
        for (int ht = 0; ht < 4; ht++) {
            const int h = 16 * ht + lr;
            float m = fmaxf(fmaxf(xchg[0][h], xchg[1][h]), fmaxf(xchg[2][h], xchg[3][h]));
            mq_new[ht] = fmaxf(mq[ht], m);
            alpha_q[ht] = __builtin_amdgcn_exp2f(mq[ht] - mq_new[ht]);
        }
        float alpha_p[4][4];
#pragma unroll
        for (int ht = 0; ht < 4; ht++) {
            const int h0 = 16 * ht + 4 * g;
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(&xchg[0][h0]);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(&xchg[1][h0]);
            const f32x4 x2 = *reinterpret_cast<const f32x4*>(&xchg[2][h0]);
            const f32x4 x3 = *reinterpret_cast<const f32x4*>(&xchg[3][h0]);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float m = fmaxf(mp[ht][i], fmaxf(fmaxf(x0[i], x1[i]), fmaxf(x2[i], x3[i])));
                alpha_p[ht][i] = __builtin_amdgcn_exp2f(mp[ht][i] - m);
                mp[ht][i] = m;
            }
        }
        // (5) P = exp2(s2 - m), bf16; partial denominators from the rounded P
#pragma unroll
        for (int ht = 0; ht < 4; ht++) {
            float pr[4];
            float sum = 0.f;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[ht][i], p.score_scale, -mq_new[ht]));
                pr[i] = bf16_round(pr[i]);
                sum += pr[i];
            }
            lq[ht] = lq[ht] * alpha_q[ht] + sum;
            mq[ht] = mq_new[ht];
            const int h = 16 * ht + lr;
            const int ch = (2 * w + (g >> 1)) ^ pswz(h);
            *reinterpret_cast<u32x2*>(plds + h * 128 + 16 * ch + 8 * (g & 1)) =
                u32x2{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])};
        }
        // (6) rescale the output accumulators to the new maxima
#pragma unroll
        for (int ht = 0; ht < 4; ht++)
#pragma unroll
            for (int dt = 0; dt < 4; dt++)
#pragma unroll
                for (int i = 0; i < 4; i++) o[ht][dt][i] *= alpha_p[ht][i];
        __syncthreads();
        // (7) O[64 heads][64w..64w+63] += P[64 x 64 tok] . V[64 tok x 64]
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

    // ---- main loop: two register sets, the next step loading during compute
    StepRegs<FP8> ra, rb;
    load_step(0, ra);
    for (int s = 0; s < nsteps; s += 2) {
        if (s + 1 < nsteps) load_step(s + 1, rb);
        compute_step(s, ra);
        if (s + 1 < nsteps) {
            if (s + 2 < nsteps) load_step(s + 2, ra);
            compute_step(s + 1, rb);
        }
    }

    // ---- denominators: lanes -> wave (xor over g) -> workgroup (LDS)
#pragma unroll
    for (int ht = 0; ht < 4; ht++) {
        float v = lq[ht];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        lq[ht] = v;
    }
    __syncthreads();   // all waves are done reading xchg
    if (g == 0) {
#pragma unroll
        for (int ht = 0; ht < 4; ht++) xchg[w][16 * ht + lr] = lq[ht];
    }
    __syncthreads();

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
            const float lsum = ((l0[i] + l1[i]) + l2[i]) + l3[i];
            const float inv = p.v_scale / lsum;
            const float lse2 = mp[ht][i] + __builtin_amdgcn_logf(lsum);  // v_log_f32 is log2
            if (single) {
                uint16_t* orow = p.out + ((int64_t)b * kHeads + h) * kHeadDim + col;
#pragma unroll
                for (int dt = 0; dt < 4; dt++)
                    orow[16 * dt] = bitcast<uint16_t>((__bf16)(o[ht][dt][i] * inv));
                if (p.lse_out && w == 0 && lr == 0) p.lse_out[b * kHeads + h] = lse2 * kLn2;
            } else {
                const int64_t pidx = (int64_t)b * p.n_chunk + c;
                float* prow = p.part_o + (pidx * kHeads + h) * kHeadDim + col;
#pragma unroll
                for (int dt = 0; dt < 4; dt++) prow[16 * dt] = o[ht][dt][i] * inv;
                if (w == 0 && lr == 0) p.part_lse[pidx * kHeads + h] = lse2;
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

hipError_t launch_attention(const AttnArgs& a, bool fp8, bool paged, int batch, hipStream_t st) {
    const dim3 grid(batch * a.n_chunk), block(256);
    if (fp8) {
        if (paged) hipLaunchKernelGGL((mfa_attn_split_kernel<true, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((mfa_attn_split_kernel<true, false>), grid, block, 0, st, a);
    } else {
        if (paged) hipLaunchKernelGGL((mfa_attn_split_kernel<false, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((mfa_attn_split_kernel<false, false>), grid, block, 0, st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_chunk <= 1) return e;
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
