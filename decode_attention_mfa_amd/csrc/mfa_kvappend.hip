// mfa_kvappend.hip -- the cache write of the KV append: the new token's key
// and value rows (one shared K head and one shared V head of 256, "Step-3 is
// Large yet Affordable", Key points) go to row L_b of sequence b, in the
// cache's format: bf16, or the FP8 E4M3 code of value / scale (the FP8
// deployment of the same Key points), contiguous or in 64-token pages
// (PagedAttention, cited by title on the Step-3 references).
//
// The projections themselves run in the skinny GEMM (mfa_qproj.hip) as fp32
// partials over K splits; this kernel sums the partials in split order,
// encodes and writes. One workgroup per sequence, one column per thread.
#include "mfa_device.h"
#include "mfa_internal.h"

namespace mfa {

namespace {

// bf16 bits of f, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// OCP E4M3FN code of f, round to nearest even. The format has no infinities:
// finite values from 448 (its largest) up, and infinities, saturate to +-448;
// NaN gives S.1111.111. A normal float keeps its top 3 mantissa bits with the
// 20 below rounded away in integer arithmetic (a carry moves into the
// exponent by itself); E4M3's exponent bias is 7 against float's 127. Below
// 2^-6 the codes are the multiples of 2^-9.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float f) {
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return sign | 0x7fu;
    if (a >= 0x43e00000u) return sign | 0x7eu;          // |f| >= 448
    if (a < 0x3c800000u)                                 // |f| < 2^-6
        return sign | (uint32_t)__builtin_rintf(__builtin_bit_cast(float, a) * 512.0f);
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
    return sign | ((r >> 20) - ((127u - 7u) << 3));
}

}  // namespace

// Block b: sequence b. Row L_b is written when L_b >= 0 and the row exists:
// contiguous, L_b < kv_stride; paged, the page-table slot L_b / 64 exists and
// names a page in [0, num_pages). Otherwise nothing is written.
// K splits whose partials are loaded all at once (7168 / 256 = 28 at the
// model's hidden size)
constexpr int kWriteBatch = 32;

template <bool FP8, bool PAGED>
__global__ __launch_bounds__(256) void mfa_kv_write_kernel(KvAppendArgs a) {
    const int b = blockIdx.x;
    const int t = a.seq_lens[b];
    if (t < 0) return;
    int64_t row;
    if constexpr (PAGED) {
        if (t / kPage >= a.pt_stride) return;
        const int page = a.page_table[(int64_t)b * a.pt_stride + t / kPage];
        if (page < 0 || page >= a.num_pages) return;
        row = (int64_t)page * kPage + (t & (kPage - 1));
    } else {
        if (t >= a.kv_stride) return;
        row = (int64_t)b * a.kv_stride + t;
    }
    const int j = threadIdx.x;
    const int64_t plane = (int64_t)a.batch * kHeadDim;
    const float* kp = a.kv_part + (int64_t)b * kHeadDim + j;
    const float* vp = kp + a.ksplit * plane;
    float ks = 0.f, vs = 0.f;
    int s = 0;
    if (a.ksplit <= kWriteBatch) {
        // every partial of this column requested before the first is added:
        // one memory round trip; the sums still run in split order
        float kr[kWriteBatch], vr[kWriteBatch];
#pragma unroll
        for (int u = 0; u < kWriteBatch; u++) {
            kr[u] = u < a.ksplit ? kp[u * plane] : 0.f;
            vr[u] = u < a.ksplit ? vp[u * plane] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kWriteBatch; u++) {
            if (u < a.ksplit) {
                ks += kr[u];
                vs += vr[u];
            }
        }
        s = a.ksplit;
    }
    for (; s + 8 <= a.ksplit; s += 8) {
        float kr[8], vr[8];
#pragma unroll
        for (int u = 0; u < 8; u++) {
            kr[u] = kp[(s + u) * plane];
            vr[u] = vp[(s + u) * plane];
        }
#pragma unroll
        for (int u = 0; u < 8; u++) {
            ks += kr[u];
            vs += vr[u];
        }
    }
    for (; s < a.ksplit; s++) {
        ks += kp[s * plane];
        vs += vp[s * plane];
    }
    const int64_t e = row * kHeadDim + j;
    if constexpr (FP8) {
        a.k[e] = (uint8_t)e4m3_rne_sat(ks / a.k_scale);
        a.v[e] = (uint8_t)e4m3_rne_sat(vs / a.v_scale);
    } else {
        reinterpret_cast<uint16_t*>(a.k)[e] = (uint16_t)bf16_rne(ks);
        reinterpret_cast<uint16_t*>(a.v)[e] = (uint16_t)bf16_rne(vs);
    }
}

hipError_t launch_kv_write(const KvAppendArgs& a, bool fp8, bool paged, const Launch& l) {
    auto kern = fp8 ? (paged ? mfa_kv_write_kernel<true, true> : mfa_kv_write_kernel<true, false>)
                    : (paged ? mfa_kv_write_kernel<false, true> : mfa_kv_write_kernel<false, false>);
    return launch_kernel(kern, dim3(a.batch), dim3(kHeadDim), l, a);
}

}  // namespace mfa
