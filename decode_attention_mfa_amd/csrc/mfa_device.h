// mfa_device.h -- device-side helpers shared by the MFA kernels (gfx950).
//
// Vector types for the CDNA4 matrix cores, FP8 E4M3 -> bf16 conversion in
// registers, and the KV-cache address generation (PieceRows) that both the
// attention kernel and the debug gather use, so that the paging test checks
// the attention kernel's own addressing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mfa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kHeads = 64;      // query heads sharing one K/V head
constexpr int kHeadDim = 256;   // head dimension of Q, K and V
constexpr int kPage = 64;       // tokens per cache page
constexpr int kStep = 64;       // tokens per attention step (one page)
constexpr int kLatent = 512;    // latent row of the latent-cache (MLA-style) comparison mode
constexpr float kLn2 = 0.69314718055994530942f;
// Headroom (base-2 exponent) a score may exceed its head's reference maximum
// before the chunk is redone with a higher reference: unnormalised P stays
// <= 2^kTau, so with |V| < 2^64 the fp32 accumulators cannot overflow.
constexpr float kTau = 48.0f;
// With FP8 P (the FP8-MFMA mode) the excess is bounded by 2^6, so that P * 4
// stays below E4M3's 448 (and a restart stays rare: the later scores of a
// piece seldom exceed its first step's maxima by six octaves).
constexpr float kTauF8 = 6.0f;

template <typename T, typename S>
__device__ __forceinline__ T bitcast(const S& s) {
    static_assert(sizeof(T) == sizeof(S), "size mismatch");
    return __builtin_bit_cast(T, s);
}

// 16x16x32 bf16 MFMA, fp32 accumulate. Lane l holds A[l%16][8*(l/16)+j],
// B[8*(l/16)+j][l%16] (j = 0..7) and D[4*(l/16)+i][l%16] (i = 0..3).
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// FP8 (E4M3 x E4M3) MFMAs, unscaled: 16x16x128 (A: lane l holds row l%16,
// k = 32(l/16) + byte; B the same with column l%16; C as mfma16) and
// 32x32x64 (A: row l%32, k = 32(l/32) + byte; C: lane l holds column l%32,
// rows 8(i/4) + 4(l/32) + i%4 for i < 16).
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x4 mfma16_fp8(const i32x8& a, const i32x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Four E4M3FN codes (one dword, byte 0 first) -> four bf16, exactly: every
// E4M3 value is a bf16 value. Scale 1.0 leaves values unchanged.
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t w) {
    bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    return u32x2{bitcast<uint32_t>(lo), bitcast<uint32_t>(hi)};
}

// Eight E4M3 codes (two dwords) -> a bf16x8 MFMA operand.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1) {
    u32x2 a = e4m3x4_to_bf16x4(w0);
    u32x2 b = e4m3x4_to_bf16x4(w1);
    return bitcast<bf16x8>(u32x4{a.x, a.y, b.x, b.y});
}

// Larger of two floats by the IEEE maximum operation (a NaN input gives NaN):
// gfx950 has it in a three-input form, and unlike fmaxf it needs no quieting
// of its inputs first.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2 v = {(__bf16)a, (__bf16)b};  // round to nearest even
    return bitcast<uint32_t>(v);
}

__device__ __forceinline__ float bf16_round(float a) {
    return (float)(__bf16)a;
}

// KV cache view used on the device.
struct KvView {
    const uint8_t* k;
    const uint8_t* v;
    const int32_t* seq_lens;
    const int32_t* page_table;  // nullptr: contiguous
    int64_t kv_stride;          // contiguous: token slots per sequence
    int32_t pt_stride;
    int32_t row_bytes;          // 256 * element size
    int32_t max_len;            // launch bound on sequence lengths
    int32_t groups;             // K/V heads per token (1 for MFA; G for grouped-query caches)
};

// Length of sequence b as the kernels use it: seq_lens[b] clamped to
// [0, max_len], so a bad length can never address rows past the launch bound.
__device__ __forceinline__ int seq_len(const KvView& kv, int b) {
    return min(max(kv.seq_lens[b], 0), kv.max_len);
}

// Row index of token t of sequence b. For a paged cache the page of token t
// is page_table[b][t / 64] and the row inside it t % 64.
template <bool PAGED>
__device__ __forceinline__ int64_t kv_row(const KvView& kv, int b, int t) {
    if constexpr (PAGED) {
        int32_t page = kv.page_table[(int64_t)b * kv.pt_stride + (t >> 6)];
        return (int64_t)page * kPage + (t & (kPage - 1));
    } else {
        return (int64_t)b * kv.kv_stride + t;
    }
}

// Row index of the first token of the 64-token step starting at t0 (a
// multiple of 64). All tokens t0..t0+63 are rows base+0..base+63.
template <bool PAGED>
__device__ __forceinline__ int64_t kv_step_base(const KvView& kv, int b, int t0) {
    return kv_row<PAGED>(kv, b, t0);
}

// The same in K/V head g of a grouped cache: contiguous [B][G][kv_stride]
// rows, pages [P][G][64] rows (G = kv.groups; g = 0 with G = 1 is
// kv_step_base).
template <bool PAGED>
__device__ __forceinline__ int64_t kv_group_step_base(const KvView& kv, int b, int g, int t0) {
    if constexpr (PAGED) {
        const int32_t page = kv.page_table[(int64_t)b * kv.pt_stride + (t0 >> 6)];
        return ((int64_t)page * kv.groups + g) * kPage;
    } else {
        return ((int64_t)b * kv.groups + g) * kv.kv_stride + t0;
    }
}

// The rows of the 64-token steps of one piece (tokens [t_begin, ...) of
// sequence b, t_begin a multiple of 64, at most kMaxPieceSteps steps), as the
// attention kernel and the debug gather address them. For a paged cache lane
// j of the wave holds the page of step j (pg0) and of step 64 + j (pg1),
// loaded once; a step reads its page back with v_readlane, so no page-table
// load sits in a step loop. Step s covers rows step_row(s) .. step_row(s)+63
// of K/V head g.
constexpr int kMaxPieceSteps = 128;
template <bool PAGED>
struct PieceRows {
    int32_t pg0 = 0, pg1 = 0;
    int32_t b = 0, t_begin = 0;

    __device__ __forceinline__ void init(const KvView& kv, int b_, int t_begin_, int nsteps, int lane) {
        b = b_;
        t_begin = t_begin_;
        if constexpr (PAGED) {
            const int32_t* pt = kv.page_table + (int64_t)b * kv.pt_stride + (t_begin >> 6);
            if (lane < nsteps) pg0 = pt[lane];
            if (64 + lane < nsteps) pg1 = pt[64 + lane];
        }
    }
    // s must be wave-uniform
    __device__ __forceinline__ int64_t step_row(const KvView& kv, int g, int s) const {
        if constexpr (PAGED) {
            const int32_t page = s < 64 ? __builtin_amdgcn_readlane(pg0, s) : __builtin_amdgcn_readlane(pg1, s - 64);
            return ((int64_t)page * kv.groups + g) * kPage;
        } else {
            return kv_group_step_base<false>(kv, b, g, t_begin + s * kStep);
        }
    }
};

}  // namespace mfa
