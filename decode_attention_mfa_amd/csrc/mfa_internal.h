// mfa_internal.h -- launch interface between the C ABI (mfa_api.hip) and the
// kernels (mfa_attn.hip, mfa_qproj.hip). Not installed, not part of the ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mfa_device.h"

namespace mfa {

// Where a kernel goes: the stream and, when timing is on, an event pair that
// hipExtLaunchKernel stamps with the kernel's own start and end (no marker
// packets between kernels, so the times match a kernel trace).
struct Launch {
    hipStream_t st;
    hipEvent_t start = nullptr, stop = nullptr;
};

template <typename... KArgs, typename... Args>
inline hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, const Launch& l,
                                Args... args) {
    hipExtLaunchKernelGGL(kernel, grid, block, 0, l.st, l.start, l.stop, 0, args...);
    return hipGetLastError();
}

struct AttnArgs {
    const uint16_t* q;      // [B][64][256] bf16
    KvView kv;
    uint16_t* out;          // [B][64][256] bf16
    float* lse_out;         // [B][64] or nullptr
    float* part_o;          // workspace: B * n_chunk slots of 32 KB; bf16 [64][256] partial rows (mfa_combine_kernel) or bf16 dumps of in-kernel merges
    float* part_lse;        // workspace [B * n_chunk][64] fp32, base-2
    int32_t* counters;      // workspace [B][nh] arrival counts (nh <= 4), zero between calls
    int32_t chunk;          // tokens per split chunk, multiple of 64
    int32_t n_chunk;        // chunks per sequence slot in the launch = ceil(max_seq_len / chunk)
    int32_t fuse_max;       // sequences with 2..fuse_max chunks are merged in the attention kernel
    float score_scale;      // softmax_scale * k_scale * log2(e)
    float v_scale;          // 1 for bf16
    int32_t balanced;       // 1: equal step ranges per workgroup (chunk, n_chunk unused)
    int32_t batch;          // cache sequences in the call (balanced and multi-token modes)
    int32_t qtok;           // query tokens per sequence (1, or t for multi-token decode)
    int32_t fp8_mma;        // 1: FP8 MFMAs for S and P.V (quantised Q and P)
    int32_t part_stride;    // workspace partial slots per sequence (balanced mode)
    int32_t nh;             // workgroups per (query row set, chunk), each taking 64 / nh heads
    int32_t kv_groups;      // K/V heads G of the cache (1: MFA); with G > 1, nh = G and workgroup i reads head i
};

// Balanced mode: each workgroup takes at least this many 64-token steps, so
// that a sequence is cut into at most ceil(steps / 4) + 1 pieces (the
// workspace holds ceil(max_context / 256) + 1 partial slots per sequence).
constexpr int kMinBalancedSteps = 4;

// Balanced mode: the ranges deal out units, a sequence's steps plus this many
// for the fixed work of its piece (the Q fetch, the ring's first loads, the
// first step's maxima, the epilogue), so that a range holding the starts of
// several short sequences gets fewer steps. Measured on 384 sequences of
// 1024..8192 tokens: 3 units 207.4 us, 5: 204.5, 8: 201.8, 12: 205.1.
constexpr int kBalancedPieceCost = 8;

// Multi-token decode: at most this many query tokens per sequence.
constexpr int kMaxQueryTokens = 16;

// Launches whose sequences all have at most this many chunks merge them
// inside the attention kernel (the last chunk to finish does it); other
// launches run mfa_combine_kernel afterwards. With more chunks the serial
// merge at the tail costs more than the second launch.
constexpr int kFusedMaxChunks = 2;

// Paged caches: at most this many 64-token steps per split chunk (the
// attention kernel keeps a chunk's page indices in two registers per lane).
constexpr int kMaxPagedChunkSteps = kMaxPieceSteps;

hipError_t launch_attn_split(const AttnArgs& a, bool fp8, bool paged, int workgroups, const Launch& l);
hipError_t launch_combine(const AttnArgs& a, int batch, const Launch& l);
// Latent-cache mode (mfa_mla.hip): q, out [batch][64][512]; kv.k holds the
// E4M3 latent rows; chunks of a.chunk tokens, two workgroups of 32 heads per
// (row, chunk); partials in 64 KB workspace slots, merged by the second launch
hipError_t launch_mla(const AttnArgs& a, bool paged, const Launch& l);
hipError_t launch_mla_combine(const AttnArgs& a, const Launch& l);
hipError_t launch_gather(const KvView& kv, bool paged, int b, int max_seq_len, void* k_dst,
                         void* v_dst, const Launch& l);
// n 32-bit words at p set to zero by a kernel (capturable in a graph, unlike
// a memset node)
hipError_t launch_fill_zero(uint32_t* p, size_t n, const Launch& l);
// n_tiles FP8 MFMAs (16 x 16 x 128, E4M3 operands) as the FP8-MFMA attention
// mode runs them: d = a . b + c per tile (c may be null: zero)
hipError_t launch_fp8_mfma(const uint8_t* a, const uint8_t* b, const float* c, float* d, int n_tiles,
                           const Launch& l);
// the matrix-core rate microbenchmark (kind 0: bf16 16x16x32, 1: E4M3
// 16x16x128): `workgroups` of four waves, each running `iters` rounds of
// independent MFMAs on register operands; the flops of such a launch
hipError_t launch_mfma_rate(int kind, int iters, int workgroups, float* sink, const Launch& l);
double mfma_rate_flops(int kind, int iters, int workgroups);

struct QprojArgs {
    const uint16_t* x;      // [B][hidden]
    const uint16_t* w_qa;   // [hidden][rank]
    const uint16_t* rms_w;  // [rank]
    const uint16_t* w_qb;   // [rank][nq]
    uint16_t* q_out;        // [B][nq]
    float* c_part;          // workspace [ksplit][B][rank] fp32
    uint16_t* chat;         // workspace [B][rank] bf16: c * gamma
    float* sumsq;           // workspace [B][rank/64]: per row and column block, sum of c^2
    int32_t* counters;      // workspace [ceil(B/32)][rank/64] arrival counts, zero between calls
    int32_t batch, hidden, rank, nq, ksplit;
    float eps;
};

// The fused RMSNorm keeps one sum of squares per 64-column block of the
// bottleneck per row in LDS: q_rank <= 64 * kMaxNormBlocks.
constexpr int kMaxNormBlocks = 64;

// Epilogues of the skinny GEMM (see mfa_skinny_gemm_kernel).
enum { kEpiPartials = 0, kEpiBf16 = 1, kEpiNormPrep = 2, kEpiBf16RowScale = 3 };
struct GemmEpi {
    const uint16_t* gamma;
    uint16_t* cg;
    float* sumsq;
    int32_t* counters;
    float eps;
    int32_t rank;
};

// The down-projection splits K into blocks of this many rows or twice as many
// (one workgroup each per column block; fp32 partials, summed by the last
// workgroup of the column block to finish); hidden must be a multiple of it.
constexpr int kQprojRowsPerSplit = 512;

struct KvAppendArgs {
    const uint16_t* x;      // [B][hidden]
    const uint16_t* w_k;    // [hidden][256]
    const uint16_t* w_v;    // [hidden][256]
    float* kv_part;         // workspace [2][ksplit][B][256] fp32 (K partials, then V)
    uint8_t* k;             // cache written at row L_b (contiguous or paged)
    uint8_t* v;
    const int32_t* seq_lens;
    const int32_t* page_table;  // nullptr: contiguous
    int64_t kv_stride;
    int32_t pt_stride, num_pages;
    int32_t batch, hidden, ksplit;
    float k_scale, v_scale;     // FP8: the stored code is E4M3(value / scale); unused for bf16
};

// The K/V projections split K into blocks of this many rows (hidden is a
// multiple of 512, so of this too).
constexpr int kKvRowsPerSplit = 256;

hipError_t launch_kv_proj(const KvAppendArgs& a, const Launch& l);
hipError_t launch_kv_write(const KvAppendArgs& a, bool fp8, bool paged, const Launch& l);

hipError_t launch_qproj_down(const QprojArgs& a, const Launch& l);
hipError_t launch_qproj_up(const QprojArgs& a, const Launch& l);

}  // namespace mfa
