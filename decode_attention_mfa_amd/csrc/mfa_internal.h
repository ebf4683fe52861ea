// mfa_internal.h -- launch interface between the C ABI (mfa_api.hip) and the
// kernels (mfa_attn.hip, mfa_qproj.hip). Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mfa_device.h"

namespace mfa {

struct AttnArgs {
    const uint16_t* q;      // [B][64][256] bf16
    KvView kv;
    uint16_t* out;          // [B][64][256] bf16
    float* lse_out;         // [B][64] or nullptr
    float* part_o;          // workspace [B * n_chunk][64][256] fp32
    float* part_lse;        // workspace [B * n_chunk][64] fp32, base-2
    int32_t chunk;          // tokens per split chunk, multiple of 64
    int32_t n_chunk;        // chunks per sequence slot in the launch = ceil(max_seq_len / chunk)
    float score_scale;      // softmax_scale * k_scale * log2(e)
    float v_scale;          // 1 for bf16
};

hipError_t launch_attn_split(const AttnArgs& a, bool fp8, bool paged, int batch, hipStream_t st);
hipError_t launch_combine(const AttnArgs& a, int batch, hipStream_t st);
hipError_t launch_gather(const KvView& kv, bool paged, int b, int max_seq_len, void* k_dst,
                         void* v_dst, hipStream_t st);

struct QprojArgs {
    const uint16_t* x;      // [B][hidden]
    const uint16_t* w_qa;   // [hidden][rank]
    const uint16_t* rms_w;  // [rank]
    const uint16_t* w_qb;   // [rank][nq]
    uint16_t* q_out;        // [B][nq]
    float* c_part;          // workspace [ksplit][B][rank] fp32
    uint16_t* chat;         // workspace [B][rank] bf16
    int32_t batch, hidden, rank, nq, ksplit;
    float eps;
};

constexpr int kQprojSplit = 8;   // K-splits of the down-projection

hipError_t launch_qproj_down(const QprojArgs& a, hipStream_t st);
hipError_t launch_rmsnorm(const QprojArgs& a, hipStream_t st);
hipError_t launch_qproj_up(const QprojArgs& a, hipStream_t st);

}  // namespace mfa
