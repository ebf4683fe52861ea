/*
 * mfa.h -- C ABI of the MI355X (gfx950) decode step of Multi-Matrix
 * Factorization Attention (MFA).
 *
 * One MFA layer, one decode step (one new query token per sequence):
 *   - a low-rank query path: hidden 7168 -> 2048-wide bottleneck ->
 *     64 query heads x 256 ("Step-3 is Large yet Affordable", Key points:
 *     hidden size, the 2048-dim query bottleneck, 64 query heads);
 *   - attention of all 64 heads against ONE shared key head and ONE shared
 *     value head of dimension 256 held in a KV cache (same page, Key points);
 *   - the cache in bf16 or FP8 E4M3 (the FP8 deployment in the same Key
 *     points), contiguous or in pages of 64 tokens (PagedAttention, cited by
 *     title on the Step-3 references);
 *   - long contexts split into chunks merged by the log-sum-exp identity
 *     (Flash-Decoding, cited by title on the DeepSeek-V4 references).
 *
 * Conventions for every entry point:
 *   - Tensor arguments are DEVICE pointers unless marked (host). The caller
 *     allocates and owns every tensor; the library never frees them.
 *   - Work is enqueued on `hip_stream` (a hipStream_t; NULL = the default
 *     stream) and returns without synchronising. Nothing reads device
 *     memory on the host.
 *   - Arguments are checked on the host before any launch; on error the call
 *     enqueues nothing, returns a negative MFA_ERR_* status and records a
 *     message readable with mfa_last_error() (thread-local).
 *   - A handle argument must be a live handle (created by mfa_create, not yet
 *     destroyed): the library keeps a registry of live handles, so a NULL,
 *     destroyed or foreign pointer is rejected with MFA_ERR_INVALID without
 *     the memory it points at being read. Destroying a handle while another
 *     thread is inside a call on it is the caller's race.
 *   - A device fault (for example a page index outside the pool) is not
 *     detected; it surfaces at the caller's next synchronisation.
 *   - A handle may be used by one stream at a time: calls that overlap on
 *     different streams share the handle's workspace and race.
 *   - Layouts are row-major, innermost index last. bf16 is IEEE binary32's
 *     upper half; FP8 is OCP E4M3FN (bias 7, max 448, S.1111.111 = NaN).
 */
#ifndef MFA_H
#define MFA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum mfa_status {
    MFA_OK = 0,
    MFA_ERR_INVALID = -1,     /* bad argument: null pointer, size out of range, bad handle */
    MFA_ERR_UNSUPPORTED = -2, /* valid but not implemented: heads != 64, head_dim != 256, ... */
    MFA_ERR_NOMEM = -3,       /* workspace allocation failed */
    MFA_ERR_HIP = -4          /* a HIP runtime call failed (message has the HIP error) */
};

enum mfa_kv_dtype {
    MFA_DTYPE_BF16 = 0,
    MFA_DTYPE_FP8_E4M3 = 1
};

/* Arithmetic of mfa_decode's scores and P.V (the FP8 deployment and its
 * BF16-attention ablation in the Step-3 Key points):
 *   MFA_ATTN_BF16_MFMA  bf16 MFMAs; FP8 codes are widened exactly to bf16, Q
 *                       stays bf16, P is rounded to bf16 (the default).
 *   MFA_ATTN_FP8_MFMA   FP8 (E4M3) MFMAs on the cache's codes: Q quantised
 *                       per head to E4M3 (a power-of-two scale puts each
 *                       head's largest |q| in [128, 256)), P quantised to
 *                       E4M3 (scaled by 4); half the MFMA cycles, and about
 *                       2^-4 relative rounding on every Q and P element (a
 *                       normwise output error of a few percent on the
 *                       workloads). FP8 caches only; not for mfa_decode_mtp. */
enum mfa_attn_math {
    MFA_ATTN_BF16_MFMA = 0,
    MFA_ATTN_FP8_MFMA = 1
};

typedef struct mfa_ctx* mfa_handle;

/* mfa_config.split_tokens value: cut the work of each call into equal ranges,
 * one per workgroup, over all sequences in order (the work-centric
 * decomposition of Stream-K, cited by title on the DeepSeek-V4 references),
 * whatever the lengths. A sequence counts its 64-token steps plus a fixed
 * cost of 8 for its piece's set-up and epilogue. A sequence cut into several
 * pieces is merged by the last piece to finish, in piece order. */
#define MFA_SPLIT_BALANCED (-1)

/* Layer configuration (host struct, copied by mfa_create). */
typedef struct {
    int32_t hidden;        /* model width, 7168; multiple of 512 */
    int32_t q_rank;        /* query bottleneck, 2048; multiple of 64, at most 4096 */
    int32_t num_heads;     /* query heads, must be 64 */
    int32_t head_dim;      /* must be 256 */
    int32_t kv_dtype;      /* enum mfa_kv_dtype */
    int32_t page_size;     /* 0 = contiguous cache; otherwise must be 64 */
    int32_t max_batch;     /* largest batch any call will pass, >= 1 */
    int32_t max_context;   /* largest sequence length any call will pass, >= 1 */
    int32_t split_tokens;  /* split-K chunk in tokens, multiple of 64, at most 8192 with a
                              paged cache (else MFA_ERR_UNSUPPORTED); MFA_SPLIT_BALANCED;
                              or 0 = chosen per call (balanced when batch >= CUs / 2,
                              else chunks sized for the batch) */
    float rms_eps;         /* RMSNorm epsilon (1e-6), >= 0 */
    float softmax_scale;   /* score scale (1/16 = 1/sqrt(256)), finite and > 0 */
    int32_t attn_math;     /* enum mfa_attn_math; MFA_ATTN_FP8_MFMA needs an FP8 cache */
    int32_t kv_heads;      /* K/V heads G: 0 or 1 = MFA's single shared K and V head; 2 or 4 =
                              grouped-query attention ("GQA: Training Generalized Multi-Query
                              Transformer Models from Multi-Head Checkpoints", named on the
                              DeepSeek-V4 references), for comparing head-sharing schemes:
                              query head h reads K/V head h / (64 / G), the cache holds G
                              heads per token (layouts in mfa_kv). G > 1 needs
                              MFA_ATTN_BF16_MFMA (bf16 or FP8 cache); mfa_decode only (not
                              mfa_decode_mtp, mfa_kv_append or mfa_debug_gather_kv) and not
                              MFA_SPLIT_BALANCED (else MFA_ERR_UNSUPPORTED) */
    int32_t kv_latent;     /* 0: MFA's K and V heads. 512: latent-cache mode, for comparing
                              head-sharing schemes with an MLA-style cache (the Step-3
                              Key points' ablation names MLA; this is the library's reading
                              of it, the pages give no latent shape): every token stores
                              ONE 512-wide E4M3 latent row c_t (kv.k; kv.v unused, may be
                              NULL; value = decode(code) * kv.k_scale) that all 64 heads
                              use as key and as value, the key and value up-projections
                              being absorbed into the query and the output projection:
                              q and out are [batch][64][512] bf16, s_ht = softmax_scale *
                              <q_h, c_t>, out_h = sum_t softmax_t(s_h) c_t. Needs an FP8
                              cache, kv_heads 1, MFA_ATTN_BF16_MFMA and chunked splits;
                              mfa_decode only (else MFA_ERR_UNSUPPORTED) */
} mfa_config;

/* KV cache of one layer for one call (host struct describing device buffers).
 *   contiguous (page_size 0): k, v are [batch][kv_stride][256]; token t of
 *     sequence b is row b * kv_stride + t.
 *   paged (page_size 64): k, v are pools [num_pages][64][256] sharing page
 *     numbers; token t of sequence b is row t % 64 of page
 *     page_table[b * pt_stride + t / 64].
 *   With G = kv_heads > 1: contiguous [batch][G][kv_stride][256] (head g of
 *     token t at row (b * G + g) * kv_stride + t); paged pools
 *     [num_pages][G][64][256] (row (page * G + g) * 64 + t % 64).
 * Latent-cache handles (kv_latent 512): k holds 512-byte rows in the same
 *   layouts ([batch][kv_stride][512] or pools [num_pages][64][512]).
 * Element type: bf16 or E4M3 per the handle's kv_dtype. An FP8 element's
 * value is decode(code) * k_scale (keys) or * v_scale (values). Only rows
 * t < seq_lens[b] are read; mfa_kv_append writes row seq_lens[b]. */
typedef struct {
    const void* k;
    const void* v;
    float k_scale;              /* FP8 only: finite, > 0. Ignored for bf16 */
    float v_scale;              /* FP8 only: finite, > 0. Ignored for bf16 */
    const int32_t* seq_lens;    /* [batch], 0 <= L_b <= max_seq_len (values outside are clamped) */
    const int32_t* page_table;  /* [batch][pt_stride] int32, or NULL when contiguous */
    int32_t pt_stride;          /* paged: entries per page-table row, >= ceil(max_seq_len/64) */
    int32_t num_pages;          /* paged: pool size in pages, >= 1 (mfa_kv_append skips rows on
                                   pages outside it; mfa_decode does not check on device) */
    int64_t kv_stride;          /* contiguous: token slots per sequence, >= max_seq_len */
    int32_t max_seq_len;        /* (host) upper bound of seq_lens in this call, sizes the
                                   launch; 0 = the handle's max_context */
    int32_t min_seq_len;        /* (host) lower bound of seq_lens in this call, or 0 if
                                   unknown. Steers only the choice of work split (a
                                   wrong bound costs time, never correctness) */
} mfa_kv;

/* Create a handle for one layer shape. Validates `cfg` (host pointer) and
 * allocates the split-K workspace on the current device:
 *   max_batch * (ceil(max_context / C) + 1) * 64 * (256 * 2 + 4) bytes of
 *   chunk partials (bf16 rows and fp32 log-sum-exps), C = split_tokens when
 *   positive, else 256 (the smallest piece a per-call choice or a balanced
 *   split makes), 4 * max_batch 4-byte arrival counters (one per query row
 *   and head group; zeroed here, left at zero by every call), Q-projection
 *   scratch of
 *   max_batch * q_rank * (4 * hidden / 512 + 2) + (q_rank / 64) * (max_batch
 *   + ceil(max_batch / 32)) * 4 bytes (its arrival counters zeroed here and
 *   left at zero), and K/V-projection partials of
 *   2 * (hidden / 256) * max_batch * 256 * 4 bytes.
 * On success stores the handle in *out (host pointer) and returns MFA_OK. */
int mfa_create(const mfa_config* cfg, mfa_handle* out);

/* Query projection with RMSNorm on the bottleneck (Step-3 Key points: the
 * 2048-dim low-rank query bottleneck; the norm's placement is this
 * library's reading, the pages do not state it):
 *   c    = x . w_qa                         x [batch][hidden] bf16,
 *                                           w_qa [hidden][q_rank] bf16
 *   chat = c * rsqrt(mean(c^2) + rms_eps) * rms_w      rms_w [q_rank] bf16
 *   q    = chat . w_qb                      w_qb [q_rank][64*256] bf16
 * q_out is [batch][64][256] bf16 (= [batch][16384]); c accumulates in fp32;
 * c * rms_w is rounded to bf16 before the second product, whose fp32 result
 * is multiplied by the row's rsqrt(mean(c^2) + rms_eps) before rounding
 * (the same product, the norm factor applied after it).
 * 1 <= batch <= max_batch. */
int mfa_qproj(mfa_handle h, const void* x, const void* w_qa, const void* rms_w,
              const void* w_qb, void* q_out, int32_t batch, void* hip_stream);

/* Decode attention of one step:
 *   s_bht  = softmax_scale * <q[b][h][:], K_b[t][:]>      for t < L_b
 *   out[b][h][:] = sum_t softmax_t(s_bh) * V_b[t][:]       bf16
 *   lse_out[b][h] = log(sum_t exp(s_bht))                  fp32, natural log
 * q [batch][64][256] bf16; out [batch][64][256] bf16; lse_out [batch][64]
 * fp32 or NULL. L_b = 0 gives out = 0 and lse = -inf.
 * The KV range of each sequence is cut into chunks of split_tokens tokens
 * (or a per-call choice when split_tokens is 0), or by a balanced split
 * (MFA_SPLIT_BALANCED, and the per-call choice for batches of at least half
 * the CU count whose length bounds do not show equal step counts) into the
 * pieces that equal ranges of work over the whole batch give; partials
 * (normalised, rounded to bf16, with fp32 log-sum-exps) go to the handle's
 * workspace and are merged in fp32 by the log-sum-exp identity, in chunk
 * order: inside the attention kernel by the last chunk to finish when
 * no sequence of the call has more than two chunks or the split is balanced,
 * else by a second kernel on the same stream. The result depends only on the
 * logical K/V values, the lengths and the chunking, not on the cache layout:
 * paged and contiguous caches holding the same rows give bitwise equal
 * outputs. 1 <= batch <= max_batch.
 * Latent-cache handles (mfa_config.kv_latent = 512): q and out are
 * [batch][64][512] bf16, kv.k the latent rows; two workgroups of 32 heads per
 * (sequence, chunk), chunks of split_tokens or of the per-call choice; a
 * sequence with several chunks is merged by a second kernel. */
int mfa_decode(mfa_handle h, const void* q, const mfa_kv* kv, void* out, float* lse_out,
               int32_t batch, void* hip_stream);

/* mfa_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): no
 * handle; cfg (host pointer) is checked as by mfa_create and copied, and the
 * workspace is a static device array of the library (64 MiB on every GPU the
 * library runs on, held until the process ends). The result is the one
 * mfa_decode gives on a handle created with the same cfg (same kernels and
 * split). The call allocates nothing, host or device. Limits: max_batch <=
 * 65536, and the call's split must fit 2000 partial slots: query rows times
 * chunks per sequence for a chunked split (mfa_split_tokens gives the chunk;
 * for example 128 sequences of 4096 tokens in two chunks use 256), or rows
 * times (ceil(max_context / 256) + 1) for a balanced one; beyond them the
 * call returns MFA_ERR_UNSUPPORTED before enqueueing anything. Every call on
 * one GPU shares that workspace: calls that overlap on one GPU (other
 * streams, other host threads) race and must be serialised by the caller.
 * The first call on a device enqueues one small clearing kernel on
 * hip_stream before the attention. Other arguments, ownership and errors as
 * for mfa_decode. */
int mfa_decode_noalloc(const mfa_config* cfg, const void* q, const mfa_kv* kv, void* out,
                       float* lse_out, int32_t batch, void* hip_stream);

/* Multi-token decode (several new tokens per sequence in one step, as
 * multi-token prediction does; Step-3 Key points name it among the future
 * directions): num_tokens query tokens per sequence attend to the same cache.
 * The cache already holds the new tokens' K/V rows, token j of sequence b at
 * row L_b - num_tokens + j, and token j sees rows t < L_b - (num_tokens-1-j)
 * (itself and everything before it; a token with no row gives out = 0, lse =
 * -inf):
 *   q [batch][num_tokens][64][256] bf16, out [batch][num_tokens][64][256]
 *   bf16, lse_out [batch][num_tokens][64] fp32 or NULL.
 * The workgroups of a sequence's tokens run side by side on one XCD, so most
 * of their reads of a cached row after the first come from that XCD's L2.
 * Uses the chunked split (split_tokens, or the per-call choice for batch *
 * num_tokens rows that mfa_split_tokens_mtp reports).
 * 1 <= num_tokens <= 16; batch * num_tokens <= max_batch (the workspace holds
 * partials per query token). num_tokens = 1 is mfa_decode with the chunked
 * split. */
int mfa_decode_mtp(mfa_handle h, const void* q, const mfa_kv* kv, int32_t num_tokens, void* out,
                   float* lse_out, int32_t batch, void* hip_stream);

/* KV append: the new token's key and value rows, written into the cache
 * before that token's attention (Step-3 Key points: one shared key head and
 * one shared value head of 256, so one K row and one V row per token; the
 * FP8 cache of the same Key points; pages as in PagedAttention):
 *   k_new = x . w_k,  v_new = x . w_v      x [batch][hidden] bf16,
 *                                          w_k, w_v [hidden][256] bf16
 * accumulated in fp32, then stored at row L_b = kv->seq_lens[b] of sequence b
 * (the layout rules of mfa_kv) as bf16 by round-to-nearest-even, or for an
 * FP8 handle as the E4M3 code of k_new / k_scale (v_new / v_scale), rounded to
 * nearest even, saturating at +-448. The library WRITES through kv->k and
 * kv->v here (they must be writable device memory); nothing else in the cache
 * changes and seq_lens is not advanced (the caller attends with L_b + 1).
 * A sequence whose row does not exist is skipped, not an error: L_b < 0;
 * contiguous, L_b >= kv_stride; paged, L_b / 64 >= pt_stride or a page
 * number outside [0, num_pages) (the caller allocates pages). The other
 * kv fields are checked as for mfa_decode. 1 <= batch <= max_batch. */
int mfa_kv_append(mfa_handle h, const void* x, const void* w_k, const void* w_v,
                  const mfa_kv* kv, int32_t batch, void* hip_stream);

/* The split-K chunk (tokens) mfa_decode uses for this batch and the length
 * bounds kv->max_seq_len and kv->min_seq_len; 0 when it uses the balanced
 * split. */
int32_t mfa_split_tokens(mfa_handle h, int32_t batch, int32_t max_seq_len, int32_t min_seq_len);

/* The split-K chunk (tokens) mfa_decode_mtp uses for batch sequences of
 * num_tokens query tokens each and the length bound kv->max_seq_len (always a
 * chunked split: split_tokens if the handle fixes it, else chunks of up to
 * 8192 tokens sized for batch * num_tokens query-row sets, so that the
 * workgroups of a sequence's tokens take it whole where the grid allows).
 * num_tokens = 1 gives mfa_decode's chunked split. MFA_ERR_INVALID for
 * num_tokens outside [1, 16] or batch * num_tokens outside [1, max_batch];
 * MFA_ERR_UNSUPPORTED for num_tokens > 1 on a handle mfa_decode_mtp rejects
 * (latent or grouped caches, FP8-MFMA arithmetic). */
int32_t mfa_split_tokens_mtp(mfa_handle h, int32_t batch, int32_t num_tokens, int32_t max_seq_len);

/* The number of workgroups that share the 64 query heads of one (sequence,
 * chunk) in that split: 1; 2 (heads 0-31 and 32-63, which then read the same
 * K/V rows, the second read from L2) with attn_math MFA_ATTN_FP8_MFMA and a
 * chunked split whose doubled grid fits on the compute units at once; 4
 * (16 heads each) for a bf16 cache whose grid would otherwise use at most a
 * quarter of the compute units; or kv_heads for a grouped-query cache (one
 * workgroup per K/V head). For a given chunk the result of mfa_decode does
 * not depend on it. Negative status on error. */
int32_t mfa_head_groups(mfa_handle h, int32_t batch, int32_t max_seq_len, int32_t min_seq_len);

/* Test support: copy the logical K and V rows t < L_b of sequence b into
 * contiguous device buffers k_dst, v_dst ([max_seq_len][256] elements of the
 * cache type) with the attention kernel's own address generation (for a paged
 * cache: the page indices of a piece of up to 128 steps held in registers and
 * read back per 64-token step). The page table is trusted as in mfa_decode. */
int mfa_debug_gather_kv(mfa_handle h, const mfa_kv* kv, int32_t b, void* k_dst, void* v_dst,
                        void* hip_stream);

/* Test support: the FP8 matrix operation of the MFA_ATTN_FP8_MFMA mode on
 * given operands, so that its arithmetic can be measured: for each of n_tiles
 * tiles, d = a . b + c with a [16][128] and b [128][16] OCP E4M3 codes and c,
 * d [16][16] fp32, all row-major and contiguous per tile (a, b, c, d device
 * pointers; c may be NULL for zero). No handle; 0 <= n_tiles <= 2^20.
 * Asynchronous on hip_stream. */
int mfa_debug_fp8_mfma(const void* a, const void* b, const float* c, float* d, int32_t n_tiles,
                       void* hip_stream);

/* Measurement support: the matrix-core rate microbenchmark, to set the MFMA
 * rates the attention reaches beside what the chip sustains. One launch of
 * two workgroups of four waves per compute unit (two waves per SIMD); each
 * wave runs iters rounds of eight independent MFMAs on operands held in
 * registers, with no memory traffic: kind 0 v_mfma_f32_16x16x32_bf16 (the
 * bf16 MFMA of the attention and the Q projection), kind 1 the unit-scaled
 * v_mfma_f32_16x16x128_f8f6f4 on E4M3 codes (the FP8-MFMA mode). *flops
 * (host) receives the launch's floating-point operations (2 per
 * multiply-add); dividing by its duration gives the rate. sink is a device
 * float the kernel may write (it never does for these operands; the write
 * keeps the work). No handle; 1 <= iters <= 2^24 (about 7 ms per 2^16 on
 * MI355X). Asynchronous on hip_stream. */
int mfa_debug_mfma_rate(int32_t kind, int32_t iters, float* sink, double* flops, void* hip_stream);

/* Kernel kinds reported by mfa_profile_read. */
enum mfa_kernel_kind {
    MFA_KERNEL_ATTENTION = 0,   /* chunked decode attention */
    MFA_KERNEL_COMBINE = 1,     /* log-sum-exp merge of chunk partials */
    MFA_KERNEL_QPROJ_DOWN = 2,  /* x . w_qa */
    MFA_KERNEL_RMSNORM = 3,     /* (not launched: the RMSNorm is split between the two
                                   projection kernels) */
    MFA_KERNEL_QPROJ_UP = 4,    /* chat . w_qb */
    MFA_KERNEL_KV_PROJ = 5,     /* x . w_k and x . w_v (K-split partials) */
    MFA_KERNEL_KV_WRITE = 6,    /* partial sums, encoding and the row write */
    MFA_KERNEL_KINDS = 7
};

/* Per-kernel timing for benchmarks, off by default. While enabled, every
 * kernel that mfa_decode, mfa_qproj or mfa_kv_append launches is bracketed by a pair of
 * hipEvents recorded on the call's stream (events are created here, on the
 * current device). enable = 0 releases them. */
int mfa_profile_enable(mfa_handle h, int enable);

/* Wait for the launches recorded since the last read and return, per kernel
 * kind (arrays of MFA_KERNEL_KINDS on the host), how many ran and their summed
 * durations in milliseconds; then forget them. At most 4096 launches are kept
 * between reads (older ones are overwritten). */
int mfa_profile_read(mfa_handle h, int32_t* launches, double* total_ms);

/* Release the handle and its workspace. NULL is accepted (MFA_OK); a pointer
 * that is not a live handle (already destroyed, never created) returns
 * MFA_ERR_INVALID and frees nothing. The caller must ensure no enqueued call
 * that uses the handle is still running. */
int mfa_destroy(mfa_handle h);

/* Static text for a status code. */
const char* mfa_status_string(int status);

/* Message of the last failed call on this thread ("" if none). */
const char* mfa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MFA_H */
