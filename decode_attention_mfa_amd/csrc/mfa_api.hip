// mfa_api.hip -- the C ABI declared in include/mfa.h: argument checks,
// workspace ownership, split selection and kernel launches. Every check runs
// on the host before anything is enqueued; no call synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <string>
#include <unordered_set>
#include <vector>

#include "mfa.h"
#include "mfa_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(MFA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMinAutoSplit = 256;
constexpr int kMaxAutoSplit = 2048;

}  // namespace

// ---------------------------------------------------------------- scratch
// Device workspace of mfa_decode_noalloc, for callers that cannot allocate:
// a file-scope array that every GPU the library runs on holds until the
// process ends. The first kNoAllocCounterBytes hold the arrival counters
// (zero between calls: cleared once per device, and every kernel that counts
// resets what it used); the rest holds the chunk partials. Host code uses
// the array only through the per-device address taken once with
// hipGetSymbolAddress (its name on the host is not a device address).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
constexpr size_t kNoAllocCounterBytes = size_t(1) << 20;   // [max_batch <= 65536][4] int32
// partial slots (a [64][256] bf16 row block and 64 fp32 log-sum-exps each)
constexpr int64_t kSlotBytes = 64 * 256 * 2 + 64 * 4;
constexpr int64_t kNoAllocSlots = (int64_t)(kNoAllocScratchBytes - kNoAllocCounterBytes) / kSlotBytes;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
struct ScratchSlot {
    uint8_t* ptr = nullptr;   // device address of `scratch` on this device
    int num_cu = 0;
    bool cleared = false;     // the counter region's clear has been enqueued
};
std::mutex g_scratch_mutex;
ScratchSlot g_scratch[kMaxDevices];
}  // namespace

// Optional per-kernel timing: a ring of hipEvent pairs, each pair stamped
// with one kernel's start and end by the launch itself.
struct Profiler {
    static constexpr int kCap = 4096;
    bool on = false;
    std::vector<hipEvent_t> ev;   // 2 * kCap events, created on enable
    std::vector<int> kind;        // kind of each recorded pair, -1 = empty
    int next = 0;
};

struct mfa_ctx {
    Profiler prof;
    mfa_config cfg;
    int device;
    int num_cu;
    int max_chunks;        // per sequence, at the smallest chunk this handle may use
    int64_t part_slots;    // partial slots the workspace holds
    float* part_o;         // [max_batch * max_chunks][64][256] bf16
    float* part_lse;       // [max_batch * max_chunks][64]
    int32_t* counters;     // [max_batch][2], zero between calls
    float* c_part;         // [hidden / kQprojRowsPerSplit][max_batch][q_rank]
    uint16_t* chat;        // [max_batch][q_rank]: c * gamma, bf16
    float* sumsq;          // [max_batch][q_rank / 64]
    int32_t* qcounters;    // [ceil(max_batch / 32)][q_rank / 64], zero between calls
    float* kv_part;        // [2][hidden / kKvRowsPerSplit][max_batch][256]
};

// Live handles, so that a pointer that is not one (never created, or
// destroyed) is rejected without reading the memory it points at.
static std::mutex g_handles_mutex;
static std::unordered_set<const mfa_ctx*>& live_handles() {
    static std::unordered_set<const mfa_ctx*>* set = new std::unordered_set<const mfa_ctx*>();
    return *set;
}
static bool valid_handle(mfa_handle h) {
    if (!h) return false;
    std::lock_guard<std::mutex> lock(g_handles_mutex);
    return live_handles().count(h) != 0;
}

// Launch `fn(launch)` on `st`; when profiling is on, with the next event pair
// of the ring attached to the kernel's own start and end.
template <typename F>
static hipError_t timed_launch(mfa_ctx* h, int kind, hipStream_t st, F&& fn) {
    Profiler& p = h->prof;
    mfa::Launch l{st};
    if (!p.on) return fn(l);
    const int i = p.next;
    p.next = (p.next + 1) % Profiler::kCap;
    l.start = p.ev[2 * i];
    l.stop = p.ev[2 * i + 1];
    const hipError_t e = fn(l);
    if (e == hipSuccess) p.kind[i] = kind;
    return e;
}

static void profiler_release(Profiler& p) {
    for (hipEvent_t e : p.ev) (void)hipEventDestroy(e);
    p.ev.clear();
    p.kind.clear();
    p.on = false;
    p.next = 0;
}

static int round_up(int64_t a, int64_t m) { return (int)(((a + m - 1) / m) * m); }

// K splits of the K/V projections: the most (256 rows each, the fewest
// tiles per workgroup) that keep the launch within about two workgroups per
// compute unit (8 column blocks of 64 for K and V, one row block per 64
// sequences); halved (rows per split doubled) while it would exceed that and
// the rows still divide hidden.
static int32_t kv_ksplit(int32_t hidden, int32_t batch) {
    const int64_t col_row_blocks = 2 * (mfa::kHeadDim / 64) * (int64_t)((batch + 63) / 64);
    int32_t rows = mfa::kKvRowsPerSplit;
    while (col_row_blocks * (hidden / rows) > 512 && hidden % (2 * rows) == 0) rows *= 2;
    return hidden / rows;
}

// Balanced work split (equal step ranges per workgroup) when the caller asks
// for it, or by default for batches of at least half a workgroup per CU
// (there every sequence spans few ranges, so the last range of a sequence to
// finish merges its pieces cheaply) unless the caller's length bounds show
// that every sequence has the same number of 64-token steps: then equal
// chunks are already balanced and need no length scan. Smaller batches of
// long sequences keep per-sequence chunks and the separate merge kernel.
static bool use_balanced(const mfa_ctx* h, int32_t batch, int32_t max_len, int32_t min_len) {
    if (h->cfg.kv_heads > 1) return false;   // grouped caches: chunks, one workgroup per K/V head
    if (h->cfg.split_tokens == MFA_SPLIT_BALANCED) return true;
    if (h->cfg.split_tokens != 0 || 2 * batch < h->num_cu) return false;
    const bool uniform = min_len > 0 && (min_len + mfa::kStep - 1) / mfa::kStep == (max_len + mfa::kStep - 1) / mfa::kStep;
    return !uniform;
}

static int32_t choose_split(const mfa_ctx* h, int32_t batch, int32_t max_len, int32_t max_auto = kMaxAutoSplit) {
    if (h->cfg.split_tokens > 0) return h->cfg.split_tokens;
    if (max_len <= 0) return kMinAutoSplit;
    // one chunk per compute unit's share of the batch's tokens, whole pages
    int64_t share = ((int64_t)batch * max_len + h->num_cu - 1) / h->num_cu;
    int64_t c = round_up(share, mfa::kStep);
    if (c < kMinAutoSplit) c = kMinAutoSplit;
    if (c > max_auto) c = max_auto;
    if (c > round_up(max_len, mfa::kStep)) c = round_up(max_len, mfa::kStep);
    return (int32_t)c;
}

// The chunked split of a call with `rows` query-row sets (qtok query tokens
// per sequence): the chunk and the number of head groups per (row set,
// chunk). Head groups read the same K/V rows (the later ones mostly from
// the XCD's L2, their block indices 8 apart).
//   - bf16 caches, one query token, a grid that would use at most a quarter
//     of the compute units: four groups of 16 heads on the same chunks
//     (each group's piece then has a quarter of the MFMA and softmax work;
//     the result is bitwise the one of 64-head workgroups). With more
//     workgroups the groups' repeated K/V reads cost more than they save:
//     the bf16 step loop waits on its loads (two 64 KB steps in the ring);
//   - the FP8-MFMA mode: two groups of 32 on chunks twice as long when the
//     doubled grid fits, so a sequence needs half as many chunks;
//   - FP8 caches with bf16 MFMAs keep 64 heads per workgroup: each group
//     would widen every FP8 row itself, and that VALU work costs more than
//     the merges it saves.
static void plan_chunks(const mfa_ctx* h, int32_t rows, int32_t qtok, int32_t max_len, int32_t* chunk,
                        int32_t* nh) {
    if (h->cfg.kv_heads > 1) {   // grouped caches: one workgroup per (row set, chunk, K/V head)
        *nh = h->cfg.kv_heads;
        *chunk = choose_split(h, *nh * rows, max_len, mfa::kMaxPagedChunkSteps * mfa::kStep);
        return;
    }
    *nh = 1;
    // multi-token decode: chunks up to the paged limit, so that the t
    // workgroups of a sequence (one per token, side by side on one XCD) take
    // it whole where the grid allows: no merges and fewer rounds of
    // workgroups (t = 2 at 128 x 4096: 256 single pieces instead of 512
    // half-length ones)
    *chunk = choose_split(h, rows, max_len, qtok > 1 ? mfa::kMaxPagedChunkSteps * mfa::kStep : kMaxAutoSplit);
    if (h->cfg.kv_dtype == MFA_DTYPE_BF16 && qtok == 1 && max_len > 0) {
        const int64_t n = (max_len + *chunk - 1) / *chunk;
        if (4 * (int64_t)rows * n <= h->num_cu) *nh = 4;
        return;
    }
    if (h->cfg.attn_math != MFA_ATTN_FP8_MFMA || max_len <= 0) return;
    // chunks up to the paged limit: with two workgroups per chunk, the
    // longer chunk still leaves every compute unit one workgroup
    const int32_t c2 = choose_split(h, 2 * rows, max_len, mfa::kMaxPagedChunkSteps * mfa::kStep);
    const int64_t n2 = (max_len + c2 - 1) / c2;
    if (2 * (int64_t)rows * n2 <= h->num_cu) {
        *chunk = c2;
        *nh = 2;
    }
}

// Latent-cache mode: the chunk for `rows` query rows, two workgroups of 32
// heads per (row, chunk).
static int32_t latent_chunk(const mfa_ctx* h, int32_t rows, int32_t max_len) {
    return choose_split(h, 2 * rows, max_len, mfa::kMaxPagedChunkSteps * mfa::kStep);
}

extern "C" {

const char* mfa_status_string(int status) {
    switch (status) {
        case MFA_OK: return "ok";
        case MFA_ERR_INVALID: return "invalid argument";
        case MFA_ERR_UNSUPPORTED: return "unsupported configuration";
        case MFA_ERR_NOMEM: return "out of device memory";
        case MFA_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* mfa_last_error(void) { return g_last_error; }

// Checks a configuration and fills in its defaults (kv_heads 0 -> 1); fn
// names the entry point in the error message.
static int validate_config(const mfa_config* cfg, mfa_config* out, const char* fn) {
    mfa_config c = *cfg;
    if (c.num_heads != mfa::kHeads || c.head_dim != mfa::kHeadDim)
        return fail(MFA_ERR_UNSUPPORTED, "%s: only 64 heads x 256 are supported (got %d x %d)", fn,
                    c.num_heads, c.head_dim);
    if (c.hidden <= 0 || c.hidden % mfa::kQprojRowsPerSplit != 0)
        return fail(MFA_ERR_UNSUPPORTED, "%s: hidden must be a positive multiple of %d (got %d)", fn,
                    mfa::kQprojRowsPerSplit, c.hidden);
    if (c.q_rank <= 0 || c.q_rank % 64 != 0 || c.q_rank > 64 * mfa::kMaxNormBlocks)
        return fail(MFA_ERR_UNSUPPORTED, "%s: q_rank must be a positive multiple of 64, at most %d (got %d)", fn,
                    64 * mfa::kMaxNormBlocks, c.q_rank);
    if (c.kv_dtype != MFA_DTYPE_BF16 && c.kv_dtype != MFA_DTYPE_FP8_E4M3)
        return fail(MFA_ERR_INVALID, "%s: bad kv_dtype %d", fn, c.kv_dtype);
    if (c.page_size != 0 && c.page_size != mfa::kPage)
        return fail(MFA_ERR_UNSUPPORTED, "%s: page_size must be 0 or 64 (got %d)", fn, c.page_size);
    if (c.max_batch < 1 || c.max_context < 1)
        return fail(MFA_ERR_INVALID, "%s: max_batch and max_context must be >= 1", fn);
    if (c.split_tokens < MFA_SPLIT_BALANCED || (c.split_tokens > 0 && c.split_tokens % mfa::kStep != 0))
        return fail(MFA_ERR_INVALID,
                    "%s: split_tokens must be 0, MFA_SPLIT_BALANCED or a positive multiple of 64 (got %d)", fn,
                    c.split_tokens);
    if (c.page_size != 0 && c.split_tokens > mfa::kMaxPagedChunkSteps * mfa::kStep)
        return fail(MFA_ERR_UNSUPPORTED, "%s: with a paged cache split_tokens must be <= %d (got %d)", fn,
                    mfa::kMaxPagedChunkSteps * mfa::kStep, c.split_tokens);
    if (!(c.softmax_scale > 0.f) || !isfinite(c.softmax_scale))
        return fail(MFA_ERR_INVALID, "%s: softmax_scale must be finite and > 0", fn);
    if (!(c.rms_eps >= 0.f) || !isfinite(c.rms_eps))
        return fail(MFA_ERR_INVALID, "%s: rms_eps must be finite and >= 0", fn);
    if (c.attn_math != MFA_ATTN_BF16_MFMA && c.attn_math != MFA_ATTN_FP8_MFMA)
        return fail(MFA_ERR_INVALID, "%s: bad attn_math %d", fn, c.attn_math);
    if (c.attn_math == MFA_ATTN_FP8_MFMA && c.kv_dtype != MFA_DTYPE_FP8_E4M3)
        return fail(MFA_ERR_UNSUPPORTED, "%s: attn_math FP8_MFMA needs an FP8 cache", fn);
    if (c.kv_heads == 0) c.kv_heads = 1;
    if (c.kv_heads != 1 && c.kv_heads != 2 && c.kv_heads != 4)
        return fail(MFA_ERR_INVALID, "%s: kv_heads must be 1, 2 or 4 (got %d)", fn, c.kv_heads);
    if (c.kv_heads > 1 && (c.attn_math != MFA_ATTN_BF16_MFMA || c.split_tokens == MFA_SPLIT_BALANCED))
        return fail(MFA_ERR_UNSUPPORTED, "%s: kv_heads > 1 needs MFA_ATTN_BF16_MFMA and chunked splits", fn);
    if (c.kv_latent != 0 && c.kv_latent != mfa::kLatent)
        return fail(MFA_ERR_INVALID, "%s: kv_latent must be 0 or %d (got %d)", fn, mfa::kLatent, c.kv_latent);
    if (c.kv_latent && (c.kv_dtype != MFA_DTYPE_FP8_E4M3 || c.kv_heads > 1 || c.attn_math != MFA_ATTN_BF16_MFMA ||
                        c.split_tokens == MFA_SPLIT_BALANCED))
        return fail(MFA_ERR_UNSUPPORTED,
                    "%s: kv_latent needs an FP8 cache, kv_heads 1, MFA_ATTN_BF16_MFMA and chunked splits", fn);

    *out = c;
    return MFA_OK;
}

// Chunks per sequence at the smallest chunk the configuration allows (the
// workspace holds one more partial slot per sequence: a balanced split may
// cut a sequence into ceil(steps / 4) + 1 pieces).
static int64_t workspace_chunks(const mfa_config& c) {
    const int min_chunk = c.split_tokens > 0 ? c.split_tokens : kMinAutoSplit;
    return ((int64_t)c.max_context + min_chunk - 1) / min_chunk;
}

int mfa_create(const mfa_config* cfg, mfa_handle* out) {
    g_last_error[0] = 0;
    if (!cfg || !out) return fail(MFA_ERR_INVALID, "mfa_create: null cfg or out");
    *out = nullptr;
    mfa_config c;
    int rc = validate_config(cfg, &c, "mfa_create");
    if (rc) return rc;

    const int64_t max_chunks = workspace_chunks(c);
    // one more slot per sequence than chunks: a balanced split may cut a
    // sequence into ceil(steps / 4) + 1 pieces
    const int64_t nparts = (int64_t)c.max_batch * (max_chunks + 1);
    // bounds that keep every size below in int64 (and far beyond any GPU's memory)
    if (max_chunks > (1 << 24) || nparts > (int64_t)1 << 31)
        return fail(MFA_ERR_INVALID, "mfa_create: max_batch * max_context too large");
    if ((int64_t)c.max_batch * c.hidden > (int64_t)1 << 40)
        return fail(MFA_ERR_INVALID, "mfa_create: max_batch * hidden too large");
    const int64_t row_dim = c.kv_latent ? mfa::kLatent : mfa::kHeadDim;   // output row width
    const int64_t bytes_o = nparts * mfa::kHeads * row_dim * 2;          // bf16 partials
    const int64_t bytes_lse = nparts * mfa::kHeads * 4;
    const int64_t bytes_c = (int64_t)(c.hidden / mfa::kQprojRowsPerSplit) * c.max_batch * c.q_rank * 4;
    const int64_t bytes_chat = (int64_t)c.max_batch * c.q_rank * 2;
    const int64_t bytes_kv = 2 * (int64_t)(c.hidden / mfa::kKvRowsPerSplit) * c.max_batch * mfa::kHeadDim * 4;
    const int64_t bytes_sumsq = (int64_t)(c.q_rank / 64) * c.max_batch * 4;
    const int64_t bytes_qctr = (int64_t)((c.max_batch + 31) / 32) * (c.q_rank / 64) * 4;

    mfa_ctx* h = new (std::nothrow) mfa_ctx();
    if (!h) return fail(MFA_ERR_NOMEM, "mfa_create: host allocation failed");
    h->cfg = c;
    h->max_chunks = (int)max_chunks;
    h->part_slots = nparts;
    hipError_t e = hipGetDevice(&h->device);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&h->num_cu, hipDeviceAttributeMultiprocessorCount, h->device);
    if (e != hipSuccess) {
        delete h;
        return hip_fail(e, "mfa_create: device query");
    }
    constexpr int kBuffers = 8;
    void* p[kBuffers] = {};
    const int64_t bytes_ctr = 4 * (int64_t)c.max_batch * 4;   // per (query row set, head group)
    const int64_t sizes[kBuffers] = {bytes_o,  bytes_lse, bytes_c,     bytes_chat, bytes_ctr,
                                     bytes_kv, bytes_sumsq, bytes_qctr};
    for (int i = 0; i < kBuffers; i++) {
        e = hipMalloc(&p[i], (size_t)sizes[i]);
        if (e != hipSuccess) {
            for (int j = 0; j < i; j++) (void)hipFree(p[j]);
            delete h;
            (void)hipGetLastError();
            return fail(MFA_ERR_NOMEM, "mfa_create: workspace allocation of %lld bytes failed: %s",
                        (long long)sizes[i], hipGetErrorString(e));
        }
    }
    h->part_o = (float*)p[0];
    h->part_lse = (float*)p[1];
    h->c_part = (float*)p[2];
    h->chat = (uint16_t*)p[3];
    h->counters = (int32_t*)p[4];
    h->kv_part = (float*)p[5];
    h->sumsq = (float*)p[6];
    h->qcounters = (int32_t*)p[7];
    e = hipMemset(h->counters, 0, (size_t)bytes_ctr);
    if (e == hipSuccess) e = hipMemset(h->qcounters, 0, (size_t)bytes_qctr);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        for (int j = 0; j < kBuffers; j++) (void)hipFree(p[j]);
        delete h;
        return hip_fail(e, "mfa_create: clearing the workspace");
    }
    {
        std::lock_guard<std::mutex> lock(g_handles_mutex);
        live_handles().insert(h);
    }
    *out = h;
    return MFA_OK;
}

int mfa_destroy(mfa_handle h) {
    g_last_error[0] = 0;
    if (!h) return MFA_OK;
    {
        std::lock_guard<std::mutex> lock(g_handles_mutex);
        if (live_handles().erase(h) == 0) return fail(MFA_ERR_INVALID, "mfa_destroy: not a live handle");
    }
    profiler_release(h->prof);
    (void)hipFree(h->part_o);
    (void)hipFree(h->part_lse);
    (void)hipFree(h->c_part);
    (void)hipFree(h->chat);
    (void)hipFree(h->counters);
    (void)hipFree(h->kv_part);
    (void)hipFree(h->sumsq);
    (void)hipFree(h->qcounters);
    delete h;
    return MFA_OK;
}

int32_t mfa_split_tokens(mfa_handle h, int32_t batch, int32_t max_seq_len, int32_t min_seq_len) {
    if (!valid_handle(h)) return fail(MFA_ERR_INVALID, "mfa_split_tokens: not a live handle");
    if (max_seq_len <= 0) max_seq_len = h->cfg.max_context;
    if (h->cfg.kv_latent) return latent_chunk(h, batch, max_seq_len);
    if (use_balanced(h, batch, max_seq_len, min_seq_len)) return 0;
    int32_t chunk, nh;
    plan_chunks(h, batch, 1, max_seq_len, &chunk, &nh);
    return chunk;
}

int32_t mfa_split_tokens_mtp(mfa_handle h, int32_t batch, int32_t num_tokens, int32_t max_seq_len) {
    if (!valid_handle(h)) return fail(MFA_ERR_INVALID, "mfa_split_tokens_mtp: not a live handle");
    if (num_tokens < 1 || num_tokens > mfa::kMaxQueryTokens)
        return fail(MFA_ERR_INVALID, "mfa_split_tokens_mtp: num_tokens %d outside [1, %d]", num_tokens,
                    mfa::kMaxQueryTokens);
    if (batch < 1 || (int64_t)batch * num_tokens > h->cfg.max_batch)
        return fail(MFA_ERR_INVALID, "mfa_split_tokens_mtp: batch %d x num_tokens %d outside [1, max_batch %d]", batch,
                    num_tokens, h->cfg.max_batch);
    if (num_tokens > 1 && (h->cfg.kv_latent || h->cfg.kv_heads > 1 || h->cfg.attn_math == MFA_ATTN_FP8_MFMA))
        return fail(MFA_ERR_UNSUPPORTED, "mfa_split_tokens_mtp: this handle decodes one token per sequence");
    if (max_seq_len <= 0) max_seq_len = h->cfg.max_context;
    if (h->cfg.kv_latent) return latent_chunk(h, batch, max_seq_len);
    int32_t chunk, nh;
    plan_chunks(h, batch * num_tokens, num_tokens, max_seq_len, &chunk, &nh);
    return chunk;
}

int32_t mfa_head_groups(mfa_handle h, int32_t batch, int32_t max_seq_len, int32_t min_seq_len) {
    if (!valid_handle(h)) return fail(MFA_ERR_INVALID, "mfa_head_groups: not a live handle");
    if (max_seq_len <= 0) max_seq_len = h->cfg.max_context;
    if (h->cfg.kv_latent) return 2;
    if (use_balanced(h, batch, max_seq_len, min_seq_len)) return 1;
    int32_t chunk, nh;
    plan_chunks(h, batch, 1, max_seq_len, &chunk, &nh);
    return nh;
}

int mfa_qproj(mfa_handle h, const void* x, const void* w_qa, const void* rms_w, const void* w_qb,
              void* q_out, int32_t batch, void* hip_stream) {
    g_last_error[0] = 0;
    if (!valid_handle(h)) return fail(MFA_ERR_INVALID, "mfa_qproj: not a live handle");
    if (h->cfg.kv_latent) return fail(MFA_ERR_UNSUPPORTED, "mfa_qproj: not for a latent-cache handle");
    if (!x || !w_qa || !rms_w || !w_qb || !q_out)
        return fail(MFA_ERR_INVALID, "mfa_qproj: null tensor pointer");
    if (batch < 1 || batch > h->cfg.max_batch)
        return fail(MFA_ERR_INVALID, "mfa_qproj: batch %d outside [1, %d]", batch, h->cfg.max_batch);
    mfa::QprojArgs a;
    a.x = (const uint16_t*)x;
    a.w_qa = (const uint16_t*)w_qa;
    a.rms_w = (const uint16_t*)rms_w;
    a.w_qb = (const uint16_t*)w_qb;
    a.q_out = (uint16_t*)q_out;
    a.c_part = h->c_part;
    a.chat = h->chat;
    a.sumsq = h->sumsq;
    a.counters = h->qcounters;
    a.batch = batch;
    a.hidden = h->cfg.hidden;
    a.rank = h->cfg.q_rank;
    a.nq = mfa::kHeads * mfa::kHeadDim;
    // K splits for the down-projection: the most that still give every
    // workgroup its own compute unit (column blocks x row blocks x splits <=
    // CUs), among the divisors of hidden / 64 tiles with at least 512 rows
    // per split (the partial workspace's size)
    {
        const int tiles = a.hidden / 64;
        const int blocks = (a.rank / 64) * (batch <= 32 ? 1 : (batch + 63) / 64);
        a.ksplit = 1;
        for (int d = 1; d <= a.hidden / mfa::kQprojRowsPerSplit; d++)
            if (tiles % d == 0 && (int64_t)blocks * d <= h->num_cu) a.ksplit = d;
    }
    a.eps = h->cfg.rms_eps;
    hipStream_t st = (hipStream_t)hip_stream;
    // the RMSNorm is split between the two launches (see mfa_qproj.hip)
    hipError_t e = timed_launch(h, MFA_KERNEL_QPROJ_DOWN, st, [&](const mfa::Launch& l) { return mfa::launch_qproj_down(a, l); });
    if (e == hipSuccess) e = timed_launch(h, MFA_KERNEL_QPROJ_UP, st, [&](const mfa::Launch& l) { return mfa::launch_qproj_up(a, l); });
    if (e != hipSuccess) return hip_fail(e, "mfa_qproj: launch");
    return MFA_OK;
}

static int check_kv(const mfa_ctx* h, const mfa_kv* kv, int32_t batch, const char* fn, int32_t* max_len) {
    if (!kv) return fail(MFA_ERR_INVALID, "%s: null kv", fn);
    if (!kv->k || (!kv->v && !h->cfg.kv_latent) || !kv->seq_lens)
        return fail(MFA_ERR_INVALID, "%s: null k, v or seq_lens", fn);
    const int32_t ml = kv->max_seq_len > 0 ? kv->max_seq_len : h->cfg.max_context;
    if (kv->max_seq_len < 0 || ml > h->cfg.max_context)
        return fail(MFA_ERR_INVALID, "%s: max_seq_len %d outside [0, max_context %d]", fn, kv->max_seq_len,
                    h->cfg.max_context);
    if (h->cfg.page_size) {
        if (!kv->page_table) return fail(MFA_ERR_INVALID, "%s: paged handle needs a page_table", fn);
        if (kv->pt_stride < (ml + mfa::kPage - 1) / mfa::kPage)
            return fail(MFA_ERR_INVALID, "%s: pt_stride %d < ceil(max_seq_len/64) = %d", fn, kv->pt_stride,
                        (ml + mfa::kPage - 1) / mfa::kPage);
        if (kv->num_pages < 1) return fail(MFA_ERR_INVALID, "%s: num_pages must be >= 1", fn);
    } else {
        if (kv->page_table) return fail(MFA_ERR_INVALID, "%s: contiguous handle got a page_table", fn);
        if (kv->kv_stride < ml)
            return fail(MFA_ERR_INVALID, "%s: kv_stride %lld < max_seq_len %d", fn, (long long)kv->kv_stride, ml);
    }
    if (h->cfg.kv_dtype == MFA_DTYPE_FP8_E4M3) {
        const float vs = h->cfg.kv_latent ? kv->k_scale : kv->v_scale;   // a latent row is key and value
        if (!(kv->k_scale > 0.f) || !isfinite(kv->k_scale) || !(vs > 0.f) || !isfinite(vs))
            return fail(MFA_ERR_INVALID, "%s: FP8 scales must be finite and > 0 (k %g, v %g)", fn,
                        (double)kv->k_scale, (double)kv->v_scale);
    }
    if (batch < 1 || batch > h->cfg.max_batch)
        return fail(MFA_ERR_INVALID, "%s: batch %d outside [1, %d]", fn, batch, h->cfg.max_batch);
    *max_len = ml;
    return MFA_OK;
}

static mfa::KvView make_view(const mfa_ctx* h, const mfa_kv* kv, int32_t max_len) {
    mfa::KvView v;
    v.k = (const uint8_t*)kv->k;
    v.v = (const uint8_t*)kv->v;
    v.seq_lens = kv->seq_lens;
    v.page_table = h->cfg.page_size ? kv->page_table : nullptr;
    v.kv_stride = kv->kv_stride;
    v.pt_stride = kv->pt_stride;
    v.row_bytes = (h->cfg.kv_latent ? mfa::kLatent : mfa::kHeadDim) * (h->cfg.kv_dtype == MFA_DTYPE_FP8_E4M3 ? 1 : 2);
    v.max_len = max_len;
    v.groups = h->cfg.kv_heads;
    return v;
}

// Latent-cache mode: one query token per sequence, chunks of latent_chunk
// tokens, partials merged by a second launch when a sequence has several.
static int decode_latent(mfa_ctx* h, const void* q, const mfa_kv* kv, int32_t max_len, void* out, float* lse_out,
                         int32_t batch, int32_t qtok, void* hip_stream, const char* fn) {
    if (qtok != 1) return fail(MFA_ERR_UNSUPPORTED, "%s: a latent-cache handle decodes one token per sequence", fn);
    mfa::AttnArgs a{};
    a.q = (const uint16_t*)q;
    a.kv = make_view(h, kv, max_len);
    a.out = (uint16_t*)out;
    a.lse_out = lse_out;
    a.part_o = h->part_o;
    a.part_lse = h->part_lse;
    a.counters = h->counters;
    a.batch = batch;
    a.qtok = 1;
    a.nh = 2;
    a.kv_groups = 1;
    a.chunk = h->cfg.split_tokens > 0 ? h->cfg.split_tokens : latent_chunk(h, batch, max_len);
    a.n_chunk = std::max<int32_t>(1, (max_len + a.chunk - 1) / a.chunk);
    if (a.n_chunk > h->max_chunks)
        return fail(MFA_ERR_INVALID, "%s: %d chunks exceed the workspace (%d)", fn, a.n_chunk, h->max_chunks);
    a.part_stride = a.n_chunk;
    if ((int64_t)batch * a.n_chunk > h->part_slots)
        return fail(MFA_ERR_UNSUPPORTED, "%s: %d rows x %d partial slots exceed the workspace's %lld", fn, batch,
                    a.n_chunk, (long long)h->part_slots);
    const float log2e = 1.4426950408889634f;
    a.score_scale = h->cfg.softmax_scale * kv->k_scale * log2e;
    a.v_scale = kv->k_scale;
    hipStream_t st = (hipStream_t)hip_stream;
    const bool paged = h->cfg.page_size != 0;
    hipError_t e = timed_launch(h, MFA_KERNEL_ATTENTION, st, [&](const mfa::Launch& l) { return mfa::launch_mla(a, paged, l); });
    if (e == hipSuccess && a.n_chunk > 1)
        e = timed_launch(h, MFA_KERNEL_COMBINE, st, [&](const mfa::Launch& l) { return mfa::launch_mla_combine(a, l); });
    if (e != hipSuccess) return hip_fail(e, (std::string(fn) + ": launch").c_str());
    return MFA_OK;
}

// mfa_decode (qtok 1) and mfa_decode_mtp (qtok query tokens per sequence).
static int decode_impl(mfa_ctx* h, const void* q, const mfa_kv* kv, int32_t qtok, void* out, float* lse_out,
                       int32_t batch, void* hip_stream, const char* fn) {
    if (!q || !out) return fail(MFA_ERR_INVALID, "%s: null q or out", fn);
    if (qtok < 1 || qtok > mfa::kMaxQueryTokens)
        return fail(MFA_ERR_INVALID, "%s: num_tokens %d outside [1, %d]", fn, qtok, mfa::kMaxQueryTokens);
    int32_t max_len = 0;
    int rc = check_kv(h, kv, batch, fn, &max_len);
    if (rc) return rc;
    if (qtok > 1 && h->cfg.attn_math == MFA_ATTN_FP8_MFMA)
        return fail(MFA_ERR_UNSUPPORTED, "%s: multi-token decode runs with bf16 MFMAs only", fn);
    if (qtok > 1 && h->cfg.kv_heads > 1)
        return fail(MFA_ERR_UNSUPPORTED, "%s: multi-token decode needs kv_heads 1", fn);
    const int32_t rows = batch * qtok;   // query-row sets (one per sequence and token)
    if (rows > h->cfg.max_batch)
        return fail(MFA_ERR_INVALID, "%s: batch %d x num_tokens %d exceeds max_batch %d", fn, batch, qtok,
                    h->cfg.max_batch);
    const bool fp8 = h->cfg.kv_dtype == MFA_DTYPE_FP8_E4M3;
    if (h->cfg.kv_latent) return decode_latent(h, q, kv, max_len, out, lse_out, batch, qtok, hip_stream, fn);
    mfa::AttnArgs a;
    a.q = (const uint16_t*)q;
    a.kv = make_view(h, kv, max_len);
    a.out = (uint16_t*)out;
    a.lse_out = lse_out;
    a.part_o = h->part_o;
    a.part_lse = h->part_lse;
    a.counters = h->counters;
    a.batch = batch;
    a.qtok = qtok;
    a.fp8_mma = h->cfg.attn_math == MFA_ATTN_FP8_MFMA ? 1 : 0;
    int workgroups;
    if (qtok == 1 && use_balanced(h, batch, max_len, kv->min_seq_len)) {
        // equal ranges of at least 4 and at most 128 units: one workgroup per
        // CU, or more when the batch's units could exceed 128 per workgroup
        a.balanced = 1;
        a.chunk = 0;
        a.n_chunk = 0;
        a.part_stride = h->max_chunks + 1;
        a.fuse_max = 1 << 30;   // the last piece of a sequence always merges
        a.nh = 1;
        a.kv_groups = 1;
        // units the ranges deal out (steps plus the per-sequence piece cost)
        const int64_t bound = (int64_t)batch * ((max_len + mfa::kStep - 1) / mfa::kStep + mfa::kBalancedPieceCost);
        int64_t g = h->num_cu;
        if (bound > g * mfa::kMaxPagedChunkSteps) g = round_up((bound + mfa::kMaxPagedChunkSteps - 1) / mfa::kMaxPagedChunkSteps, h->num_cu);
        workgroups = (int)g;
    } else {
        a.balanced = 0;
        plan_chunks(h, rows, qtok, max_len, &a.chunk, &a.nh);
        a.kv_groups = h->cfg.kv_heads;
        a.n_chunk = (max_len + a.chunk - 1) / a.chunk;
        if (a.n_chunk < 1) a.n_chunk = 1;
        if (a.n_chunk > h->max_chunks)
            return fail(MFA_ERR_INVALID, "%s: %d chunks exceed the workspace (%d)", fn, a.n_chunk, h->max_chunks);
        a.part_stride = a.n_chunk;
        a.fuse_max = a.n_chunk <= mfa::kFusedMaxChunks ? mfa::kFusedMaxChunks : 1;
        // several workgroups per (sequence, chunk) (tokens, head halves):
        // groups of 8 work items times their number (see the kernel)
        const int reps = qtok * a.nh;
        workgroups = reps == 1 ? batch * a.n_chunk : round_up((int64_t)batch * a.n_chunk, 8) * reps;
    }
    if ((int64_t)rows * a.part_stride > h->part_slots)
        return fail(MFA_ERR_UNSUPPORTED, "%s: %d query rows x %d partial slots exceed the workspace's %lld", fn, rows,
                    a.part_stride, (long long)h->part_slots);
    const float log2e = 1.4426950408889634f;
    a.score_scale = h->cfg.softmax_scale * (fp8 ? kv->k_scale : 1.0f) * log2e;
    a.v_scale = fp8 ? kv->v_scale : 1.0f;
    hipStream_t st = (hipStream_t)hip_stream;
    const bool paged = h->cfg.page_size != 0;
    hipError_t e = timed_launch(h, MFA_KERNEL_ATTENTION, st,
                                [&](const mfa::Launch& l) { return mfa::launch_attn_split(a, fp8, paged, workgroups, l); });
    if (e == hipSuccess && !a.balanced && a.n_chunk > a.fuse_max)
        e = timed_launch(h, MFA_KERNEL_COMBINE, st, [&](const mfa::Launch& l) { return mfa::launch_combine(a, rows, l); });
    if (e != hipSuccess) return hip_fail(e, (std::string(fn) + ": launch").c_str());
    return MFA_OK;
}

int mfa_decode(mfa_handle h, const void* q, const mfa_kv* kv, void* out, float* lse_out, int32_t batch,
               void* hip_stream) {
    g_last_error[0] = 0;
    if (!valid_handle(h)) return fail(MFA_ERR_INVALID, "mfa_decode: not a live handle");
    return decode_impl(h, q, kv, 1, out, lse_out, batch, hip_stream, "mfa_decode");
}

int mfa_decode_mtp(mfa_handle h, const void* q, const mfa_kv* kv, int32_t num_tokens, void* out, float* lse_out,
                   int32_t batch, void* hip_stream) {
    g_last_error[0] = 0;
    if (!valid_handle(h)) return fail(MFA_ERR_INVALID, "mfa_decode_mtp: not a live handle");
    return decode_impl(h, q, kv, num_tokens, out, lse_out, batch, hip_stream, "mfa_decode_mtp");
}

// The workspace of mfa_decode_noalloc on the current device: the address of
// `scratch` there, taken once per device with the device current, and the
// compute-unit count; the counter region is cleared by a fill kernel on the
// first call's stream (a kernel, not a memset, so that the call may be
// captured in a graph).
static int noalloc_setup(hipStream_t st, ScratchSlot* out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "mfa_decode_noalloc: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MFA_ERR_UNSUPPORTED, "mfa_decode_noalloc: device %d beyond the %d supported", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    ScratchSlot& sl = g_scratch[dev];
    if (!sl.ptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return hip_fail(e, "mfa_decode_noalloc: hipGetSymbolAddress(scratch)");
        int ncu = 0;
        e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return hip_fail(e, "mfa_decode_noalloc: device query");
        sl.ptr = (uint8_t*)p;
        sl.num_cu = ncu;
    }
    if (!sl.cleared) {
        e = mfa::launch_fill_zero((uint32_t*)sl.ptr, kNoAllocCounterBytes / 4, mfa::Launch{st});
        if (e != hipSuccess) return hip_fail(e, "mfa_decode_noalloc: clearing the counters");
        sl.cleared = true;
    }
    *out = sl;
    return MFA_OK;
}

int mfa_decode_noalloc(const mfa_config* cfg, const void* q, const mfa_kv* kv, void* out, float* lse_out,
                       int32_t batch, void* hip_stream) {
    g_last_error[0] = 0;
    if (!cfg) return fail(MFA_ERR_INVALID, "mfa_decode_noalloc: null cfg");
    mfa_config c;
    int rc = validate_config(cfg, &c, "mfa_decode_noalloc");
    if (rc) return rc;
    if (c.kv_latent) return fail(MFA_ERR_UNSUPPORTED, "mfa_decode_noalloc: not for a latent cache");
    if ((int64_t)c.max_batch * 4 * 4 > (int64_t)kNoAllocCounterBytes)
        return fail(MFA_ERR_UNSUPPORTED, "mfa_decode_noalloc: max_batch %d exceeds the scratch's %d", c.max_batch,
                    (int)(kNoAllocCounterBytes / 16));
    hipStream_t st = (hipStream_t)hip_stream;
    ScratchSlot sl;
    rc = noalloc_setup(st, &sl);
    if (rc) return rc;
    // a handle on the stack: the kernels see the same arguments as through
    // mfa_create, with the workspace in the scratch (counters first, then
    // kNoAllocSlots partial row blocks, then their log-sum-exps); the call's
    // split is checked against kNoAllocSlots in decode_impl
    mfa_ctx h{};
    h.cfg = c;
    h.num_cu = sl.num_cu;
    (void)hipGetDevice(&h.device);
    h.max_chunks = (int)workspace_chunks(c);
    h.part_slots = kNoAllocSlots;
    h.counters = (int32_t*)sl.ptr;
    h.part_o = (float*)(sl.ptr + kNoAllocCounterBytes);
    h.part_lse = (float*)(sl.ptr + kNoAllocCounterBytes + kNoAllocSlots * mfa::kHeads * mfa::kHeadDim * 2);
    rc = decode_impl(&h, q, kv, 1, out, lse_out, batch, hip_stream, "mfa_decode_noalloc");
    return rc;
}

int mfa_kv_append(mfa_handle h, const void* x, const void* w_k, const void* w_v, const mfa_kv* kv,
                  int32_t batch, void* hip_stream) {
    g_last_error[0] = 0;
    if (!valid_handle(h)) return fail(MFA_ERR_INVALID, "mfa_kv_append: not a live handle");
    if (h->cfg.kv_heads > 1 || h->cfg.kv_latent)
        return fail(MFA_ERR_UNSUPPORTED, "mfa_kv_append: needs kv_heads 1 and no latent cache");
    if (!x || !w_k || !w_v) return fail(MFA_ERR_INVALID, "mfa_kv_append: null x, w_k or w_v");
    int32_t max_len = 0;
    int rc = check_kv(h, kv, batch, "mfa_kv_append", &max_len);
    if (rc) return rc;
    const bool fp8 = h->cfg.kv_dtype == MFA_DTYPE_FP8_E4M3;
    const bool paged = h->cfg.page_size != 0;
    mfa::KvAppendArgs a;
    a.x = (const uint16_t*)x;
    a.w_k = (const uint16_t*)w_k;
    a.w_v = (const uint16_t*)w_v;
    a.kv_part = h->kv_part;
    a.k = (uint8_t*)const_cast<void*>(kv->k);
    a.v = (uint8_t*)const_cast<void*>(kv->v);
    a.seq_lens = kv->seq_lens;
    a.page_table = paged ? kv->page_table : nullptr;
    a.kv_stride = kv->kv_stride;
    a.pt_stride = kv->pt_stride;
    a.num_pages = kv->num_pages;
    a.batch = batch;
    a.hidden = h->cfg.hidden;
    a.ksplit = kv_ksplit(a.hidden, batch);
    a.k_scale = fp8 ? kv->k_scale : 1.0f;
    a.v_scale = fp8 ? kv->v_scale : 1.0f;
    hipStream_t st = (hipStream_t)hip_stream;
    hipError_t e = timed_launch(h, MFA_KERNEL_KV_PROJ, st, [&](const mfa::Launch& l) { return mfa::launch_kv_proj(a, l); });
    if (e == hipSuccess)
        e = timed_launch(h, MFA_KERNEL_KV_WRITE, st,
                         [&](const mfa::Launch& l) { return mfa::launch_kv_write(a, fp8, paged, l); });
    if (e != hipSuccess) return hip_fail(e, "mfa_kv_append: launch");
    return MFA_OK;
}

int mfa_debug_gather_kv(mfa_handle h, const mfa_kv* kv, int32_t b, void* k_dst, void* v_dst,
                        void* hip_stream) {
    g_last_error[0] = 0;
    if (!valid_handle(h)) return fail(MFA_ERR_INVALID, "mfa_debug_gather_kv: not a live handle");
    if (h->cfg.kv_heads > 1 || h->cfg.kv_latent)
        return fail(MFA_ERR_UNSUPPORTED, "mfa_debug_gather_kv: needs kv_heads 1 and no latent cache");
    if (!k_dst || !v_dst) return fail(MFA_ERR_INVALID, "mfa_debug_gather_kv: null destination");
    int32_t max_len = 0;
    int rc = check_kv(h, kv, h->cfg.max_batch, "mfa_debug_gather_kv", &max_len);
    if (rc) return rc;
    if (b < 0 || b >= h->cfg.max_batch)
        return fail(MFA_ERR_INVALID, "mfa_debug_gather_kv: sequence %d outside [0, %d)", b, h->cfg.max_batch);
    hipError_t e = mfa::launch_gather(make_view(h, kv, max_len), h->cfg.page_size != 0, b, max_len, k_dst, v_dst,
                                      mfa::Launch{(hipStream_t)hip_stream});
    if (e != hipSuccess) return hip_fail(e, "mfa_debug_gather_kv: launch");
    return MFA_OK;
}

int mfa_debug_fp8_mfma(const void* a, const void* b, const float* c, float* d, int32_t n_tiles,
                       void* hip_stream) {
    g_last_error[0] = 0;
    if (!a || !b || !d) return fail(MFA_ERR_INVALID, "mfa_debug_fp8_mfma: null a, b or d");
    if (n_tiles < 0 || n_tiles > (1 << 20))
        return fail(MFA_ERR_INVALID, "mfa_debug_fp8_mfma: n_tiles %d outside [0, 2^20]", n_tiles);
    if (n_tiles == 0) return MFA_OK;
    hipError_t e = mfa::launch_fp8_mfma((const uint8_t*)a, (const uint8_t*)b, c, d, n_tiles,
                                        mfa::Launch{(hipStream_t)hip_stream});
    if (e != hipSuccess) return hip_fail(e, "mfa_debug_fp8_mfma: launch");
    return MFA_OK;
}

int mfa_debug_mfma_rate(int32_t kind, int32_t iters, float* sink, double* flops, void* hip_stream) {
    g_last_error[0] = 0;
    if (kind != 0 && kind != 1) return fail(MFA_ERR_INVALID, "mfa_debug_mfma_rate: kind %d is not 0 or 1", kind);
    if (iters < 1 || iters > (1 << 24))
        return fail(MFA_ERR_INVALID, "mfa_debug_mfma_rate: iters %d outside [1, 2^24]", iters);
    if (!sink || !flops) return fail(MFA_ERR_INVALID, "mfa_debug_mfma_rate: null sink or flops");
    int dev = 0, ncu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "mfa_debug_mfma_rate: device query");
    const int workgroups = 2 * ncu;   // two waves per SIMD
    *flops = mfa::mfma_rate_flops(kind, iters, workgroups);
    e = mfa::launch_mfma_rate(kind, iters, workgroups, sink, mfa::Launch{(hipStream_t)hip_stream});
    if (e != hipSuccess) return hip_fail(e, "mfa_debug_mfma_rate: launch");
    return MFA_OK;
}

int mfa_profile_enable(mfa_handle h, int enable) {
    g_last_error[0] = 0;
    if (!valid_handle(h)) return fail(MFA_ERR_INVALID, "mfa_profile_enable: not a live handle");
    Profiler& p = h->prof;
    if (!enable) {
        profiler_release(p);
        return MFA_OK;
    }
    if (p.on) return MFA_OK;
    p.ev.assign(2 * Profiler::kCap, nullptr);
    p.kind.assign(Profiler::kCap, -1);
    for (auto& e : p.ev) {
        hipError_t r = hipEventCreateWithFlags(&e, hipEventReleaseToDevice);
        if (r != hipSuccess) {
            profiler_release(p);
            return hip_fail(r, "mfa_profile_enable: hipEventCreate");
        }
    }
    p.next = 0;
    p.on = true;
    return MFA_OK;
}

int mfa_profile_read(mfa_handle h, int32_t* launches, double* total_ms) {
    g_last_error[0] = 0;
    if (!valid_handle(h)) return fail(MFA_ERR_INVALID, "mfa_profile_read: not a live handle");
    if (!launches || !total_ms) return fail(MFA_ERR_INVALID, "mfa_profile_read: null output");
    for (int k = 0; k < MFA_KERNEL_KINDS; k++) {
        launches[k] = 0;
        total_ms[k] = 0.0;
    }
    Profiler& p = h->prof;
    if (!p.on) return MFA_OK;
    for (int i = 0; i < Profiler::kCap; i++) {
        if (p.kind[i] < 0) continue;
        hipError_t r = hipEventSynchronize(p.ev[2 * i + 1]);
        float ms = 0.f;
        if (r == hipSuccess) r = hipEventElapsedTime(&ms, p.ev[2 * i], p.ev[2 * i + 1]);
        if (r != hipSuccess) return hip_fail(r, "mfa_profile_read");
        launches[p.kind[i]] += 1;
        total_ms[p.kind[i]] += ms;
        p.kind[i] = -1;
    }
    p.next = 0;
    return MFA_OK;
}

}  // extern "C"
