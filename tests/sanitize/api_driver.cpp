// api_driver.cpp -- drives every entry point of the C ABI over the host-memory
// HIP stand-in (hip_stub.cpp), built with sanitizers: argument checks,
// split planning for many shapes, workspace bounds (checked by the stand-in's
// launchers), handle lifetime (a destroyed or foreign pointer is rejected
// without reading freed memory), allocation-failure clean-up and concurrent
// create / use / destroy from several threads. Exits 0 when every expectation
// holds; prints the first failure and exits 1 otherwise.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <thread>
#include <vector>

#include "mfa.h"
#include "stub_control.h"

static int g_failures = 0;

#define EXPECT(cond, ...)                                           \
    do {                                                            \
        if (!(cond)) {                                              \
            fprintf(stderr, "%s:%d: expectation failed: %s: ", __FILE__, __LINE__, #cond); \
            fprintf(stderr, __VA_ARGS__);                           \
            fprintf(stderr, " [last error: %s]\n", mfa_last_error()); \
            g_failures++;                                           \
        }                                                           \
    } while (0)

static mfa_config base_config() {
    mfa_config c;
    memset(&c, 0, sizeof c);
    c.hidden = 7168;
    c.q_rank = 2048;
    c.num_heads = 64;
    c.head_dim = 256;
    c.kv_dtype = MFA_DTYPE_FP8_E4M3;
    c.page_size = 0;
    c.max_batch = 32;
    c.max_context = 4096;
    c.split_tokens = 0;
    c.rms_eps = 1e-6f;
    c.softmax_scale = 1.0f / 16.0f;
    c.attn_math = MFA_ATTN_BF16_MFMA;
    c.kv_heads = 0;
    return c;
}

// a dummy device buffer: the stand-in's launchers never read tensors
static char g_dummy[64];

struct Kv {
    std::vector<int32_t> lens, pt;
    mfa_kv kv;
};

static Kv make_kv(const mfa_config& c, int batch, int max_len, int min_len) {
    Kv r;
    r.lens.assign((size_t)batch, 0);
    for (int b = 0; b < batch; b++) r.lens[(size_t)b] = min_len + (max_len - min_len) * b / (batch > 1 ? batch - 1 : 1);
    memset(&r.kv, 0, sizeof r.kv);
    r.kv.k = g_dummy;
    r.kv.v = g_dummy;
    r.kv.k_scale = 0.05f;
    r.kv.v_scale = 0.02f;
    r.kv.seq_lens = r.lens.data();
    r.kv.max_seq_len = max_len;
    r.kv.min_seq_len = min_len;
    const int ml = max_len > 0 ? max_len : c.max_context;
    if (c.page_size) {
        r.kv.pt_stride = (ml + 63) / 64;
        r.pt.assign((size_t)batch * r.kv.pt_stride, 0);
        r.kv.page_table = r.pt.data();
        r.kv.num_pages = 1;
    } else {
        r.kv.kv_stride = ml;
    }
    return r;
}

static void bad_configs() {
    mfa_handle h = nullptr;
    EXPECT(mfa_create(nullptr, &h) == MFA_ERR_INVALID, "null cfg");
    mfa_config c = base_config();
    EXPECT(mfa_create(&c, nullptr) == MFA_ERR_INVALID, "null out");
    struct Case {
        void (*edit)(mfa_config&);
        int want;
    } cases[] = {
        {[](mfa_config& c) { c.num_heads = 32; }, MFA_ERR_UNSUPPORTED},
        {[](mfa_config& c) { c.head_dim = 128; }, MFA_ERR_UNSUPPORTED},
        {[](mfa_config& c) { c.hidden = 7000; }, MFA_ERR_UNSUPPORTED},
        {[](mfa_config& c) { c.hidden = -512; }, MFA_ERR_UNSUPPORTED},
        {[](mfa_config& c) { c.q_rank = 100; }, MFA_ERR_UNSUPPORTED},
        {[](mfa_config& c) { c.q_rank = 8192; }, MFA_ERR_UNSUPPORTED},
        {[](mfa_config& c) { c.kv_dtype = 7; }, MFA_ERR_INVALID},
        {[](mfa_config& c) { c.page_size = 16; }, MFA_ERR_UNSUPPORTED},
        {[](mfa_config& c) { c.max_batch = 0; }, MFA_ERR_INVALID},
        {[](mfa_config& c) { c.max_context = -5; }, MFA_ERR_INVALID},
        {[](mfa_config& c) { c.split_tokens = 100; }, MFA_ERR_INVALID},
        {[](mfa_config& c) { c.split_tokens = -2; }, MFA_ERR_INVALID},
        {[](mfa_config& c) { c.page_size = 64; c.split_tokens = 16384; }, MFA_ERR_UNSUPPORTED},
        {[](mfa_config& c) { c.softmax_scale = 0.f; }, MFA_ERR_INVALID},
        {[](mfa_config& c) { c.softmax_scale = __builtin_nanf(""); }, MFA_ERR_INVALID},
        {[](mfa_config& c) { c.softmax_scale = __builtin_inff(); }, MFA_ERR_INVALID},
        {[](mfa_config& c) { c.rms_eps = -1.f; }, MFA_ERR_INVALID},
        {[](mfa_config& c) { c.attn_math = 5; }, MFA_ERR_INVALID},
        {[](mfa_config& c) { c.kv_dtype = MFA_DTYPE_BF16; c.attn_math = MFA_ATTN_FP8_MFMA; }, MFA_ERR_UNSUPPORTED},
        {[](mfa_config& c) { c.kv_heads = 3; }, MFA_ERR_INVALID},
        {[](mfa_config& c) { c.kv_heads = 2; c.attn_math = MFA_ATTN_FP8_MFMA; }, MFA_ERR_UNSUPPORTED},
        {[](mfa_config& c) { c.kv_heads = 4; c.split_tokens = MFA_SPLIT_BALANCED; }, MFA_ERR_UNSUPPORTED},
        {[](mfa_config& c) { c.max_batch = 1 << 30; c.max_context = 1 << 30; }, MFA_ERR_INVALID},
        {[](mfa_config& c) { c.kv_latent = 256; }, MFA_ERR_INVALID},
        {[](mfa_config& c) { c.kv_latent = 512; c.kv_dtype = MFA_DTYPE_BF16; }, MFA_ERR_UNSUPPORTED},
        {[](mfa_config& c) { c.kv_latent = 512; c.split_tokens = MFA_SPLIT_BALANCED; }, MFA_ERR_UNSUPPORTED},
    };
    for (const Case& k : cases) {
        mfa_config b = base_config();
        k.edit(b);
        h = (mfa_handle)g_dummy;
        const int rc = mfa_create(&b, &h);
        EXPECT(rc == k.want, "config case: got %d want %d", rc, k.want);
        EXPECT(h == nullptr, "failed create leaves *out null");
        EXPECT(strlen(mfa_last_error()) > 0, "failed create sets a message");
        const int rc2 = mfa_decode_noalloc(&b, g_dummy, nullptr, g_dummy, nullptr, 1, nullptr);
        EXPECT(rc2 < 0, "noalloc config case: got %d", rc2);
    }
}

// every call shape on one handle: the launchers check the workspace bounds
static void sweep(const mfa_config& c) {
    mfa_handle h = nullptr;
    int rc = mfa_create(&c, &h);
    EXPECT(rc == MFA_OK, "create (dtype %d page %d split %d math %d G %d)", c.kv_dtype, c.page_size,
           c.split_tokens, c.attn_math, c.kv_heads);
    if (rc) return;
    const int G = c.kv_heads > 1 ? c.kv_heads : 1;
    const int batches[] = {1, 2, 7, c.max_batch / 2, c.max_batch};
    const int lens[] = {0, 1, 63, 64, 65, 1000, c.max_context - 1, c.max_context};
    for (int batch : batches) {
        if (batch < 1) continue;
        for (int ml : lens) {
            for (int minl : {0, 1, ml}) {
                if (minl > (ml > 0 ? ml : c.max_context)) continue;
                Kv kv = make_kv(c, batch, ml, minl);
                rc = mfa_decode(h, g_dummy, &kv.kv, g_dummy, (float*)g_dummy, batch, nullptr);
                EXPECT(rc == MFA_OK, "decode batch %d max %d min %d: %d", batch, ml, minl, rc);
                const int32_t st = mfa_split_tokens(h, batch, ml, minl);
                const int32_t hg = mfa_head_groups(h, batch, ml, minl);
                EXPECT(st >= 0 && st % 64 == 0, "split tokens %d", st);
                EXPECT(hg >= 1 && hg <= 4, "head groups %d", hg);
                if (G > 1) EXPECT(hg == G, "grouped head groups %d", hg);
                if (G == 1 && c.attn_math == MFA_ATTN_BF16_MFMA && !c.kv_latent) {
                    for (int t : {2, 3, 4, 16}) {
                        const int want = batch * t <= c.max_batch ? MFA_OK : MFA_ERR_INVALID;
                        rc = mfa_decode_mtp(h, g_dummy, &kv.kv, t, g_dummy, nullptr, batch, nullptr);
                        EXPECT(rc == want, "mtp %d x %d: %d", batch, t, rc);
                        const int32_t sm = mfa_split_tokens_mtp(h, batch, t, ml);
                        if (want == MFA_OK) EXPECT(sm > 0 && sm % 64 == 0 && sm <= 8192, "mtp split %d", sm);
                        else EXPECT(sm == MFA_ERR_INVALID, "mtp split %d x %d: %d", batch, t, sm);
                    }
                }
                if (G == 1) {
                    rc = mfa_kv_append(h, g_dummy, g_dummy, g_dummy, &kv.kv, batch, nullptr);
                    EXPECT(rc == (c.kv_latent ? MFA_ERR_UNSUPPORTED : MFA_OK), "append batch %d: %d", batch, rc);
                }
                rc = mfa_decode_noalloc(&c, g_dummy, &kv.kv, g_dummy, nullptr, batch, nullptr);
                EXPECT(rc == MFA_OK || rc == MFA_ERR_UNSUPPORTED, "noalloc batch %d max %d: %d", batch, ml, rc);
            }
        }
        rc = mfa_qproj(h, g_dummy, g_dummy, g_dummy, g_dummy, g_dummy, batch, nullptr);
        EXPECT(rc == (c.kv_latent ? MFA_ERR_UNSUPPORTED : MFA_OK), "qproj batch %d: %d", batch, rc);
    }
    // rejections on a live handle
    Kv kv = make_kv(c, 4, 100, 0);
    EXPECT(mfa_decode(h, g_dummy, &kv.kv, g_dummy, nullptr, 0, nullptr) == MFA_ERR_INVALID, "batch 0");
    EXPECT(mfa_decode(h, g_dummy, &kv.kv, g_dummy, nullptr, c.max_batch + 1, nullptr) == MFA_ERR_INVALID,
           "batch > max");
    EXPECT(mfa_decode(h, nullptr, &kv.kv, g_dummy, nullptr, 4, nullptr) == MFA_ERR_INVALID, "null q");
    EXPECT(mfa_decode(h, g_dummy, nullptr, g_dummy, nullptr, 4, nullptr) == MFA_ERR_INVALID, "null kv");
    EXPECT(mfa_decode_mtp(h, g_dummy, &kv.kv, 17, g_dummy, nullptr, 1, nullptr) != MFA_OK, "17 tokens");
    EXPECT(mfa_decode_mtp(h, g_dummy, &kv.kv, 0, g_dummy, nullptr, 1, nullptr) != MFA_OK, "0 tokens");
    mfa_kv bad = kv.kv;
    bad.max_seq_len = c.max_context + 1;
    EXPECT(mfa_decode(h, g_dummy, &bad, g_dummy, nullptr, 4, nullptr) == MFA_ERR_INVALID, "max_seq_len > max");
    bad = kv.kv;
    bad.max_seq_len = -1;
    EXPECT(mfa_decode(h, g_dummy, &bad, g_dummy, nullptr, 4, nullptr) == MFA_ERR_INVALID, "max_seq_len < 0");
    bad = kv.kv;
    bad.seq_lens = nullptr;
    EXPECT(mfa_decode(h, g_dummy, &bad, g_dummy, nullptr, 4, nullptr) == MFA_ERR_INVALID, "null lens");
    if (c.page_size) {
        bad = kv.kv;
        bad.page_table = nullptr;
        EXPECT(mfa_decode(h, g_dummy, &bad, g_dummy, nullptr, 4, nullptr) == MFA_ERR_INVALID, "no page table");
        bad = kv.kv;
        bad.pt_stride = 1;
        EXPECT(mfa_decode(h, g_dummy, &bad, g_dummy, nullptr, 4, nullptr) == MFA_ERR_INVALID, "short pt_stride");
        bad = kv.kv;
        bad.num_pages = 0;
        EXPECT(mfa_decode(h, g_dummy, &bad, g_dummy, nullptr, 4, nullptr) == MFA_ERR_INVALID, "no pages");
    } else {
        bad = kv.kv;
        bad.kv_stride = 99;
        EXPECT(mfa_decode(h, g_dummy, &bad, g_dummy, nullptr, 4, nullptr) == MFA_ERR_INVALID, "short kv_stride");
        bad = kv.kv;
        bad.page_table = kv.lens.data();
        EXPECT(mfa_decode(h, g_dummy, &bad, g_dummy, nullptr, 4, nullptr) == MFA_ERR_INVALID, "unexpected table");
    }
    if (c.kv_dtype == MFA_DTYPE_FP8_E4M3) {
        bad = kv.kv;
        bad.k_scale = 0.f;
        EXPECT(mfa_decode(h, g_dummy, &bad, g_dummy, nullptr, 4, nullptr) == MFA_ERR_INVALID, "zero k_scale");
        bad = kv.kv;
        bad.v_scale = __builtin_inff();   // ignored by a latent cache (its rows are keys and values)
        EXPECT(mfa_decode(h, g_dummy, &bad, g_dummy, nullptr, 4, nullptr) == (c.kv_latent ? MFA_OK : MFA_ERR_INVALID),
               "inf v_scale");
    }
    EXPECT(mfa_qproj(h, nullptr, g_dummy, g_dummy, g_dummy, g_dummy, 1, nullptr) < 0, "qproj null");
    EXPECT(mfa_kv_append(h, g_dummy, nullptr, g_dummy, &kv.kv, 1, nullptr) != MFA_OK, "append null");
    if (G == 1 && !c.kv_latent) {
        EXPECT(mfa_debug_gather_kv(h, &kv.kv, 0, g_dummy, g_dummy, nullptr) == MFA_OK, "gather");
        EXPECT(mfa_debug_gather_kv(h, &kv.kv, c.max_batch, g_dummy, g_dummy, nullptr) == MFA_ERR_INVALID,
               "gather b out of range");
    }
    // profiling: events around every launch, read back, released
    EXPECT(mfa_profile_enable(h, 1) == MFA_OK, "profile on");
    EXPECT(mfa_profile_enable(h, 1) == MFA_OK, "profile on twice");
    for (int i = 0; i < 5000; i++)   // more launches than the event ring holds
        (void)mfa_decode(h, g_dummy, &kv.kv, g_dummy, nullptr, 4, nullptr);
    int32_t n[MFA_KERNEL_KINDS];
    double ms[MFA_KERNEL_KINDS];
    EXPECT(mfa_profile_read(h, n, ms) == MFA_OK, "profile read");
    EXPECT(n[MFA_KERNEL_ATTENTION] > 0 && n[MFA_KERNEL_ATTENTION] <= 4096, "attention launches %d", n[0]);
    EXPECT(mfa_profile_read(h, nullptr, ms) == MFA_ERR_INVALID, "profile read null");
    EXPECT(mfa_profile_enable(h, 0) == MFA_OK, "profile off");
    EXPECT(mfa_profile_read(h, n, ms) == MFA_OK && n[0] == 0, "profile read when off");
    EXPECT(mfa_profile_enable(h, 1) == MFA_OK, "profile on again (released by destroy)");
    EXPECT(mfa_destroy(h) == MFA_OK, "destroy");
}

// a destroyed pointer, a pointer that never was a handle and NULL are
// rejected by every entry point that takes a handle, without touching them
static void stale_handles() {
    mfa_config c = base_config();
    mfa_handle h = nullptr;
    EXPECT(mfa_create(&c, &h) == MFA_OK, "create");
    EXPECT(mfa_destroy(h) == MFA_OK, "destroy");
    long fake_storage[64] = {0};
    mfa_handle foreign = (mfa_handle)fake_storage;
    Kv kv = make_kv(c, 2, 64, 0);
    int32_t n[MFA_KERNEL_KINDS];
    double ms[MFA_KERNEL_KINDS];
    for (mfa_handle x : {h, foreign, (mfa_handle) nullptr}) {
        EXPECT(mfa_decode(x, g_dummy, &kv.kv, g_dummy, nullptr, 2, nullptr) == MFA_ERR_INVALID, "decode");
        EXPECT(mfa_decode_mtp(x, g_dummy, &kv.kv, 2, g_dummy, nullptr, 1, nullptr) == MFA_ERR_INVALID, "mtp");
        EXPECT(mfa_qproj(x, g_dummy, g_dummy, g_dummy, g_dummy, g_dummy, 1, nullptr) == MFA_ERR_INVALID, "qproj");
        EXPECT(mfa_kv_append(x, g_dummy, g_dummy, g_dummy, &kv.kv, 1, nullptr) == MFA_ERR_INVALID, "append");
        EXPECT(mfa_debug_gather_kv(x, &kv.kv, 0, g_dummy, g_dummy, nullptr) == MFA_ERR_INVALID, "gather");
        EXPECT(mfa_split_tokens(x, 1, 64, 0) == MFA_ERR_INVALID, "split_tokens");
        EXPECT(mfa_head_groups(x, 1, 64, 0) == MFA_ERR_INVALID, "head_groups");
        EXPECT(mfa_profile_enable(x, 1) == MFA_ERR_INVALID, "profile_enable");
        EXPECT(mfa_profile_read(x, n, ms) == MFA_ERR_INVALID, "profile_read");
        if (x) EXPECT(mfa_destroy(x) == MFA_ERR_INVALID, "destroy again");
    }
    EXPECT(mfa_destroy(nullptr) == MFA_OK, "destroy null");
}

// the k-th workspace allocation fails: NOMEM, nothing left allocated
static void allocation_failures() {
    mfa_config c = base_config();
    for (int k = 0; k < 8; k++) {
        const long before = stub_live_allocations();
        stub_fail_malloc_at(k);
        mfa_handle h = (mfa_handle)g_dummy;
        const int rc = mfa_create(&c, &h);
        stub_fail_malloc_at(-1);
        EXPECT(rc == MFA_ERR_NOMEM, "allocation %d fails: %d", k, rc);
        EXPECT(h == nullptr, "no handle after failure");
        EXPECT(stub_live_allocations() == before, "allocation %d: %ld blocks left", k,
               stub_live_allocations() - before);
    }
}

static void noalloc_limits() {
    mfa_config c = base_config();
    c.max_batch = 65537;
    Kv kv = make_kv(c, 1, 64, 0);
    EXPECT(mfa_decode_noalloc(&c, g_dummy, &kv.kv, g_dummy, nullptr, 1, nullptr) == MFA_ERR_UNSUPPORTED,
           "max_batch beyond the scratch");
    c = base_config();
    c.max_batch = 4096;
    c.max_context = 65536;
    c.split_tokens = MFA_SPLIT_BALANCED;
    Kv big = make_kv(c, 4096, 65536, 0);
    EXPECT(mfa_decode_noalloc(&c, g_dummy, &big.kv, g_dummy, nullptr, 4096, nullptr) == MFA_ERR_UNSUPPORTED,
           "split beyond the scratch's partial slots");
    EXPECT(mfa_decode_noalloc(nullptr, g_dummy, &kv.kv, g_dummy, nullptr, 1, nullptr) == MFA_ERR_INVALID, "null cfg");
}

// the matrix-core rate microbenchmark: argument checks and the flop count
static void mfma_rate() {
    double fl = 0;
    for (int kind : {0, 1}) {
        EXPECT(mfa_debug_mfma_rate(kind, 100, (float*)g_dummy, &fl, nullptr) == MFA_OK, "mfma rate kind %d", kind);
        EXPECT(fl == 2.0 * 256 * 4 * 100 * 8 * 2 * 16 * 16 * (kind == 0 ? 32 : 128), "mfma rate flops %g", fl);
    }
    EXPECT(mfa_debug_mfma_rate(2, 100, (float*)g_dummy, &fl, nullptr) == MFA_ERR_INVALID, "mfma rate kind 2");
    EXPECT(mfa_debug_mfma_rate(0, 0, (float*)g_dummy, &fl, nullptr) == MFA_ERR_INVALID, "mfma rate iters 0");
    EXPECT(mfa_debug_mfma_rate(0, (1 << 24) + 1, (float*)g_dummy, &fl, nullptr) == MFA_ERR_INVALID, "mfma rate iters");
    EXPECT(mfa_debug_mfma_rate(0, 100, nullptr, &fl, nullptr) == MFA_ERR_INVALID, "mfma rate null sink");
    EXPECT(mfa_debug_mfma_rate(0, 100, (float*)g_dummy, nullptr, nullptr) == MFA_ERR_INVALID, "mfma rate null flops");
}

// handles created, used and destroyed on several threads at once
static void threads() {
    std::vector<std::thread> ts;
    std::vector<int> bad(8, 0);
    for (int t = 0; t < 8; t++) {
        ts.emplace_back([t, &bad] {
            mfa_config c = base_config();
            c.max_batch = 8;
            c.max_context = 1024;
            c.page_size = (t & 1) ? 64 : 0;
            for (int i = 0; i < 50; i++) {
                mfa_handle h = nullptr;
                if (mfa_create(&c, &h) != MFA_OK) { bad[t]++; continue; }
                Kv kv = make_kv(c, 8, 1024, 0);
                if (mfa_decode(h, g_dummy, &kv.kv, g_dummy, nullptr, 8, nullptr) != MFA_OK) bad[t]++;
                if (mfa_destroy(h) != MFA_OK) bad[t]++;
                if (mfa_decode(h, g_dummy, &kv.kv, g_dummy, nullptr, 8, nullptr) != MFA_ERR_INVALID) bad[t]++;
            }
        });
    }
    for (auto& th : ts) th.join();
    for (int t = 0; t < 8; t++) EXPECT(bad[t] == 0, "thread %d: %d failures", t, bad[t]);
}

int main(int argc, char** argv) {
    const bool only_threads = argc > 1 && strcmp(argv[1], "threads") == 0;
    if (!only_threads) {
        bad_configs();
        for (int dtype : {MFA_DTYPE_BF16, MFA_DTYPE_FP8_E4M3})
            for (int page : {0, 64})
                for (int split : {0, MFA_SPLIT_BALANCED, 256, 1024}) {
                    mfa_config c = base_config();
                    c.kv_dtype = dtype;
                    c.page_size = page;
                    c.split_tokens = split;
                    sweep(c);
                    if (dtype == MFA_DTYPE_FP8_E4M3) {
                        c.attn_math = MFA_ATTN_FP8_MFMA;
                        sweep(c);
                        c.attn_math = MFA_ATTN_BF16_MFMA;
                    }
                    if (split != MFA_SPLIT_BALANCED)
                        for (int g : {2, 4}) {
                            c.kv_heads = g;
                            sweep(c);
                        }
                }
        for (int page : {0, 64})   // latent-cache handles
            for (int split : {0, 256, 1024}) {
                mfa_config c = base_config();
                c.kv_dtype = MFA_DTYPE_FP8_E4M3;
                c.page_size = page;
                c.split_tokens = split;
                c.kv_latent = 512;
                sweep(c);
            }
        for (int cu : {1, 8, 80, 304}) {   // planning for other compute-unit counts
            stub_set_num_cu(cu);
            mfa_config c = base_config();
            c.max_batch = 300;
            c.max_context = 20000;
            sweep(c);
            c.attn_math = MFA_ATTN_FP8_MFMA;
            c.page_size = 64;
            sweep(c);
        }
        stub_set_num_cu(256);
        stale_handles();
        allocation_failures();
        noalloc_limits();
        mfma_rate();
    }
    threads();
    EXPECT(stub_live_allocations() == 0, "%ld workspace blocks never freed", stub_live_allocations());
    if (g_failures) {
        fprintf(stderr, "%d expectation(s) failed\n", g_failures);
        return 1;
    }
    printf("api_driver: ok, %ld launches checked\n", stub_launches());
    return 0;
}
