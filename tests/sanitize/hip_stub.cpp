// hip_stub.cpp -- a host-memory stand-in for the HIP runtime and the kernel
// launchers, so that the C ABI's host code (mfa_api.hip built host-only)
// runs under AddressSanitizer / UndefinedBehaviorSanitizer / ThreadSanitizer
// on a machine without a GPU.
//
// Device memory is host memory from malloc, every allocation recorded with
// its size. Each launcher checks that the workspace regions its kernel would
// touch (sizes as the kernels index them) lie inside one recorded allocation
// or registered device variable, and counts the launch; no kernel runs. A
// failed check prints what it found and aborts.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <map>
#include <mutex>

#include "mfa_internal.h"
#include "stub_control.h"

namespace {
// built on first use: the compiler's module constructor registers the
// library's __device__ variables before this file's globals are constructed
struct Registry {
    std::mutex mu;
    std::map<const char*, size_t> allocs;   // hipMalloc'd blocks: base -> bytes
    std::map<const char*, size_t> vars;     // registered __device__ variables (never freed)
};
Registry& reg() {
    static Registry* r = new Registry();
    return *r;
}
std::atomic<int> g_malloc_calls{0};
std::atomic<int> g_fail_at{-1};
std::atomic<long> g_launches{0};
int g_num_cu = 256;

[[noreturn]] void die(const char* what, const void* p, size_t need) {
    fprintf(stderr, "hip_stub: %s: %p needs %zu bytes outside any allocation\n", what, p, need);
    fflush(stderr);
    abort();
}

// p .. p + bytes must lie in one allocation or registered variable
void need(const char* what, const void* p, size_t bytes) {
    std::lock_guard<std::mutex> lock(reg().mu);
    const char* c = (const char*)p;
    for (auto* m : {&reg().allocs, &reg().vars}) {
        auto it = m->upper_bound(c);
        if (it == m->begin()) continue;
        --it;
        if (c >= it->first && c + bytes <= it->first + it->second) return;
    }
    die(what, p, bytes);
}
}  // namespace

extern "C" {
void stub_fail_malloc_at(int k) {
    g_malloc_calls = 0;
    g_fail_at = k;
}
long stub_live_allocations(void) {
    std::lock_guard<std::mutex> lock(reg().mu);
    return (long)reg().allocs.size();
}
long stub_launches(void) { return g_launches.load(); }
void stub_set_num_cu(int n) { g_num_cu = n; }

hipError_t hipGetDevice(int* d) {
    if (!d) return hipErrorInvalidValue;
    *d = 0;
    return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t a, int dev) {
    if (!v || dev != 0) return hipErrorInvalidValue;
    *v = a == hipDeviceAttributeMultiprocessorCount ? g_num_cu : 0;
    return hipSuccess;
}
hipError_t hipMalloc(void** p, size_t n) {
    if (!p) return hipErrorInvalidValue;
    *p = nullptr;
    if (g_malloc_calls++ == g_fail_at) return hipErrorOutOfMemory;
    void* q = malloc(n ? n : 1);
    if (!q) return hipErrorOutOfMemory;
    std::lock_guard<std::mutex> lock(reg().mu);
    reg().allocs[(const char*)q] = n;
    *p = q;
    return hipSuccess;
}
hipError_t hipFree(void* p) {
    if (!p) return hipSuccess;
    {
        std::lock_guard<std::mutex> lock(reg().mu);
        if (reg().allocs.erase((const char*)p) == 0) {
            fprintf(stderr, "hip_stub: hipFree of %p, not an allocation\n", p);
            abort();
        }
    }
    free(p);
    return hipSuccess;
}
hipError_t hipMemset(void* p, int v, size_t n) {
    need("hipMemset", p, n);
    memset(p, v, n);
    return hipSuccess;
}
hipError_t hipDeviceSynchronize(void) { return hipSuccess; }
hipError_t hipGetLastError(void) { return hipSuccess; }
const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "stub error"; }
hipError_t hipGetSymbolAddress(void** p, const void* sym) {
    if (!p) return hipErrorInvalidValue;
    std::lock_guard<std::mutex> lock(reg().mu);
    if (!reg().vars.count((const char*)sym)) return hipErrorInvalidSymbol;
    *p = const_cast<void*>(sym);   // the host shadow stands in for the device copy
    return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) {
    if (!e) return hipErrorInvalidValue;
    *e = (hipEvent_t)malloc(16);
    return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t e) {
    free(e);
    return hipSuccess;
}
hipError_t hipEventSynchronize(hipEvent_t e) { return e ? hipSuccess : hipErrorInvalidValue; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t a, hipEvent_t b) {
    if (!ms || !a || !b) return hipErrorInvalidValue;
    *ms = 0.001f;
    return hipSuccess;
}

// module registration emitted by the compiler for the file's __device__ variables
void** __hipRegisterFatBinary(const void*) {
    static void* handle = nullptr;
    return &handle;
}
void __hipUnregisterFatBinary(void**) {}
void __hipRegisterVar(void**, char* host_var, char*, const char*, int, size_t size, int, int) {
    std::lock_guard<std::mutex> lock(reg().mu);
    reg().vars[host_var] = size;
}
}  // extern "C"

// ----------------------------------------------------------- the launchers
namespace mfa {

static void check_attn(const AttnArgs& a, int64_t rows, const char* what) {
    if (rows < 1) die(what, nullptr, 0);
    const int64_t slots = rows * (int64_t)a.part_stride;
    need(what, a.part_o, (size_t)slots * kHeads * kHeadDim * 2);
    need(what, a.part_lse, (size_t)slots * kHeads * 4);
    need(what, a.counters, (size_t)rows * 4 * sizeof(int32_t));
}

hipError_t launch_attn_split(const AttnArgs& a, bool, bool paged, int workgroups, const Launch&) {
    if (workgroups < 1) die("launch_attn_split: workgroups", nullptr, 0);
    if (paged != (a.kv.page_table != nullptr)) die("launch_attn_split: paged flag", a.kv.page_table, 0);
    if (!a.balanced && (a.chunk <= 0 || a.chunk % kStep || (int64_t)a.chunk * a.n_chunk < a.kv.max_len))
        die("launch_attn_split: chunks do not cover max_len", nullptr, (size_t)a.chunk);
    if (paged && !a.balanced && a.chunk > kMaxPieceSteps * kStep)
        die("launch_attn_split: paged chunk beyond the page registers", nullptr, (size_t)a.chunk);
    if (a.nh < 1 || a.nh > 4) die("launch_attn_split: head groups", nullptr, (size_t)a.nh);
    check_attn(a, a.balanced ? a.batch : (int64_t)a.batch * a.qtok, "launch_attn_split");
    g_launches++;
    return hipSuccess;
}
hipError_t launch_mla(const AttnArgs& a, bool paged, const Launch&) {
    if (paged != (a.kv.page_table != nullptr)) die("launch_mla: paged flag", a.kv.page_table, 0);
    if (a.chunk <= 0 || a.chunk % kStep || (int64_t)a.chunk * a.n_chunk < a.kv.max_len)
        die("launch_mla: chunks do not cover max_len", nullptr, (size_t)a.chunk);
    const int64_t slots = (int64_t)a.batch * a.n_chunk;
    need("launch_mla part_o", a.part_o, (size_t)slots * kHeads * kLatent * 2);
    need("launch_mla part_lse", a.part_lse, (size_t)slots * kHeads * 4);
    g_launches++;
    return hipSuccess;
}
hipError_t launch_mla_combine(const AttnArgs& a, const Launch&) {
    const int64_t slots = (int64_t)a.batch * a.n_chunk;
    need("launch_mla_combine part_o", a.part_o, (size_t)slots * kHeads * kLatent * 2);
    g_launches++;
    return hipSuccess;
}
hipError_t launch_combine(const AttnArgs& a, int rows, const Launch&) {
    check_attn(a, rows, "launch_combine");
    g_launches++;
    return hipSuccess;
}
hipError_t launch_gather(const KvView&, bool, int b, int max_seq_len, void* k_dst, void* v_dst, const Launch&) {
    if (b < 0 || max_seq_len < 0 || !k_dst || !v_dst) die("launch_gather", nullptr, 0);
    g_launches++;
    return hipSuccess;
}
hipError_t launch_fill_zero(uint32_t* p, size_t n, const Launch&) {
    need("launch_fill_zero", p, n * 4);
    memset(p, 0, n * 4);
    g_launches++;
    return hipSuccess;
}
hipError_t launch_fp8_mfma(const uint8_t* a, const uint8_t* b, const float*, float* d, int n_tiles, const Launch&) {
    if (!a || !b || !d || n_tiles < 1) die("launch_fp8_mfma", nullptr, 0);
    g_launches++;
    return hipSuccess;
}
hipError_t launch_mfma_rate(int kind, int iters, int workgroups, float* sink, const Launch&) {
    if ((kind != 0 && kind != 1) || iters < 1 || workgroups < 1 || !sink) die("launch_mfma_rate", nullptr, 0);
    g_launches++;
    return hipSuccess;
}
double mfma_rate_flops(int kind, int iters, int workgroups) {
    return (double)workgroups * 4 * iters * 8 * 2.0 * 16 * 16 * (kind == 0 ? 32 : 128);
}
hipError_t launch_qproj_down(const QprojArgs& a, const Launch&) {
    if (a.ksplit < 1 || a.hidden % (64 * a.ksplit) || a.hidden / a.ksplit < kQprojRowsPerSplit)
        die("launch_qproj_down: ksplit", nullptr, 0);
    need("launch_qproj_down c_part", a.c_part, (size_t)a.ksplit * a.batch * a.rank * 4);
    need("launch_qproj_down sumsq", a.sumsq, (size_t)a.batch * (a.rank / 64) * 4);
    need("launch_qproj_down counters", a.counters, (size_t)((a.batch + 31) / 32) * (a.rank / 64) * 4);
    need("launch_qproj_down chat", a.chat, (size_t)a.batch * a.rank * 2);
    g_launches++;
    return hipSuccess;
}
hipError_t launch_qproj_up(const QprojArgs& a, const Launch&) {
    need("launch_qproj_up chat", a.chat, (size_t)a.batch * a.rank * 2);
    need("launch_qproj_up sumsq", a.sumsq, (size_t)a.batch * (a.rank / 64) * 4);
    g_launches++;
    return hipSuccess;
}
hipError_t launch_kv_proj(const KvAppendArgs& a, const Launch&) {
    if (a.ksplit < 1 || a.hidden % a.ksplit || (a.hidden / a.ksplit) % kKvRowsPerSplit)
        die("launch_kv_proj: ksplit", nullptr, 0);
    need("launch_kv_proj kv_part", a.kv_part, (size_t)2 * a.ksplit * a.batch * kHeadDim * 4);
    g_launches++;
    return hipSuccess;
}
hipError_t launch_kv_write(const KvAppendArgs& a, bool, bool paged, const Launch&) {
    if (paged != (a.page_table != nullptr)) die("launch_kv_write: paged flag", a.page_table, 0);
    need("launch_kv_write kv_part", a.kv_part, (size_t)2 * a.ksplit * a.batch * kHeadDim * 4);
    g_launches++;
    return hipSuccess;
}

}  // namespace mfa
