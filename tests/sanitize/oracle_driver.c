/*
 * oracle_driver.c -- calls every function the oracle exports on small
 * ragged, paged, split and grouped cases, with every buffer allocated at
 * exactly the size the function's documented layout needs, so that a build
 * with AddressSanitizer / UndefinedBehaviorSanitizer sees any access outside
 * them. Also checks a few identities the oracle must satisfy on these cases
 * (paged equals contiguous bit for bit, split equals unsplit to rounding,
 * empty sequences give o = 0 and lse = -inf). Exits 0 and prints
 * "oracle_driver: ok" when all hold.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* the oracle's exported functions (oracle/mfa_oracle.c) */
double oracle_bf16_to_f64(uint16_t b);
double oracle_e4m3_to_f64(uint8_t c);
void oracle_e4m3_table(double* out256);
void oracle_decode_bf16(const uint16_t* in, double* out, int64_t n);
void oracle_decode_e4m3(const uint8_t* in, double* out, int64_t n);
int oracle_max_threads(void);
int oracle_qproj(int B, int hidden, int rank, int nq, const uint16_t* x, const uint16_t* w_qa,
                 const uint16_t* gamma, const uint16_t* w_qb, double eps, double* c_out,
                 double* chat_out, double* q_out, int nthreads);
int oracle_attention_grouped(int B, int H, int G, int D, const double* q, int kv_dtype,
                             const void* k, const void* v, double k_scale, double v_scale,
                             const int32_t* seq_lens, const int32_t* page_table, int pt_stride,
                             int page_size, int64_t kv_stride, double softmax_scale, int chunk,
                             double* o, double* lse, int nthreads);
int oracle_attention(int B, int H, int D, const double* q, int kv_dtype, const void* k,
                     const void* v, double k_scale, double v_scale, const int32_t* seq_lens,
                     const int32_t* page_table, int pt_stride, int page_size, int64_t kv_stride,
                     double softmax_scale, int chunk, double* o, double* lse, int nthreads);
int oracle_fp8_q_exponent(double amax);
int oracle_attention_fp8mma(int B, int H, int D, const uint16_t* q, const uint8_t* k,
                            const uint8_t* v, double k_scale, double v_scale,
                            const int32_t* seq_lens, const int32_t* page_table, int pt_stride,
                            int page_size, int64_t kv_stride, double softmax_scale, double* o,
                            double* lse, int nthreads);
int oracle_weights(int H, int D, const double* q, int b, int h, int kv_dtype, const void* k,
                   double k_scale, const int32_t* seq_lens, const int32_t* page_table,
                   int pt_stride, int page_size, int64_t kv_stride, double softmax_scale,
                   double* w);
int oracle_gather_kv(int b, int D, int elem_bytes, const void* k, const void* v,
                     const int32_t* seq_lens, const int32_t* page_table, int pt_stride,
                     int page_size, int64_t kv_stride, void* k_dst, void* v_dst);
uint16_t oracle_f32_to_bf16(float x);
uint8_t oracle_f32_to_e4m3(float x);
void oracle_encode_bf16(const float* in, uint16_t* out, int64_t n);
void oracle_encode_e4m3(const float* in, uint8_t* out, int64_t n);
int oracle_kv_project(int B, int hidden, int D, const uint16_t* x, const uint16_t* w_k,
                      const uint16_t* w_v, double* k_out, double* v_out, int nthreads);
int oracle_kv_append(int B, int D, int kv_dtype, const double* k_new, const double* v_new,
                     double k_scale, double v_scale, void* k, void* v, const int32_t* seq_lens,
                     const int32_t* page_table, int pt_stride, int page_size, int64_t kv_stride,
                     int num_pages);

static int failures = 0;
#define CHECK(c, ...)                                                      \
    do {                                                                   \
        if (!(c)) {                                                        \
            fprintf(stderr, "%s:%d: %s: ", __FILE__, __LINE__, #c);        \
            fprintf(stderr, __VA_ARGS__);                                  \
            fprintf(stderr, "\n");                                         \
            failures++;                                                    \
        }                                                                  \
    } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double urand(void) { /* xorshift64*, uniform in [-1, 1) */
    rng ^= rng >> 12;
    rng ^= rng << 25;
    rng ^= rng >> 27;
    return (double)((rng * 2685821657736338717ull) >> 11) / 4503599627370496.0 - 1.0;
}
static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}
static uint16_t* bf16_buf(size_t n, double amp) {
    uint16_t* p = (uint16_t*)xmalloc(n * 2);
    for (size_t i = 0; i < n; i++)
        p[i] = oracle_f32_to_bf16((float)(amp * urand()));
    return p;
}
static uint8_t* e4m3_buf(size_t n, double amp) {
    uint8_t* p = (uint8_t*)xmalloc(n);
    for (size_t i = 0; i < n; i++)
        p[i] = oracle_f32_to_e4m3((float)(amp * urand()));
    return p;
}

/* one attention configuration: contiguous and paged copies of the same rows */
static void attention_case(int H, int G, int D, int kv_dtype, const int32_t* lens, int B) {
    const int page = 16;
    int maxL = 0, pages = 0;
    for (int b = 0; b < B; b++) {
        if (lens[b] > maxL)
            maxL = lens[b];
        pages += (lens[b] + page - 1) / page;
    }
    const int pt_stride = (maxL + page - 1) / page > 0 ? (maxL + page - 1) / page : 1;
    const int64_t stride = maxL;
    const size_t eb = kv_dtype ? 1 : 2;
    const size_t rowb = (size_t)D * eb;
    /* contiguous [B][G][stride][D], paged pool [pages][G][page][D] */
    size_t nc = (size_t)B * G * stride, np = (size_t)pages * G * page;
    char* kc = (char*)xmalloc(nc * rowb);
    char* vc = (char*)xmalloc(nc * rowb);
    char* kp = (char*)xmalloc(np * rowb);
    char* vp = (char*)xmalloc(np * rowb);
    memset(kp, 0, np * rowb);
    memset(vp, 0, np * rowb);
    for (size_t i = 0; i < nc * D; i++) {
        if (kv_dtype) {
            ((uint8_t*)kc)[i] = oracle_f32_to_e4m3((float)(4.0 * urand()));
            ((uint8_t*)vc)[i] = oracle_f32_to_e4m3((float)(4.0 * urand()));
        } else {
            ((uint16_t*)kc)[i] = oracle_f32_to_bf16((float)urand());
            ((uint16_t*)vc)[i] = oracle_f32_to_bf16((float)urand());
        }
    }
    int32_t* pt = (int32_t*)xmalloc((size_t)B * pt_stride * sizeof(int32_t));
    int next = 0;
    for (int b = 0; b < B; b++)
        for (int i = 0; i < pt_stride; i++) {
            if (i * page < lens[b]) {
                int pg = pages - 1 - next++; /* pages in reverse order */
                pt[(size_t)b * pt_stride + i] = pg;
                for (int g = 0; g < G; g++)
                    for (int r = 0; r < page && i * page + r < lens[b]; r++) {
                        size_t src = ((size_t)b * G + g) * stride + i * page + r;
                        size_t dst = ((size_t)pg * G + g) * page + r;
                        memcpy(kp + dst * rowb, kc + src * rowb, rowb);
                        memcpy(vp + dst * rowb, vc + src * rowb, rowb);
                    }
            } else {
                pt[(size_t)b * pt_stride + i] = -1; /* never read */
            }
        }
    double* q = (double*)xmalloc((size_t)B * H * D * sizeof(double));
    for (size_t i = 0; i < (size_t)B * H * D; i++)
        q[i] = urand();
    size_t no = (size_t)B * H * D;
    double* o1 = (double*)xmalloc(no * sizeof(double));
    double* o2 = (double*)xmalloc(no * sizeof(double));
    double* o3 = (double*)xmalloc(no * sizeof(double));
    double* l1 = (double*)xmalloc((size_t)B * H * sizeof(double));
    double* l2 = (double*)xmalloc((size_t)B * H * sizeof(double));
    double* l3 = (double*)xmalloc((size_t)B * H * sizeof(double));
    const double ks = 0.3, vs = 0.7, sc = 1.0 / sqrt((double)D);
    int rc = oracle_attention_grouped(B, H, G, D, q, kv_dtype, kc, vc, ks, vs, lens, NULL, 0, 0,
                                      stride, sc, 0, o1, l1, 1);
    CHECK(rc == 0, "contiguous rc %d", rc);
    rc = oracle_attention_grouped(B, H, G, D, q, kv_dtype, kp, vp, ks, vs, lens, pt, pt_stride,
                                  page, 0, sc, 0, o2, l2, 1);
    CHECK(rc == 0, "paged rc %d", rc);
    CHECK(memcmp(o1, o2, no * sizeof(double)) == 0, "paged output differs (G %d)", G);
    for (int chunk = 16; chunk <= 64; chunk *= 2) {
        rc = oracle_attention_grouped(B, H, G, D, q, kv_dtype, kp, vp, ks, vs, lens, pt, pt_stride,
                                      page, 0, sc, chunk, o3, l3, 1);
        CHECK(rc == 0, "split rc %d", rc);
        for (size_t i = 0; i < no; i++)
            CHECK(fabs(o3[i] - o1[i]) <= 1e-12 * (1.0 + fabs(o1[i])), "split %d differs at %zu", chunk, i);
    }
    for (int b = 0; b < B; b++)
        for (int h = 0; h < H; h++) {
            if (lens[b] == 0) {
                CHECK(isinf(l1[b * H + h]) && l1[b * H + h] < 0, "empty lse");
                for (int d = 0; d < D; d++)
                    CHECK(o1[((size_t)b * H + h) * D + d] == 0.0, "empty output");
            } else {
                CHECK(isfinite(l1[b * H + h]), "lse finite");
            }
        }
    if (G == 1) {
        rc = oracle_attention(B, H, D, q, kv_dtype, kc, vc, ks, vs, lens, NULL, 0, 0, stride, sc,
                              0, o3, NULL, 1);
        CHECK(rc == 0 && memcmp(o1, o3, no * sizeof(double)) == 0, "G=1 wrapper");
        double* w = (double*)xmalloc((size_t)(maxL > 0 ? maxL : 1) * sizeof(double));
        for (int b = 0; b < B; b++) {
            int n = oracle_weights(H, D, q, b, H - 1, kv_dtype, kp, ks, lens, pt, pt_stride, page,
                                   0, sc, w);
            double s = 0.0;
            for (int t = 0; t < n; t++)
                s += w[t];
            CHECK(n == lens[b] && (n == 0 || fabs(s - 1.0) < 1e-12), "weights of %d", b);
        }
        free(w);
        char* kd = (char*)xmalloc((size_t)(maxL > 0 ? maxL : 1) * rowb);
        char* vd = (char*)xmalloc((size_t)(maxL > 0 ? maxL : 1) * rowb);
        for (int b = 0; b < B; b++) {
            int n = oracle_gather_kv(b, D, (int)eb, kp, vp, lens, pt, pt_stride, page, 0, kd, vd);
            CHECK(n == lens[b], "gather length");
            CHECK(n == 0 || memcmp(kd, kc + (size_t)b * stride * rowb, (size_t)n * rowb) == 0, "gather K");
            CHECK(n == 0 || memcmp(vd, vc + (size_t)b * stride * rowb, (size_t)n * rowb) == 0, "gather V");
        }
        free(kd);
        free(vd);
        if (kv_dtype) {
            uint16_t* qb = bf16_buf((size_t)B * H * D, 3.0);
            rc = oracle_attention_fp8mma(B, H, D, qb, (uint8_t*)kc, (uint8_t*)vc, ks, vs, lens, NULL,
                                         0, 0, stride, sc, o1, l1, 1);
            CHECK(rc == 0, "fp8mma contiguous");
            rc = oracle_attention_fp8mma(B, H, D, qb, (uint8_t*)kp, (uint8_t*)vp, ks, vs, lens, pt,
                                         pt_stride, page, 0, sc, o2, NULL, 1);
            CHECK(rc == 0 && memcmp(o1, o2, no * sizeof(double)) == 0, "fp8mma paged");
            free(qb);
        }
    }
    /* argument rejections */
    int32_t bad_len = -1;
    CHECK(oracle_attention(1, H, D, q, kv_dtype, kc, vc, ks, vs, &bad_len, NULL, 0, 0, stride, sc,
                           0, o3, l3, 1) != 0, "negative length accepted");
    if (B > 0) {
        int32_t* long_lens = (int32_t*)xmalloc((size_t)B * sizeof(int32_t));
        for (int b = 0; b < B; b++)
            long_lens[b] = (int32_t)stride + 1;
        CHECK(oracle_attention(B, H, D, q, kv_dtype, kc, vc, ks, vs, long_lens, NULL, 0, 0, stride,
                               sc, 0, o3, l3, 1) != 0, "length beyond kv_stride accepted");
        for (int b = 0; b < B; b++)
            long_lens[b] = pt_stride * page + 1;
        CHECK(oracle_attention(B, H, D, q, kv_dtype, kp, vp, ks, vs, long_lens, pt, pt_stride, page,
                               0, sc, 0, o3, l3, 1) != 0, "length beyond the page table accepted");
        free(long_lens);
    }
    CHECK(oracle_attention_grouped(B, H, 3, D, q, kv_dtype, kc, vc, ks, vs, lens, NULL, 0, 0,
                                   stride, sc, 0, o3, l3, 1) != 0 || H % 3 == 0, "G not dividing H");
    free(kc), free(vc), free(kp), free(vp), free(pt), free(q);
    free(o1), free(o2), free(o3), free(l1), free(l2), free(l3);
}

static void projection_cases(void) {
    const int B = 3, hidden = 64, rank = 32, nq = 48, D = 16;
    uint16_t* x = bf16_buf((size_t)B * hidden, 1.0);
    uint16_t* wa = bf16_buf((size_t)hidden * rank, 0.2);
    uint16_t* g = bf16_buf((size_t)rank, 1.0);
    uint16_t* wb = bf16_buf((size_t)rank * nq, 0.2);
    double* c = (double*)xmalloc((size_t)B * rank * sizeof(double));
    double* ch = (double*)xmalloc((size_t)B * rank * sizeof(double));
    double* q = (double*)xmalloc((size_t)B * nq * sizeof(double));
    CHECK(oracle_qproj(B, hidden, rank, nq, x, wa, g, wb, 1e-6, c, ch, q, 1) == 0, "qproj");
    CHECK(oracle_qproj(B, hidden, rank, nq, x, wa, g, wb, 1e-6, NULL, NULL, q, 1) == 0, "qproj null outs");
    CHECK(oracle_qproj(0, hidden, rank, nq, x, wa, g, wb, 1e-6, NULL, NULL, q, 1) == 0, "qproj B = 0");
    CHECK(oracle_qproj(B, 0, rank, nq, x, wa, g, wb, 1e-6, NULL, NULL, q, 1) != 0, "qproj hidden 0");
    uint16_t* wk = bf16_buf((size_t)hidden * D, 0.2);
    uint16_t* wv = bf16_buf((size_t)hidden * D, 0.2);
    double* kn = (double*)xmalloc((size_t)B * D * sizeof(double));
    double* vn = (double*)xmalloc((size_t)B * D * sizeof(double));
    CHECK(oracle_kv_project(B, hidden, D, x, wk, wv, kn, vn, 1) == 0, "kv_project");
    /* append into a contiguous cache of 4 slots and a paged pool of 3 pages of 2 */
    for (int dt = 0; dt < 2; dt++) {
        const size_t eb = dt ? 1 : 2;
        int32_t lens[3] = {0, 3, 4}; /* the last is beyond the contiguous capacity */
        char* k = (char*)xmalloc((size_t)B * 4 * D * eb);
        char* v = (char*)xmalloc((size_t)B * 4 * D * eb);
        memset(k, 0, (size_t)B * 4 * D * eb);
        memset(v, 0, (size_t)B * 4 * D * eb);
        int n = oracle_kv_append(B, D, dt, kn, vn, 0.5, 0.25, k, v, lens, NULL, 0, 0, 4, 0);
        CHECK(n == 2, "contiguous append wrote %d", n);
        int32_t pt[3 * 2] = {0, 1, 2, -1, 2, 7}; /* seq 2's row 4 -> page 7, outside the pool */
        char* kp = (char*)xmalloc((size_t)3 * 2 * D * eb);
        char* vp = (char*)xmalloc((size_t)3 * 2 * D * eb);
        int32_t plens[3] = {1, 2, 3};
        n = oracle_kv_append(B, D, dt, kn, vn, 0.5, 0.25, kp, vp, plens, pt, 2, 2, 0, 3);
        CHECK(n == 1, "paged append wrote %d (seq 1: page -1, seq 2: page 7)", n);
        free(k), free(v), free(kp), free(vp);
    }
    free(x), free(wa), free(g), free(wb), free(c), free(ch), free(q);
    free(wk), free(wv), free(kn), free(vn);
}

static void codec_cases(void) {
    double t[256];
    oracle_e4m3_table(t);
    for (int c = 0; c < 256; c++) {
        double d = oracle_e4m3_to_f64((uint8_t)c);
        CHECK((isnan(d) && isnan(t[c])) || d == t[c], "table %d", c);
        if (!isnan(d))
            CHECK(oracle_f32_to_e4m3((float)d) == (uint8_t)c || d == 0.0, "round trip %d", c);
    }
    const float specials[] = {0.f, -0.f, 1e-30f, -1e-30f, 448.f, 449.f, 1e30f, -1e30f,
                              INFINITY, -INFINITY, NAN, 3.4e38f, 1.17e-38f};
    const int ns = (int)(sizeof specials / sizeof specials[0]);
    uint8_t e8[sizeof specials / sizeof specials[0]];
    uint16_t e16[sizeof specials / sizeof specials[0]];
    oracle_encode_e4m3(specials, e8, ns);
    oracle_encode_bf16(specials, e16, ns);
    double d8[sizeof specials / sizeof specials[0]], d16[sizeof specials / sizeof specials[0]];
    oracle_decode_e4m3(e8, d8, ns);
    oracle_decode_bf16(e16, d16, ns);
    CHECK(d8[5] == 448.0 && d8[6] == 448.0 && d8[7] == -448.0, "E4M3 saturates");
    CHECK(isnan(d16[10]) && isinf(d16[8]), "bf16 keeps NaN and inf");
    const double amaxes[] = {0.0, -1.0, 5e-324, 1e-300, 1.0, 128.0, 255.9, 256.0, 1e300, NAN};
    for (int i = 0; i < (int)(sizeof amaxes / sizeof amaxes[0]); i++) {
        int e = oracle_fp8_q_exponent(amaxes[i]);
        CHECK(e >= -100 && e <= 100, "exponent %d", e);
        if (amaxes[i] > 1e-20 && amaxes[i] < 1e20) {
            double s = ldexp(amaxes[i], e);
            CHECK(s >= 128.0 && s < 256.0, "scaled amax %g", s);
        }
    }
    CHECK(oracle_max_threads() >= 1, "threads");
}

int main(void) {
    codec_cases();
    projection_cases();
    const int32_t lens_a[4] = {0, 1, 37, 70};
    const int32_t lens_b[1] = {16};
    for (int dt = 0; dt < 2; dt++) {
        attention_case(4, 1, 16, dt, lens_a, 4);
        attention_case(4, 2, 16, dt, lens_a, 4);
        attention_case(4, 4, 8, dt, lens_a, 4);
        attention_case(2, 1, 32, dt, lens_b, 1);
    }
    attention_case(4, 1, 16, 1, lens_a, 0); /* an empty batch */
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle_driver: ok\n");
    return 0;
}
