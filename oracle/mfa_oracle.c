/*
 * mfa_oracle.c -- plain fp64 CPU oracle for the decode step of Multi-Matrix
 * Factorization Attention (MFA).
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, obviously-correct
 * definition that the GPU library is checked against. Only the tests, the
 * smoke check and the benchmark's CPU-baseline leg may load it; the product
 * path never calls it. It shares no code with the GPU library.
 *
 * What it follows (all on the Step-3 summary page, "Step-3 is Large yet
 * Affordable: Model-system Co-design for Cost-effective Decoding", Key points):
 *   - hidden size 7168 per layer;
 *   - 64 query heads sharing ONE key head and ONE value head, each of dim 256
 *     (so every head attends to the same cached K/V rows: multi-query
 *     structure, "Fast Transformer Decoding: One Write-Head is All You Need",
 *     cited by title on the DeepSeek-V4 page's references);
 *   - queries pass through a 2048-wide low-rank bottleneck.
 * Readings where the pages are silent (each is listed in the design notes):
 *   - RMSNorm sits on the 2048-wide bottleneck, multiplies by gamma, eps given;
 *   - weights are row-major [in][out], so c = x . W;
 *   - scaled dot-product softmax attention ("Attention Is All You Need", cited
 *     by title): s_t = scale * <q, k_t>, w = softmax(s), o = sum_t w_t v_t,
 *     and lse = log sum_t exp(s_t); no mask, no positional rotation;
 *   - FP8 is OCP E4M3FN (bias 7, no infinities, NaN = S.1111.111); the stored
 *     value is decode(code) * per-tensor scale;
 *   - paged caches: page_table[b][t / page_size] names the page holding
 *     token t, at row t % page_size (PagedAttention, cited by title);
 *   - split-K (Flash-Decoding, cited by title on the DeepSeek-V4 page): chunks
 *     of `chunk` tokens from token 0, each reduced to (max, sum, normalised
 *     output), merged by the log-sum-exp identity;
 *   - the new token's K and V rows are x . W_k and x . W_v (hidden -> 256),
 *     rounded to float, divided by the tensor's scale for FP8, encoded by
 *     round-to-nearest-even (E4M3 saturating at +-448) and written at row L_b;
 *   - for the head-sharing comparison, grouped-query attention (GQA, cited by
 *     title on the DeepSeek-V4 page): G K/V heads, query head h reading head
 *     h / (H / G), caches [B][G][S][D] or pools [P][G][page][D].
 *
 * Every floating-point step runs in IEEE double. Inputs in bf16 / E4M3 are
 * decoded exactly (both formats are subsets of double).
 *
 * Parity pins (tests/test_oracle.py): softmax weights sum to 1, identical keys
 * give mean(V), one-token context returns that V row exactly, KV permutation
 * invariance, scale 0 gives mean(V), a dominant key returns its V row,
 * 50-digit decimal brute force on tiny inputs, numpy dgemm for the
 * projections, RMSNorm scale invariance and closed form, the 256-code E4M3
 * table against the OCP closed form and torch.float8_e4m3fn, paged equals
 * contiguous bit for bit, split equals unsplit; for the append: the encoders
 * against torch and against exact midpoints between neighbouring codes (ties
 * to even), saturation, the K/V projection against numpy dgemm and decimal
 * brute force, and the append touching exactly row L_b (paged and contiguous
 * agreeing); grouped attention against torch's grouped SDPA (enable_gqa),
 * as G independent single-head problems, paged equal to contiguous, and a
 * decimal brute force.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_BF16 = 0, OR_FP8_E4M3 = 1 };

/* bf16 -> double: the bf16 pattern is the top half of an IEEE binary32. */
double oracle_bf16_to_f64(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP E4M3FN code -> double, from the format's definition:
 * sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
 * exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN;
 * there are no infinities. */
double oracle_e4m3_to_f64(uint8_t c) {
    int sign = (c >> 7) & 1;
    int e = (c >> 3) & 0xF;
    int m = c & 0x7;
    double v;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

static double g_e4m3[256];
static int g_e4m3_ready = 0;

static void e4m3_table_init(void) {
    if (g_e4m3_ready)
        return;
    for (int c = 0; c < 256; c++)
        g_e4m3[c] = oracle_e4m3_to_f64((uint8_t)c);
    g_e4m3_ready = 1;
}

void oracle_e4m3_table(double* out256) {
    e4m3_table_init();
    memcpy(out256, g_e4m3, sizeof g_e4m3);
}

void oracle_decode_bf16(const uint16_t* in, double* out, int64_t n) {
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_bf16_to_f64(in[i]);
}

void oracle_decode_e4m3(const uint8_t* in, double* out, int64_t n) {
    e4m3_table_init();
    for (int64_t i = 0; i < n; i++)
        out[i] = g_e4m3[in[i]];
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ Q path */

/* c = x . W_qa  (x [B][hidden], W_qa [hidden][rank], row-major [in][out])
 * r_b = 1 / sqrt(mean_j c_bj^2 + eps)
 * chat = c * r_b * gamma
 * q = chat . W_qb  (W_qb [rank][nq]); q is [B][nq] with nq = heads * head_dim.
 * c_out (may be NULL) receives c; chat_out (may be NULL) receives chat. */
int oracle_qproj(int B, int hidden, int rank, int nq,
                 const uint16_t* x, const uint16_t* w_qa, const uint16_t* gamma,
                 const uint16_t* w_qb, double eps, double* c_out, double* chat_out,
                 double* q_out, int nthreads) {
    if (B < 0 || hidden <= 0 || rank <= 0 || nq <= 0)
        return -1;
    set_threads(nthreads);
    double* c = (double*)calloc((size_t)B * rank, sizeof(double));
    double* chat = (double*)calloc((size_t)B * rank, sizeof(double));
    if (!c || !chat) {
        free(c);
        free(chat);
        return -3;
    }
    /* step 1: down-projection, one output column at a time */
    #pragma omp parallel for schedule(static)
    for (int j = 0; j < rank; j++) {
        for (int b = 0; b < B; b++) {
            double acc = 0.0;
            for (int i = 0; i < hidden; i++)
                acc += oracle_bf16_to_f64(x[(size_t)b * hidden + i]) *
                       oracle_bf16_to_f64(w_qa[(size_t)i * rank + j]);
            c[(size_t)b * rank + j] = acc;
        }
    }
    /* step 2: RMSNorm over the bottleneck */
    for (int b = 0; b < B; b++) {
        double ss = 0.0;
        for (int j = 0; j < rank; j++)
            ss += c[(size_t)b * rank + j] * c[(size_t)b * rank + j];
        double r = 1.0 / sqrt(ss / (double)rank + eps);
        for (int j = 0; j < rank; j++)
            chat[(size_t)b * rank + j] = c[(size_t)b * rank + j] * r * oracle_bf16_to_f64(gamma[j]);
    }
    /* step 3: up-projection to 64 heads x 256 */
    #pragma omp parallel for schedule(static)
    for (int n = 0; n < nq; n++) {
        for (int b = 0; b < B; b++) {
            double acc = 0.0;
            for (int j = 0; j < rank; j++)
                acc += chat[(size_t)b * rank + j] * oracle_bf16_to_f64(w_qb[(size_t)j * nq + n]);
            q_out[(size_t)b * nq + n] = acc;
        }
    }
    if (c_out)
        memcpy(c_out, c, (size_t)B * rank * sizeof(double));
    if (chat_out)
        memcpy(chat_out, chat, (size_t)B * rank * sizeof(double));
    free(c);
    free(chat);
    return 0;
}

/* ------------------------------------------------------------ KV addressing */

typedef struct {
    int kv_dtype;              /* OR_BF16 or OR_FP8_E4M3 */
    const void* k;
    const void* v;
    double k_scale, v_scale;   /* applied to FP8 values only */
    const int32_t* page_table; /* NULL: contiguous */
    int pt_stride;
    int page_size;
    int64_t kv_stride;         /* contiguous: token slots per sequence */
    int D;
    int G;                     /* KV heads (1: one K and one V head shared by all query heads) */
    int g;                     /* the KV head this view reads */
} kv_view;

/* Row index (in units of D elements) of token t of sequence b in KV head
 * kv->g. Contiguous: K/V [B][G][kv_stride][D]; paged: pools
 * [P][G][page_size][D], page_table[b][t / page_size] naming the page. With
 * G = 1 these are [B][kv_stride][D] and [P][page_size][D]. */
static int64_t kv_row(const kv_view* kv, int b, int t) {
    if (kv->page_table) {
        int32_t page = kv->page_table[(size_t)b * kv->pt_stride + t / kv->page_size];
        return ((int64_t)page * kv->G + kv->g) * kv->page_size + t % kv->page_size;
    }
    return ((int64_t)b * kv->G + kv->g) * kv->kv_stride + t;
}

static double kv_value(const kv_view* kv, const void* base, double scale, int64_t row, int d) {
    size_t idx = (size_t)row * kv->D + d;
    if (kv->kv_dtype == OR_BF16)
        return oracle_bf16_to_f64(((const uint16_t*)base)[idx]);
    return g_e4m3[((const uint8_t*)base)[idx]] * scale;
}

/* ------------------------------------------------------------ attention */

/* Scores of one (b, h) against tokens [t0, t1): s[t - t0]. */
static void scores(const kv_view* kv, const double* qv, int b, int t0, int t1,
                   double softmax_scale, double* s) {
    for (int t = t0; t < t1; t++) {
        int64_t row = kv_row(kv, b, t);
        double dot = 0.0;
        for (int d = 0; d < kv->D; d++)
            dot += qv[d] * kv_value(kv, kv->k, kv->k_scale, row, d);
        s[t - t0] = softmax_scale * dot;
    }
}

/* Plain softmax attention over tokens [t0, t1) for one (b, h):
 * M = max s, w_t = exp(s_t - M) / sum_u exp(s_u - M), o = sum_t w_t v_t,
 * lse = M + log(sum_u exp(s_u - M)). Empty range: o = 0, lse = -inf. */
static void attend_range(const kv_view* kv, const double* qv, int b, int t0, int t1,
                         double softmax_scale, double* s, double* o, double* lse) {
    int D = kv->D;
    for (int d = 0; d < D; d++)
        o[d] = 0.0;
    if (t1 <= t0) {
        *lse = -INFINITY;
        return;
    }
    scores(kv, qv, b, t0, t1, softmax_scale, s);
    double M = -INFINITY;
    for (int t = 0; t < t1 - t0; t++)
        if (s[t] > M)
            M = s[t];
    double sum = 0.0;
    for (int t = 0; t < t1 - t0; t++)
        sum += exp(s[t] - M);
    for (int t = t0; t < t1; t++) {
        double w = exp(s[t - t0] - M) / sum;
        int64_t row = kv_row(kv, b, t);
        for (int d = 0; d < D; d++)
            o[d] += w * kv_value(kv, kv->v, kv->v_scale, row, d);
    }
    *lse = M + log(sum);
}

static int check_args(int B, int H, int D, const int32_t* seq_lens, int page_size,
                      const int32_t* page_table, int pt_stride, int64_t kv_stride) {
    if (B < 0 || H <= 0 || D <= 0 || !seq_lens)
        return -1;
    for (int b = 0; b < B; b++) {
        if (seq_lens[b] < 0)
            return -1;
        if (page_table) {
            if (page_size <= 0 || (int64_t)(seq_lens[b] + page_size - 1) / page_size > pt_stride)
                return -1;
        } else if (seq_lens[b] > kv_stride) {
            return -1;
        }
    }
    return 0;
}

/* q [B][H][D] fp64. Outputs o [B][H][D], lse [B][H] (lse may be NULL).
 * G KV heads (grouped-query attention, "GQA: Training Generalized
 * Multi-Query Transformer Models from Multi-Head Checkpoints", named on the
 * DeepSeek-V4 card's references): query head h reads KV head
 * h / (H / G), consecutive query heads sharing one; G = 1 is MFA's single
 * shared K/V head, G = H is multi-head attention. G must divide H.
 * chunk <= 0: one softmax over all L_b tokens.
 * chunk > 0: split-K. Each chunk [c*chunk, min(L_b, (c+1)*chunk)) yields
 * lse_c and the chunk-normalised output o_c; then
 * LSE = M + log sum_c exp(lse_c - M) with M = max_c lse_c and
 * o = sum_c exp(lse_c - LSE) * o_c. */
int oracle_attention_grouped(int B, int H, int G, int D, const double* q, int kv_dtype,
                             const void* k, const void* v, double k_scale, double v_scale,
                             const int32_t* seq_lens, const int32_t* page_table, int pt_stride,
                             int page_size, int64_t kv_stride, double softmax_scale, int chunk,
                             double* o, double* lse, int nthreads) {
    int rc = check_args(B, H, D, seq_lens, page_size, page_table, pt_stride, kv_stride);
    if (rc)
        return rc;
    if (G <= 0 || H % G != 0)
        return -1;
    if (kv_dtype != OR_BF16 && kv_dtype != OR_FP8_E4M3)
        return -2;
    e4m3_table_init();
    set_threads(nthreads);
    const kv_view kv0 = {kv_dtype, k, v, k_scale, v_scale, page_table, pt_stride, page_size,
                         kv_stride, D, G, 0};
    int maxL = 0;
    for (int b = 0; b < B; b++)
        if (seq_lens[b] > maxL)
            maxL = seq_lens[b];
    int failed = 0;
    #pragma omp parallel
    {
        double* s = (double*)malloc(((size_t)maxL + 1) * sizeof(double));
        if (!s) {
            #pragma omp atomic write
            failed = 1;
        }
        #pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < (int64_t)B * H; bh++) {
            if (failed)
                continue;
            int b = (int)(bh / H);
            kv_view kv = kv0;
            kv.g = (int)(bh % H) / (H / G);   /* the KV head of query head h */
            const double* qv = q + (size_t)bh * D;
            double* ov = o + (size_t)bh * D;
            double l_out;
            int L = seq_lens[b];
            if (chunk <= 0 || L == 0) {
                attend_range(&kv, qv, b, 0, L, softmax_scale, s, ov, &l_out);
            } else {
                int nc = (L + chunk - 1) / chunk;
                double* lcs = (double*)malloc((size_t)nc * sizeof(double));
                double* ocs = (double*)malloc((size_t)nc * D * sizeof(double));
                if (!lcs || !ocs) {
                    free(lcs);
                    free(ocs);
                    #pragma omp atomic write
                    failed = 1;
                    continue;
                }
                /* each chunk on its own: lse_c and the chunk-normalised o_c */
                for (int c = 0; c < nc; c++) {
                    int t0 = c * chunk, t1 = t0 + chunk < L ? t0 + chunk : L;
                    attend_range(&kv, qv, b, t0, t1, softmax_scale, s, ocs + (size_t)c * D, &lcs[c]);
                }
                /* log-sum-exp merge */
                double M = -INFINITY;
                for (int c = 0; c < nc; c++)
                    if (lcs[c] > M)
                        M = lcs[c];
                double sum = 0.0;
                for (int c = 0; c < nc; c++)
                    sum += exp(lcs[c] - M);
                double LSE = M + log(sum);
                for (int d = 0; d < D; d++)
                    ov[d] = 0.0;
                for (int c = 0; c < nc; c++) {
                    double w = exp(lcs[c] - LSE);
                    for (int d = 0; d < D; d++)
                        ov[d] += w * ocs[(size_t)c * D + d];
                }
                l_out = LSE;
                free(lcs);
                free(ocs);
            }
            if (lse)
                lse[bh] = l_out;
        }
        free(s);
    }
    return failed ? -3 : 0;
}

/* One K and one V head shared by all H query heads (MFA's attention). */
int oracle_attention(int B, int H, int D, const double* q, int kv_dtype,
                     const void* k, const void* v, double k_scale, double v_scale,
                     const int32_t* seq_lens, const int32_t* page_table, int pt_stride,
                     int page_size, int64_t kv_stride, double softmax_scale, int chunk,
                     double* o, double* lse, int nthreads) {
    return oracle_attention_grouped(B, H, 1, D, q, kv_dtype, k, v, k_scale, v_scale, seq_lens,
                                    page_table, pt_stride, page_size, kv_stride, softmax_scale,
                                    chunk, o, lse, nthreads);
}

/* ------------------------------------------------- FP8 attention arithmetic */
/*
 * Attention computed in FP8, the precision the Step-3 summary card's Key
 * points give for its decoding throughput (4K context, FP8; a BF16-attention
 * ablation is slower). The pages do not say how the query and the softmax
 * weights are quantised; the reading taken here:
 *
 *   1. each head's query q (bf16 values) is scaled by 2^e, the power of two
 *      that puts its largest |q_d| in [128, 256): e = 7 - floor(log2 max|q|),
 *      limited to [-100, 100] (e = 0 for an all-zero head); every q_d * 2^e
 *      is rounded (as a float) to E4M3 by round-to-nearest-even, giving q8;
 *   2. scores are exact dot products of q8 with the cached key codes, in
 *      base 2: s2_t = <q8, k_t> * softmax_scale * k_scale * log2(e) * 2^-e;
 *   3. the weights are taken against an integer reference r = ceil(max_t
 *      s2_t): P_t = 2^(s2_t - r) lies in (0, 1], and 4 P_t is rounded (as a
 *      float) to E4M3 by round-to-nearest-even, subnormal codes included;
 *      p8_t is that E4M3 value divided by 4;
 *   4. o = v_scale * sum_t p8_t v_t / S8 with S8 = sum_t p8_t (the weights
 *      applied to V sum to one), and lse = ln(2) * (r + log2 S8).
 *
 * Because r is an integer, E4M3's normal range makes p8 independent of which
 * integer reference is used (a power of two scales every code exactly), so
 * the result does not depend on how the context is cut into pieces, except
 * for weights whose 4 P falls below E4M3's smallest normal value (2^-6).
 * With E4M3 replaced by exact arithmetic (inputs whose q * 2^e and 4 P are
 * E4M3 values) this is plain softmax attention, oracle_attention.
 *
 * q is given as bf16 bits [B][H][D]; k and v are E4M3 codes, contiguous
 * [B][kv_stride][D] or paged [P][page_size][D]. Outputs o [B][H][D] and lse
 * [B][H] (NULL allowed); an empty sequence gives o = 0 and lse = -inf.
 */
uint8_t oracle_f32_to_e4m3(float x);   /* defined with the KV append below */

static double e4m3_round_f32(double x) {
    return g_e4m3[oracle_f32_to_e4m3((float)x)];
}

/* The exponent e of step 1 for a head whose largest |q_d| is amax. */
int oracle_fp8_q_exponent(double amax) {
    if (!(amax > 0.0))
        return 0;
    int x;
    (void)frexp(amax, &x);              /* amax = f * 2^x, f in [0.5, 1) */
    int e = 7 - (x - 1);                /* floor(log2 amax) = x - 1 */
    if (e > 100)
        e = 100;
    if (e < -100)
        e = -100;
    return e;
}

int oracle_attention_fp8mma(int B, int H, int D, const uint16_t* q, const uint8_t* k,
                            const uint8_t* v, double k_scale, double v_scale,
                            const int32_t* seq_lens, const int32_t* page_table, int pt_stride,
                            int page_size, int64_t kv_stride, double softmax_scale,
                            double* o, double* lse, int nthreads) {
    int rc = check_args(B, H, D, seq_lens, page_size, page_table, pt_stride, kv_stride);
    if (rc)
        return rc;
    e4m3_table_init();
    set_threads(nthreads);
    const kv_view kv = {OR_FP8_E4M3, k, v, 1.0, 1.0, page_table, pt_stride, page_size,
                        kv_stride, D, 1, 0};
    const double log2e = 1.0 / log(2.0);
    int maxL = 0;
    for (int b = 0; b < B; b++)
        if (seq_lens[b] > maxL)
            maxL = seq_lens[b];
    int failed = 0;
    #pragma omp parallel
    {
        double* s2 = (double*)malloc(((size_t)maxL + 1) * sizeof(double));
        double* q8 = (double*)malloc((size_t)D * sizeof(double));
        if (!s2 || !q8) {
            #pragma omp atomic write
            failed = 1;
        }
        #pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < (int64_t)B * H; bh++) {
            if (failed)
                continue;
            int b = (int)(bh / H);
            int L = seq_lens[b];
            double* ov = o + (size_t)bh * D;
            for (int d = 0; d < D; d++)
                ov[d] = 0.0;
            if (L == 0) {
                if (lse)
                    lse[bh] = -INFINITY;
                continue;
            }
            /* step 1: per-head power-of-two scale, E4M3 query */
            const uint16_t* qh = q + (size_t)bh * D;
            double amax = 0.0;
            for (int d = 0; d < D; d++) {
                double a = fabs(oracle_bf16_to_f64(qh[d]));
                if (a > amax)
                    amax = a;
            }
            int e = oracle_fp8_q_exponent(amax);
            for (int d = 0; d < D; d++)
                q8[d] = e4m3_round_f32(ldexp(oracle_bf16_to_f64(qh[d]), e));
            /* step 2: exact scores, base 2 */
            double sc = softmax_scale * k_scale * log2e * ldexp(1.0, -e);
            for (int t = 0; t < L; t++) {
                int64_t row = kv_row(&kv, b, t);
                double dot = 0.0;
                for (int d = 0; d < D; d++)
                    dot += q8[d] * g_e4m3[k[(size_t)row * D + d]];
                s2[t] = dot * sc;
            }
            /* step 3: weights against the integer reference, E4M3 of 4 P */
            double M = -INFINITY;
            for (int t = 0; t < L; t++)
                if (s2[t] > M)
                    M = s2[t];
            double r = ceil(M);
            double S8 = 0.0;
            for (int t = 0; t < L; t++) {
                s2[t] = e4m3_round_f32(4.0 * exp2(s2[t] - r)) / 4.0;   /* p8_t, in place */
                S8 += s2[t];
            }
            /* step 4: weighted V, normalised by the sum of the applied weights */
            for (int t = 0; t < L; t++) {
                int64_t row = kv_row(&kv, b, t);
                for (int d = 0; d < D; d++)
                    ov[d] += s2[t] * g_e4m3[v[(size_t)row * D + d]];
            }
            for (int d = 0; d < D; d++)
                ov[d] = ov[d] * v_scale / S8;
            if (lse)
                lse[bh] = log(2.0) * r + log(S8);
        }
        free(s2);
        free(q8);
    }
    return failed ? -3 : 0;
}

/* Softmax weights of one (b, h) over all L_b tokens, in token order:
 * w[t] = exp(s_t - M) / sum_u exp(s_u - M). For the sum-to-one pin. */
int oracle_weights(int H, int D, const double* q, int b, int h, int kv_dtype,
                   const void* k, double k_scale, const int32_t* seq_lens,
                   const int32_t* page_table, int pt_stride, int page_size, int64_t kv_stride,
                   double softmax_scale, double* w) {
    (void)H;
    e4m3_table_init();
    kv_view kv = {kv_dtype, k, k, k_scale, 1.0, page_table, pt_stride, page_size, kv_stride, D, 1, 0};
    int L = seq_lens[b];
    if (L <= 0)
        return 0;
    const double* qv = q + ((size_t)b * H + h) * D;
    scores(&kv, qv, b, 0, L, softmax_scale, w);
    double M = -INFINITY;
    for (int t = 0; t < L; t++)
        if (w[t] > M)
            M = w[t];
    double sum = 0.0;
    for (int t = 0; t < L; t++)
        sum += exp(w[t] - M);
    for (int t = 0; t < L; t++)
        w[t] = exp(w[t] - M) / sum;
    return L;
}

/* Copy the logical K and V rows t < L_b of sequence b, in token order, into
 * contiguous byte buffers (elem_bytes = 2 for bf16, 1 for FP8). Used to check
 * the GPU's page-table address generation byte for byte. */
int oracle_gather_kv(int b, int D, int elem_bytes, const void* k, const void* v,
                     const int32_t* seq_lens, const int32_t* page_table, int pt_stride,
                     int page_size, int64_t kv_stride, void* k_dst, void* v_dst) {
    kv_view kv = {0, k, v, 1.0, 1.0, page_table, pt_stride, page_size, kv_stride, D, 1, 0};
    int L = seq_lens[b];
    size_t rb = (size_t)D * elem_bytes;
    for (int t = 0; t < L; t++) {
        int64_t row = kv_row(&kv, b, t);
        memcpy((char*)k_dst + (size_t)t * rb, (const char*)k + (size_t)row * rb, rb);
        memcpy((char*)v_dst + (size_t)t * rb, (const char*)v + (size_t)row * rb, rb);
    }
    return L;
}

/* ---------------------------------------------------------------- KV append */
/*
 * The step before attention in a decode layer: the new token's key and value
 * from its hidden state, k = x . W_k and v = x . W_v (hidden -> D each, one
 * shared K head and one shared V head: Step-3 summary card, Key points),
 * written at row L_b of sequence b (paged: page page_table[b][L_b / 64], row
 * L_b % 64, as in PagedAttention). The cache stores bf16, or E4M3 of the
 * value divided by the tensor's scale.
 *
 * The rounding to the cache format is an integer decision taken from a
 * floating-point value: it is taken here from the value rounded to float
 * (and divided by the scale in float), the precision the GPU computes in.
 */

/* bf16 bits of a float by round-to-nearest-even; NaN stays a quiet NaN. */
uint16_t oracle_f32_to_bf16(float x) {
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

/* OCP E4M3FN code of a float by round-to-nearest-even. Finite values beyond
 * the largest code (448) saturate to +-448 (the format has no infinities);
 * NaN gives 0x7f with the sign. Written from the format's definition: value
 * = 2^(e-7) * (1 + m/8) for exponent field e >= 1, 2^-6 * m/8 for e = 0. */
uint8_t oracle_f32_to_e4m3(float x) {
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs((double)x);
    if (isnan(x))
        return sign | 0x7f;
    if (a >= 448.0)
        return sign | 0x7e;
    if (a < 0.015625) {                 /* below 2^-6: multiples of 2^-9 */
        double u = a * 512.0;           /* exact */
        double r = nearbyint(u);        /* ties to even (default rounding mode) */
        return sign | (uint8_t)r;       /* 8 is the smallest normal, code 0x08 */
    }
    int e2;
    double f = frexp(a, &e2);           /* a = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;                     /* a = (2f) * 2^e, 2f in [1, 2) */
    double m = (2.0 * f - 1.0) * 8.0;   /* exact: a float has 24 bits */
    double q = nearbyint(m);
    if (q == 8.0) {
        q = 0.0;
        e += 1;
    }
    int code = ((e + 7) << 3) | (int)q;
    if (code > 0x7e)
        code = 0x7e;
    return sign | (uint8_t)code;
}

void oracle_encode_bf16(const float* in, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_f32_to_bf16(in[i]);
}

void oracle_encode_e4m3(const float* in, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_f32_to_e4m3(in[i]);
}

/* k_out, v_out [B][D] = x [B][hidden] . W_k, W_v [hidden][D] (bf16 inputs),
 * summed in fp64. */
int oracle_kv_project(int B, int hidden, int D, const uint16_t* x, const uint16_t* w_k,
                      const uint16_t* w_v, double* k_out, double* v_out, int nthreads) {
    if (B < 0 || hidden <= 0 || D <= 0)
        return -1;
    set_threads(nthreads);
    #pragma omp parallel for schedule(static)
    for (int j = 0; j < D; j++) {
        for (int b = 0; b < B; b++) {
            double ak = 0.0, av = 0.0;
            for (int i = 0; i < hidden; i++) {
                double xi = oracle_bf16_to_f64(x[(size_t)b * hidden + i]);
                ak += xi * oracle_bf16_to_f64(w_k[(size_t)i * D + j]);
                av += xi * oracle_bf16_to_f64(w_v[(size_t)i * D + j]);
            }
            k_out[(size_t)b * D + j] = ak;
            v_out[(size_t)b * D + j] = av;
        }
    }
    return 0;
}

/* Write the new rows: for each sequence b with L_b inside the cache's
 * capacity (contiguous: L_b < kv_stride; paged: its page-table slot exists
 * and names a page in [0, num_pages)), row L_b of K and V receives the
 * encoded values. Other rows are not touched. Returns the rows written. */
int oracle_kv_append(int B, int D, int kv_dtype, const double* k_new, const double* v_new,
                     double k_scale, double v_scale, void* k, void* v, const int32_t* seq_lens,
                     const int32_t* page_table, int pt_stride, int page_size, int64_t kv_stride,
                     int num_pages) {
    int written = 0;
    for (int b = 0; b < B; b++) {
        int t = seq_lens[b];
        int64_t row;
        if (t < 0)
            continue;
        if (page_table) {
            if (t / page_size >= pt_stride)
                continue;
            int page = page_table[(size_t)b * pt_stride + t / page_size];
            if (page < 0 || page >= num_pages)
                continue;
            row = (int64_t)page * page_size + t % page_size;
        } else {
            if (t >= kv_stride)
                continue;
            row = (int64_t)b * kv_stride + t;
        }
        for (int d = 0; d < D; d++) {
            float kf = (float)k_new[(size_t)b * D + d];
            float vf = (float)v_new[(size_t)b * D + d];
            if (kv_dtype == OR_FP8_E4M3) {
                ((uint8_t*)k)[row * D + d] = oracle_f32_to_e4m3(kf / (float)k_scale);
                ((uint8_t*)v)[row * D + d] = oracle_f32_to_e4m3(vf / (float)v_scale);
            } else {
                ((uint16_t*)k)[row * D + d] = oracle_f32_to_bf16(kf);
                ((uint16_t*)v)[row * D + d] = oracle_f32_to_bf16(vf);
            }
        }
        written++;
    }
    return written;
}
