/*
 * ORACLE -- test infrastructure only.
 *
 * A plain, slow, obviously correct CPU implementation of the indexer -> Top-K ->
 * sparse MLA attention path, in double precision. Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg load it; the product path never does.
 * It shares no code, header or table with the HIP library.
 *
 * It follows the unfused decode step that the page "Day 0 Inference Adaptation
 * and Performance Optimization for Hybrid Sparse Attention LLMs" lays out in its
 * section "Operator Fusion and Multi-Stream Scheduling": score every historical
 * position against the index cache, combine the heads with their weights, take
 * the Top-K positions, gather those rows of the main KV cache through the paging,
 * and run softmax attention over them. Fusion (same page; also "Rapid Adaptation
 * and Inference Optimization", section IV) moves intermediates out of memory but
 * does not change what is computed, so this unfused form is the definition.
 *
 * Readings fixed here (the pages leave them open):
 *  - score[j,s] = sigma_s * sum_h w[j,h] * max(0, q[j,h,:] . k_s), with sigma_s the
 *    per-token fp32 scale of an fp8 index cache and 1 for a bf16 one; q.k uses the
 *    exact values of the stored bf16 / e4m3fn elements ("low-precision cache
 *    de-quantized to higher precision", "Rapid Adaptation ...", section V).
 *  - query j at position t_j sees positions 0..t_j that are also < n_b.
 *  - Top-K orders by (score descending, position ascending), keeps the first
 *    min(K, row length), and lists them by ascending position, -1 padded.
 *  - the latent row is 576 wide; keys use all 576 columns, values the first 512.
 *  - an empty selection gives a zero output and lse = -inf.
 *
 * Every function returns 0 on success and a negative value on a bad argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define SIA_ORACLE_PAGE 64

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double oracle_bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP 8-bit float E4M3 ("FN": no infinities, only S.1111.111 is NaN).
 * Normal: (-1)^s * 2^(e-7) * (1 + m/8); subnormal (e = 0): (-1)^s * 2^-6 * m/8. */
double oracle_e4m3fn_value(uint8_t code) {
    int s = code >> 7, e = (code >> 3) & 0xF, m = code & 0x7;
    double v;
    if (e == 0xF && m == 0x7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

int oracle_decode_bf16(const uint16_t *bits, double *out, int64_t n) {
    if (!bits || !out || n < 0) return -1;
    for (int64_t i = 0; i < n; i++) out[i] = oracle_bf16_value(bits[i]);
    return 0;
}

int oracle_decode_e4m3fn(const uint8_t *codes, double *out, int64_t n) {
    if (!codes || !out || n < 0) return -1;
    for (int64_t i = 0; i < n; i++) out[i] = oracle_e4m3fn_value(codes[i]);
    return 0;
}

/* Physical row of logical position s of sequence b, or -1 if unmapped. */
static int64_t phys_row(const int32_t *page_table, int32_t max_pages, int32_t b, int64_t s) {
    int64_t p = s / SIA_ORACLE_PAGE;
    if (p >= max_pages) return -1;
    int32_t page = page_table[(int64_t)b * max_pages + p];
    if (page < 0) return -1;
    return (int64_t)page * SIA_ORACLE_PAGE + (s % SIA_ORACLE_PAGE);
}

/* Visible row length of query j: positions 0..t_j that are < n_b. */
static int64_t row_length(int32_t t, int32_t n_b) {
    int64_t r = (int64_t)t + 1;
    if (r > n_b) r = n_b;
    return r < 0 ? 0 : r;
}

/*
 * Steps 1-2 of the unfused decode step: relevance per head, then the
 * head-weighted sum.
 *   k_dtype: 0 = bf16 rows (uint16 bits), 1 = e4m3fn rows (uint8 codes) with
 *            k_scale[num_pages*64] per-token scales.
 *   scores[j*ld + s] for s < row_len[j]; -inf for s in [row_len[j], ld).
 */
int oracle_indexer_scores(int32_t num_q, const int32_t *q_seq, const int32_t *q_pos,
                          int32_t batch, const int32_t *seq_lens, const int32_t *page_table,
                          int32_t max_pages, int64_t num_pages, const void *k_pool,
                          int32_t k_dtype, const float *k_scale, int32_t dim,
                          const uint16_t *q_idx, const float *w, int32_t heads,
                          double *scores, int64_t ld, int32_t *row_len) {
    if (num_q < 0 || !q_seq || !q_pos || !seq_lens || !page_table || !k_pool || !q_idx ||
        !w || !scores || !row_len || dim <= 0 || heads <= 0 || batch <= 0)
        return -1;
    if (k_dtype != 0 && k_dtype != 1) return -1;
    if (k_dtype == 1 && !k_scale) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int32_t j = 0; j < num_q; j++) {
        int32_t b = q_seq[j];
        double *row = scores + (int64_t)j * ld;
        for (int64_t s = 0; s < ld; s++) row[s] = -INFINITY;
        row_len[j] = 0;
        if (b < 0 || b >= batch) { bad = 1; continue; }
        int64_t n = row_length(q_pos[j], seq_lens[b]);
        if (n > ld) { bad = 1; continue; }
        row_len[j] = (int32_t)n;
        double *qd = (double *)malloc(sizeof(double) * (size_t)heads * dim);
        double *kd = (double *)malloc(sizeof(double) * (size_t)dim);
        for (int64_t i = 0; i < (int64_t)heads * dim; i++)
            qd[i] = oracle_bf16_value(q_idx[(int64_t)j * heads * dim + i]);
        for (int64_t s = 0; s < n; s++) {
            int64_t r = phys_row(page_table, max_pages, b, s);
            if (r < 0 || r >= num_pages * SIA_ORACLE_PAGE) { bad = 1; continue; }
            double sigma = 1.0;
            if (k_dtype == 0) {
                const uint16_t *kr = (const uint16_t *)k_pool + r * dim;
                for (int32_t d = 0; d < dim; d++) kd[d] = oracle_bf16_value(kr[d]);
            } else {
                const uint8_t *kr = (const uint8_t *)k_pool + r * dim;
                for (int32_t d = 0; d < dim; d++) kd[d] = oracle_e4m3fn_value(kr[d]);
                sigma = (double)k_scale[r];
            }
            double acc = 0.0;
            for (int32_t h = 0; h < heads; h++) {
                const double *qh = qd + (int64_t)h * dim;
                double a = 0.0; /* relevance of head h: q_h . k_s */
                for (int32_t d = 0; d < dim; d++) a += qh[d] * kd[d];
                acc += (double)w[(int64_t)j * heads + h] * (a > 0.0 ? a : 0.0);
            }
            row[s] = sigma * acc;
        }
        free(qd);
        free(kd);
    }
    return bad ? -2 : 0;
}

/*
 * MXFP8 (the index path's quantized form: "Rapid Adaptation and Inference
 * Optimization", section 5.1; "Day0 Inference Adaptation ... for a New
 * Hybrid-Attention LLM Architecture", section 4.2): e4m3 elements, one E8M0
 * scale 2^(byte - 127) per 32 consecutive elements.
 */
static double e8m0_value(uint8_t byte) { return ldexp(1.0, (int)byte - 127); }

/* The e4m3fn code whose value is nearest to v (|v| <= 448), ties to the code
 * with an even mantissa: a search over every finite non-negative code for the
 * magnitude, then v's sign bit (a negative value that rounds to zero gives -0,
 * as a round-to-nearest conversion keeps the sign). */
static uint8_t nearest_e4m3fn(double v) {
    const double a = fabs(v);
    int best = 0;
    double best_err = INFINITY;
    for (int c = 0; c < 0x7F; c++) {
        const double err = fabs(oracle_e4m3fn_value((uint8_t)c) - a);
        if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_err = err;
        }
    }
    return (uint8_t)(best | (signbit(v) ? 0x80 : 0));
}

/*
 * Quantize n_groups groups of 32 bf16 values: the scale is 2^e with e the
 * smallest integer in [-127, 127] for which the group's largest magnitude is
 * at most 448 * 2^e (the largest e4m3 value, so nothing is clipped); each
 * element is the e4m3 code nearest to x / 2^e. An all-zero group takes
 * e = -127.
 */
int oracle_quantize_mxfp8(const uint16_t *x, int64_t n_groups, uint8_t *codes, uint8_t *scales) {
    if (n_groups < 0 || !x || !codes || !scales) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < n_groups; g++) {
        double m = 0.0;
        for (int i = 0; i < 32; i++) {
            const double a = fabs(oracle_bf16_value(x[g * 32 + i]));
            if (a > m) m = a;
        }
        int e = -127;
        while (e < 127 && m > ldexp(448.0, e)) e++;
        scales[g] = (uint8_t)(e + 127);
        for (int i = 0; i < 32; i++)
            codes[g * 32 + i] = nearest_e4m3fn(oracle_bf16_value(x[g * 32 + i]) / ldexp(1.0, e));
    }
    return 0;
}

/*
 * Indexer scores on the MXFP8 path: the query and the index rows are MXFP8,
 * their values are the stored elements times their block scales, and no
 * per-token scale applies:
 *   scores[j*ld + s] = sum_h w[j,h] * max(0, q^[j,h,:] . k^_s)  for s < row_len[j]
 * k_codes [num_pages*64, dim], k_scales [num_pages*64, dim/32],
 * q_codes [num_q, heads, dim], q_scales [num_q, heads, dim/32].
 */
int oracle_indexer_scores_mx(int32_t num_q, const int32_t *q_seq, const int32_t *q_pos, int32_t batch,
                             const int32_t *seq_lens, const int32_t *page_table, int32_t max_pages,
                             int64_t num_pages, const uint8_t *k_codes, const uint8_t *k_scales,
                             int32_t dim, const uint8_t *q_codes, const uint8_t *q_scales,
                             const float *w, int32_t heads, double *scores, int64_t ld,
                             int32_t *row_len) {
    if (num_q < 0 || !q_seq || !q_pos || !seq_lens || !page_table || !k_codes || !k_scales ||
        !q_codes || !q_scales || !w || !scores || !row_len || dim <= 0 || dim % 32 || heads <= 0 ||
        batch <= 0)
        return -1;
    const int nb = dim / 32;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int32_t j = 0; j < num_q; j++) {
        int32_t b = q_seq[j];
        double *row = scores + (int64_t)j * ld;
        for (int64_t s = 0; s < ld; s++) row[s] = -INFINITY;
        row_len[j] = 0;
        if (b < 0 || b >= batch) { bad = 1; continue; }
        int64_t n = row_length(q_pos[j], seq_lens[b]);
        if (n > ld) { bad = 1; continue; }
        row_len[j] = (int32_t)n;
        double *qd = (double *)malloc(sizeof(double) * (size_t)heads * dim);
        double *kd = (double *)malloc(sizeof(double) * (size_t)dim);
        for (int64_t i = 0; i < (int64_t)heads * dim; i++) {
            const int64_t e = (int64_t)j * heads * dim + i;   /* element, block e / 32 */
            qd[i] = oracle_e4m3fn_value(q_codes[e]) *
                    e8m0_value(q_scales[((int64_t)j * heads + i / dim) * nb + (i % dim) / 32]);
        }
        for (int64_t s = 0; s < n; s++) {
            int64_t r = phys_row(page_table, max_pages, b, s);
            if (r < 0 || r >= num_pages * SIA_ORACLE_PAGE) { bad = 1; continue; }
            for (int32_t d = 0; d < dim; d++)
                kd[d] = oracle_e4m3fn_value(k_codes[r * dim + d]) * e8m0_value(k_scales[r * nb + d / 32]);
            double acc = 0.0;
            for (int32_t h = 0; h < heads; h++) {
                const double *qh = qd + (int64_t)h * dim;
                double a = 0.0;
                for (int32_t d = 0; d < dim; d++) a += qh[d] * kd[d];
                acc += (double)w[(int64_t)j * heads + h] * (a > 0.0 ? a : 0.0);
            }
            row[s] = acc;
        }
        free(qd);
        free(kd);
    }
    return bad ? -2 : 0;
}

/* Total order of the selection: higher score first, then lower position.
 * NaN ranks below every number; -0.0 equals +0.0. */
typedef struct { double v; int32_t s; } cand_t;

static int rank_cmp(const void *pa, const void *pb) {
    const cand_t *a = (const cand_t *)pa, *b = (const cand_t *)pb;
    int an = isnan(a->v), bn = isnan(b->v);
    if (an != bn) return an ? 1 : -1;
    if (!an && a->v != b->v) return a->v > b->v ? -1 : 1;
    return (a->s > b->s) - (a->s < b->s);
}

static int pos_cmp(const void *pa, const void *pb) {
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

/*
 * Step 3: Top-K of each row. Row j has candidates 0..row_len[j]-1 with values
 * scores[j*ld + s]. Writes out_idx[j*K + i] (ascending position, -1 padded) and,
 * if out_score is not NULL, the matching scores (-inf for padding).
 */
int oracle_topk(int32_t num_q, const double *scores, int64_t ld, const int32_t *row_len,
                int32_t K, int32_t *out_idx, double *out_score) {
    if (num_q < 0 || !scores || !row_len || !out_idx || K <= 0) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int32_t j = 0; j < num_q; j++) {
        int64_t n = row_len[j];
        int32_t *oi = out_idx + (int64_t)j * K;
        for (int32_t i = 0; i < K; i++) oi[i] = -1;
        if (out_score)
            for (int32_t i = 0; i < K; i++) out_score[(int64_t)j * K + i] = -INFINITY;
        if (n < 0 || n > ld) { bad = 1; continue; }
        if (n == 0) continue;
        cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)n);
        for (int64_t s = 0; s < n; s++) {
            c[s].v = scores[(int64_t)j * ld + s];
            c[s].s = (int32_t)s;
        }
        qsort(c, (size_t)n, sizeof(cand_t), rank_cmp);
        int64_t m = n < K ? n : K;
        for (int64_t i = 0; i < m; i++) oi[i] = c[i].s;
        qsort(oi, (size_t)m, sizeof(int32_t), pos_cmp);
        if (out_score)
            for (int64_t i = 0; i < m; i++)
                out_score[(int64_t)j * K + i] = scores[(int64_t)j * ld + oi[i]];
        free(c);
    }
    return bad ? -2 : 0;
}

/*
 * Steps 4-5: gather the selected latent rows through the page table and run
 * softmax attention over them, per head a:
 *   z_i = sm_scale * (q[j,a,:] . c_i)        over all dim_kv columns
 *   p_i = exp(z_i - max z) / sum exp(z - max z)
 *   out[j,a,:] = sum_i p_i c_i[0:d_v],  lse[j,a] = max z + ln sum exp(z - max z)
 * Entries of idx that are < 0 are padding and ignored; idx holds logical
 * positions of sequence q_seq[j].
 */
int oracle_sparse_mla(int32_t num_q, const int32_t *q_seq, int32_t batch,
                      const int32_t *page_table, int32_t max_pages, int64_t num_pages,
                      const uint16_t *kv_pool, int32_t dim_kv, int32_t d_v,
                      const uint16_t *q, int32_t heads, const int32_t *idx, int32_t K,
                      double sm_scale, double *out, double *lse) {
    if (num_q < 0 || !q_seq || !page_table || !kv_pool || !q || !idx || !out || !lse ||
        dim_kv <= 0 || d_v <= 0 || d_v > dim_kv || heads <= 0 || K <= 0 || batch <= 0)
        return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int32_t j = 0; j < num_q; j++) {
        int32_t b = q_seq[j];
        double *oj = out + (int64_t)j * heads * d_v;
        for (int64_t i = 0; i < (int64_t)heads * d_v; i++) oj[i] = 0.0;
        for (int32_t a = 0; a < heads; a++) lse[(int64_t)j * heads + a] = -INFINITY;
        if (b < 0 || b >= batch) { bad = 1; continue; }
        /* gather */
        int32_t m = 0;
        double *c = (double *)malloc(sizeof(double) * (size_t)K * dim_kv);
        for (int32_t i = 0; i < K; i++) {
            int32_t s = idx[(int64_t)j * K + i];
            if (s < 0) continue;
            int64_t r = phys_row(page_table, max_pages, b, s);
            if (r < 0 || r >= num_pages * SIA_ORACLE_PAGE) { bad = 1; continue; }
            for (int32_t d = 0; d < dim_kv; d++)
                c[(int64_t)m * dim_kv + d] = oracle_bf16_value(kv_pool[r * dim_kv + d]);
            m++;
        }
        if (m == 0) { free(c); continue; }
        double *qa = (double *)malloc(sizeof(double) * (size_t)dim_kv);
        double *z = (double *)malloc(sizeof(double) * (size_t)m);
        for (int32_t a = 0; a < heads; a++) {
            for (int32_t d = 0; d < dim_kv; d++)
                qa[d] = oracle_bf16_value(q[((int64_t)j * heads + a) * dim_kv + d]);
            double zmax = -INFINITY;
            for (int32_t i = 0; i < m; i++) {
                double dot = 0.0;
                for (int32_t d = 0; d < dim_kv; d++) dot += qa[d] * c[(int64_t)i * dim_kv + d];
                z[i] = sm_scale * dot;
                if (z[i] > zmax) zmax = z[i];
            }
            double l = 0.0;
            for (int32_t i = 0; i < m; i++) {
                z[i] = exp(z[i] - zmax);
                l += z[i];
            }
            double *o = oj + (int64_t)a * d_v;
            for (int32_t i = 0; i < m; i++) {
                double p = z[i] / l;
                for (int32_t d = 0; d < d_v; d++) o[d] += p * c[(int64_t)i * dim_kv + d];
            }
            lse[(int64_t)j * heads + a] = zmax + log(l);
        }
        free(qa);
        free(z);
        free(c);
    }
    return bad ? -2 : 0;
}

/* Threads the OpenMP loops above use from now on (n >= 1); returns the previous
 * count. Only the thread count changes, never what is computed. */
int oracle_set_num_threads(int n) {
#ifdef _OPENMP
    const int prev = omp_get_max_threads();
    if (n >= 1) omp_set_num_threads(n);
    return prev;
#else
    (void)n;
    return 1;
#endif
}

/*
 * Sparse attention over an FP8 latent cache (the pages' main-attention KV
 * quantization: "Rapid Adaptation and Inference Optimization", section 5.2;
 * "Day0 Inference Adaptation ... for New-Architecture LLMs", section 4: per
 * token, blocks of 128 elements share one scale). Each row is 656 bytes:
 *   bytes   0..511  e4m3fn codes of latent elements 0..511
 *   bytes 512..527  four fp32 scales, one per block of 128 latent elements
 *   bytes 528..655  the 64 rope elements (576 - 512) as bf16
 * The row's values are code * scale[d / 128] for d < 512 and the bf16 value
 * for d >= 512; then the same attention as oracle_sparse_mla.
 */
int oracle_sparse_mla_fp8(int32_t num_q, const int32_t *q_seq, int32_t batch,
                          const int32_t *page_table, int32_t max_pages, int64_t num_pages,
                          const uint8_t *kv_rows, const uint16_t *q, int32_t heads,
                          const int32_t *idx, int32_t K, double sm_scale, double *out, double *lse) {
    enum { DK = 576, DV = 512, ROW = 656 };
    if (num_q < 0 || !q_seq || !page_table || !kv_rows || !q || !idx || !out || !lse || heads <= 0 ||
        K <= 0 || batch <= 0)
        return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int32_t j = 0; j < num_q; j++) {
        int32_t b = q_seq[j];
        double *oj = out + (int64_t)j * heads * DV;
        for (int64_t i = 0; i < (int64_t)heads * DV; i++) oj[i] = 0.0;
        for (int32_t a = 0; a < heads; a++) lse[(int64_t)j * heads + a] = -INFINITY;
        if (b < 0 || b >= batch) { bad = 1; continue; }
        int32_t m = 0;
        double *c = (double *)malloc(sizeof(double) * (size_t)K * DK);
        for (int32_t i = 0; i < K; i++) {
            int32_t s = idx[(int64_t)j * K + i];
            if (s < 0) continue;
            int64_t r = phys_row(page_table, max_pages, b, s);
            if (r < 0 || r >= num_pages * SIA_ORACLE_PAGE) { bad = 1; continue; }
            const uint8_t *row = kv_rows + r * ROW;
            float sc[4];
            memcpy(sc, row + 512, sizeof sc);
            for (int32_t d = 0; d < DV; d++)
                c[(int64_t)m * DK + d] = oracle_e4m3fn_value(row[d]) * (double)sc[d / 128];
            for (int32_t d = DV; d < DK; d++) {
                uint16_t bits;
                memcpy(&bits, row + 528 + 2 * (d - DV), 2);
                c[(int64_t)m * DK + d] = oracle_bf16_value(bits);
            }
            m++;
        }
        if (m == 0) { free(c); continue; }
        double *qa = (double *)malloc(sizeof(double) * DK);
        double *z = (double *)malloc(sizeof(double) * (size_t)m);
        for (int32_t a = 0; a < heads; a++) {
            for (int32_t d = 0; d < DK; d++) qa[d] = oracle_bf16_value(q[((int64_t)j * heads + a) * DK + d]);
            double zmax = -INFINITY;
            for (int32_t i = 0; i < m; i++) {
                double dot = 0.0;
                for (int32_t d = 0; d < DK; d++) dot += qa[d] * c[(int64_t)i * DK + d];
                z[i] = sm_scale * dot;
                if (z[i] > zmax) zmax = z[i];
            }
            double l = 0.0;
            for (int32_t i = 0; i < m; i++) {
                z[i] = exp(z[i] - zmax);
                l += z[i];
            }
            double *o = oj + (int64_t)a * DV;
            for (int32_t i = 0; i < m; i++) {
                double p = z[i] / l;
                for (int32_t d = 0; d < DV; d++) o[d] += p * c[(int64_t)i * DK + d];
            }
            lse[(int64_t)j * heads + a] = zmax + log(l);
        }
        free(qa);
        free(z);
        free(c);
    }
    return bad ? -2 : 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
