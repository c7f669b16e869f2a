/* Drives every oracle entry point on tiny inputs, valid and invalid, under
 * AddressSanitizer and UndefinedBehaviorSanitizer (built by
 * tests/test_sanitizers.py). Exits non-zero if a return code is not the
 * expected one; the sanitizers abort on any memory or UB error. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_decode_bf16(const void *bits, double *out, int64_t n);
int oracle_decode_e4m3fn(const void *codes, double *out, int64_t n);
int oracle_indexer_scores(int32_t, const int32_t *, const int32_t *, int32_t, const int32_t *, const int32_t *,
                          int32_t, int64_t, const void *, int32_t, const float *, int32_t, const uint16_t *,
                          const float *, int32_t, double *, int64_t, int32_t *);
int oracle_topk(int32_t, const double *, int64_t, const int32_t *, int32_t, int32_t *, double *);
int oracle_sparse_mla(int32_t, const int32_t *, int32_t, const int32_t *, int32_t, int64_t, const uint16_t *,
                      int32_t, int32_t, const uint16_t *, int32_t, const int32_t *, int32_t, double, double *,
                      double *);
int oracle_quantize_mxfp8(const uint16_t *, int64_t, uint8_t *, uint8_t *);
int oracle_indexer_scores_mx(int32_t, const int32_t *, const int32_t *, int32_t, const int32_t *, const int32_t *,
                             int32_t, int64_t, const uint8_t *, const uint8_t *, int32_t, const uint8_t *,
                             const uint8_t *, const float *, int32_t, double *, int64_t, int32_t *);
int oracle_sparse_mla_fp8(int32_t, const int32_t *, int32_t, const int32_t *, int32_t, int64_t, const uint8_t *,
                          const uint16_t *, int32_t, const int32_t *, int32_t, double, double *, double *);

static int fails = 0;
#define EXPECT(x, want)                                                                 \
    do {                                                                                \
        int got_ = (x);                                                                 \
        if (got_ != (want)) {                                                           \
            fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #x, \
                    got_, (want));                                                      \
            fails++;                                                                    \
        }                                                                               \
    } while (0)

static uint16_t bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

int main(void) {
    enum { B = 2, MP = 3, NP = 6, D = 64, H = 4, Q = 3, K = 8, DK = 576, HA = 2 };
    int32_t seq_lens[B] = {150, 70};
    int32_t table[B * MP] = {4, 0, 2, 5, 1, -1};
    int32_t q_seq[Q] = {0, 1, 1};
    int32_t q_pos[Q] = {149, 69, 10};
    uint16_t *kb = calloc(NP * 64 * D, sizeof *kb);
    uint8_t *k8 = calloc(NP * 64 * D, 1);
    float *ksc = malloc(sizeof(float) * NP * 64);
    uint16_t *q = malloc(sizeof *q * Q * H * D);
    float w[Q * H];
    for (int i = 0; i < NP * 64 * D; i++) {
        kb[i] = bf16((float)((i * 37) % 17) - 8.f);
        k8[i] = (uint8_t)((i * 53) % 0x7E);
    }
    for (int i = 0; i < NP * 64; i++) ksc[i] = 0.5f + (float)(i % 7) / 7.f;
    for (int i = 0; i < Q * H * D; i++) q[i] = bf16((float)((i * 11) % 13) - 6.f);
    for (int i = 0; i < Q * H; i++) w[i] = 0.1f * (float)(i % 5) - 0.2f;
    const int64_t ld = 160;
    double *scores = malloc(sizeof(double) * Q * ld);
    int32_t row_len[Q];
    EXPECT(oracle_indexer_scores(Q, q_seq, q_pos, B, seq_lens, table, MP, NP, kb, 0, NULL, D, q, w, H, scores, ld,
                                 row_len), 0);
    EXPECT(oracle_indexer_scores(Q, q_seq, q_pos, B, seq_lens, table, MP, NP, k8, 1, ksc, D, q, w, H, scores, ld,
                                 row_len), 0);
    EXPECT(oracle_indexer_scores(Q, q_seq, q_pos, B, seq_lens, table, MP, NP, kb, 7, NULL, D, q, w, H, scores, ld,
                                 row_len), -1);
    int32_t bad_seq[Q] = {0, 5, -1};
    EXPECT(oracle_indexer_scores(Q, bad_seq, q_pos, B, seq_lens, table, MP, NP, kb, 0, NULL, D, q, w, H, scores,
                                 ld, row_len), -2);
    int32_t idx[Q * K];
    double top[Q * K];
    EXPECT(oracle_indexer_scores(Q, q_seq, q_pos, B, seq_lens, table, MP, NP, kb, 0, NULL, D, q, w, H, scores, ld,
                                 row_len), 0);
    EXPECT(oracle_topk(Q, scores, ld, row_len, K, idx, top), 0);
    EXPECT(oracle_topk(Q, scores, ld, row_len, 0, idx, top), -1);
    /* attention, bf16 and fp8 latent rows */
    uint16_t *kv = malloc(sizeof *kv * NP * 64 * DK);
    uint8_t *kv8 = malloc((size_t)NP * 64 * 656);
    uint16_t *qa = malloc(sizeof *qa * Q * HA * DK);
    for (int i = 0; i < NP * 64 * DK; i++) kv[i] = bf16((float)((i * 7) % 23) / 23.f - 0.5f);
    for (int r = 0; r < NP * 64; r++) {
        for (int d = 0; d < 512; d++) kv8[(size_t)r * 656 + d] = (uint8_t)((r + d) % 0x7E);
        float sc[4] = {0.01f, 0.02f, 0.03f, 0.04f};
        memcpy(kv8 + (size_t)r * 656 + 512, sc, 16);
        for (int d = 0; d < 64; d++) {
            uint16_t b = bf16(0.25f * (float)(d % 4));
            memcpy(kv8 + (size_t)r * 656 + 528 + 2 * d, &b, 2);
        }
    }
    for (int i = 0; i < Q * HA * DK; i++) qa[i] = bf16((float)((i * 3) % 7) / 7.f);
    double *out = malloc(sizeof(double) * Q * HA * 512), lse[Q * HA];
    EXPECT(oracle_sparse_mla(Q, q_seq, B, table, MP, NP, kv, DK, 512, qa, HA, idx, K, 0.04, out, lse), 0);
    EXPECT(oracle_sparse_mla_fp8(Q, q_seq, B, table, MP, NP, kv8, qa, HA, idx, K, 0.04, out, lse), 0);
    int32_t bad_idx[Q * K];
    for (int i = 0; i < Q * K; i++) bad_idx[i] = i % 3 == 0 ? -1 : 200 + i;   /* past the table */
    EXPECT(oracle_sparse_mla(Q, q_seq, B, table, MP, NP, kv, DK, 512, qa, HA, bad_idx, K, 0.04, out, lse), -2);
    EXPECT(oracle_sparse_mla_fp8(Q, bad_seq, B, table, MP, NP, kv8, qa, HA, idx, K, 0.04, out, lse), -2);
    /* MXFP8 */
    uint8_t qc[Q * H * D], qs[Q * H * D / 32], ks8[NP * 64 * D / 32];
    EXPECT(oracle_quantize_mxfp8(q, Q * H * D / 32, qc, qs), 0);
    EXPECT(oracle_quantize_mxfp8(kb, NP * 64 * D / 32, k8, ks8), 0);
    EXPECT(oracle_indexer_scores_mx(Q, q_seq, q_pos, B, seq_lens, table, MP, NP, k8, ks8, D, qc, qs, w, H, scores,
                                    ld, row_len), 0);
    EXPECT(oracle_indexer_scores_mx(Q, q_seq, q_pos, B, seq_lens, table, MP, NP, k8, ks8, 48, qc, qs, w, H, scores,
                                    ld, row_len), -1);
    double dec[16];
    EXPECT(oracle_decode_bf16(q, dec, 16), 0);
    EXPECT(oracle_decode_e4m3fn(k8, dec, 16), 0);
    free(kb); free(k8); free(ksc); free(q); free(scores); free(kv); free(kv8); free(qa); free(out);
    if (fails) return 1;
    printf("oracle driver: all checks passed\n");
    return 0;
}
