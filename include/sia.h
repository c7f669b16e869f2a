/*
 * sia.h -- C ABI of the sparse-indexer / Top-K / sparse-MLA-attention library
 * for AMD Instinct MI355X (gfx950).
 *
 * The library implements the two-stage "filter-then-compute" sparse attention
 * path of hybrid-attention LLMs:
 *
 *   stage 1  sparse_indexer_topk   -- a lightweight indexer scores every visible
 *            historical position against the query by reading the paged index-K
 *            cache directly, combines its heads with per-token head weights and
 *            keeps the Top-K positions ("Rapid Adaptation and Inference
 *            Optimization: Key Engineering Practices for Day0 LLM Support",
 *            section 4.1 "Indexer Fusion"; "Day0 Inference Adaptation and
 *            Performance Optimization for New-Architecture LLMs", section 3.1
 *            "Fused Indexer"). No score ever reaches memory. Long causal rows
 *            (prefill) take one fused pass that writes only the selected
 *            indices. Decode rows, which a single workgroup cannot stream fast
 *            enough, are split over workgroups: a scoring pass keeps, per part of
 *            a row, only the positions whose score reaches a running floor (the
 *            part's K-th largest so far, at coarse granularity) and appends them
 *            with their keys to the workspace; a selection pass then takes the
 *            exact Top-K of those candidates.
 *   stage 2  sparse_mla_attention -- gathers only the selected rows of the paged
 *            latent (MLA) KV cache and runs softmax attention over them
 *            ("Rapid Adaptation ...", section 4.2 "Sparse Attention
 *            Computation"; "Day0 ... for a New Hybrid-Attention LLM
 *            Architecture", section 2.2 "Sparse Index Attention Module").
 *
 * Indexer score (the pages say only "scores ... aggregates multi-head scores
 * with weights"; this library fixes the formula):
 *   score[j,s] = sigma_s * sum_h w[j,h] * max(0, q[j,h,:] . k_s)
 * where k_s is the exact value of the stored index-K row and sigma_s its fp32
 * per-token scale (fp8 cache) or 1 (bf16 cache). Query j at absolute position
 * t_j in sequence b sees positions s with s <= t_j and s < n_b. Top-K keeps the
 * first min(K, visible) positions in the order (score descending, position
 * ascending) and lists them by ascending position, padding with -1.
 *
 * Conventions for every entry point:
 *  - Pointers in the descriptors and arguments are DEVICE pointers unless the
 *    field says "host". The caller owns every buffer; the library never
 *    allocates, frees or synchronizes; work is enqueued on `stream`
 *    (a hipStream_t, NULL = the default stream).
 *  - Arguments are validated on the host before anything is enqueued. A bad
 *    argument returns a negative sia_status, sets sia_last_error() and launches
 *    nothing. A failed launch returns SIA_ERR_HIP.
 *  - Device data that the host cannot see (page ids, sequence ids of queries,
 *    positions, stage-2 indices) is bounds-checked by the kernels and never
 *    dereferenced when out of range; a bit is set in the status word at the
 *    start of the workspace, readable with sia_read_device_status():
 *      - a query whose sequence id is outside [0, batch): stage 1 selects
 *        nothing (all -1), stage 2 gives a zero output and lse = -inf;
 *      - a page id outside [0, num_pages): stage 1 drops the positions on
 *        that page (they are never selected), stage 2 skips the rows on it;
 *      - a stage-2 index >= n_b: the entry is skipped.
 *  - Paged caches: row r of physical page p sits at
 *    rows + ((size_t)p * page_size + r) * dim * element_size; the page size is
 *    64. Logical position s of sequence b lives on physical page
 *    page_table[b * max_pages + s / 64], row s % 64. Both caches share one
 *    page table.
 *  - Inputs are never written.
 */
#ifndef SIA_H
#define SIA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SIA_OK = 0,
    SIA_ERR_INVALID_ARG = -1, /* null pointer, negative size, inconsistent shapes */
    SIA_ERR_UNSUPPORTED = -2, /* valid but not built: head count, dim, dtype, page size */
    SIA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than the size query says */
    SIA_ERR_HIP = -4          /* a HIP runtime call failed */
} sia_status;

typedef enum {
    SIA_BF16 = 0,         /* bfloat16 */
    SIA_FP8_E4M3FN = 1,   /* OCP float8 E4M3 (max 448, no infinities) */
    SIA_MXFP8_E4M3 = 2    /* MXFP8: E4M3 elements, one E8M0 scale (2^(byte - 127)) per 32
                             consecutive elements of a row ("Rapid Adaptation ...", section 5.1
                             "Full Quantization for the Indexer Path"; index caches only) */
} sia_dtype;

/* Page table shared by the index-K cache and the latent KV cache. */
typedef struct {
    const int32_t *page_table; /* device [batch, max_pages]; physical page ids, -1 = unused */
    const int32_t *seq_lens;   /* device [batch]; n_b, positions 0..n_b-1 are valid */
    int32_t batch;
    int32_t max_pages;         /* row stride of page_table; n_b <= 64 * max_pages */
    int32_t page_size;         /* must be 64 */
} sia_page_table;

/* One paged cache: [num_pages, page_size, dim] rows (+ their scales). */
typedef struct {
    const void *rows;          /* device [num_pages, 64, dim] elements of `dtype` */
    const void *scale;         /* device; SIA_FP8_E4M3FN: fp32 [num_pages, 64] per-token scales;
                                  SIA_MXFP8_E4M3: uint8 E8M0 [num_pages, 64, dim / 32] block scales;
                                  NULL for SIA_BF16 */
    int64_t num_pages;
    int32_t dim;
    int32_t dtype;             /* sia_dtype */
} sia_paged_cache;

/* The query tokens of one call. */
typedef struct {
    int32_t num_q;
    const int32_t *q_seq;      /* device [num_q]; sequence id b_j in [0, batch) */
    const int32_t *q_pos;      /* device [num_q]; absolute position t_j >= 0 */
    int32_t group;             /* host; queries [g*group, (g+1)*group) belong to one sequence.
                                  1 is always valid. 2 for two draft tokens per sequence;
                                  a prefill chunk of one sequence may pass its length. Larger
                                  groups let one pass over the cache serve several queries. */
    int32_t max_visible;       /* host; >= max_j min(t_j + 1, n_{b_j}); sizes the launch. A query
                                  whose visible row is longer is not scored past this bound and
                                  sets SIA_DEVSTATUS_ROW_TOO_LONG. */
} sia_queries;

/* Bits of the device status word (first 4 bytes of every workspace). */
#define SIA_DEVSTATUS_BAD_SEQ 1u        /* q_seq out of [0, batch) */
#define SIA_DEVSTATUS_BAD_PAGE 2u       /* page id out of [0, num_pages) for a visible position */
#define SIA_DEVSTATUS_ROW_TOO_LONG 4u   /* visible row longer than max_visible */
#define SIA_DEVSTATUS_BAD_INDEX 8u      /* stage 2: idx entry >= n_b */

/* Scheduling of long causal rows (prefill) over the compute units. */
typedef enum {
    SIA_SCHED_AUTO = -1,     /* library choice (SIA_SCHED_HEAVY_FIRST) */
    SIA_SCHED_NAIVE = 0,     /* one workgroup per query tile, in tile order */
    SIA_SCHED_HEAVY_FIRST = 1, /* persistent workgroups take tiles longest-row first */
    SIA_SCHED_ZIGZAG = 2     /* workgroup i takes tiles i and T-1-i (head paired with tail) */
} sia_sched;

/* ------------------------------------------------------------------ stage 1 */

/* Bytes of workspace sparse_indexer_topk / sparse_indexer_scores need for these
 * shapes (always >= 256). Returns 0 if the arguments are invalid. */
size_t sia_indexer_workspace_size(const sia_page_table *pt, const sia_paged_cache *index_k,
                                  const sia_queries *qs, int32_t heads, int32_t topk);

/*
 * Fused indexer + Top-K.
 *   q_idx     device bf16 [num_q, heads, dim]   indexer query heads (dim = index_k->dim)
 *   w         device fp32 [num_q, heads]        per-token head weights
 *   topk      1 <= K <= 8192
 *   out_idx   device int32 [num_q, topk]        selected logical positions, ascending, -1 padded
 *   out_score device fp32 [num_q, topk] or NULL scores of out_idx entries (-inf for padding)
 *   sched     sia_sched for long causal rows; results do not depend on it
 * Supported: 1 <= heads <= 64, dim in {64, 128}, index_k dtype bf16 or fp8
 * e4m3fn, page size 64.
 */
int sparse_indexer_topk(const sia_page_table *pt, const sia_paged_cache *index_k,
                        const sia_queries *qs, const void *q_idx, const float *w,
                        int32_t heads, int32_t topk, int32_t *out_idx, float *out_score,
                        int32_t sched, void *workspace, size_t workspace_bytes, void *stream);

/*
 * The indexer on the MXFP8 path: an index cache of dtype SIA_MXFP8_E4M3 (dim
 * 128) and an MXFP8 query,
 *   score[j,s] = sum_h w[j,h] * max(0, q^[j,h,:] . k^_s)
 * with q^ and k^ the exact values of the stored elements times their block
 * scales (no per-token scale). Same selection, outputs, workspace
 * (sia_indexer_workspace_size with the MXFP8 cache descriptor), scheduling and
 * error conventions as sparse_indexer_topk.
 *   q_codes   device uint8 [num_q, heads, dim]       e4m3 codes of the query
 *   q_scales  device uint8 [num_q, heads, dim / 32]  their E8M0 block scales
 * ("Rapid Adaptation ...", section 5.1; "Day0 ... New-Architecture LLMs",
 * section 4 "Layered Quantization": index Q/K in MXFP8.)
 */
int sparse_indexer_topk_mxfp8(const sia_page_table *pt, const sia_paged_cache *index_k,
                              const sia_queries *qs, const uint8_t *q_codes, const uint8_t *q_scales,
                              const float *w, int32_t heads, int32_t topk, int32_t *out_idx,
                              float *out_score, int32_t sched, void *workspace,
                              size_t workspace_bytes, void *stream);

/* Test hook: the MXFP8 path's scores (as sparse_indexer_scores). */
int sparse_indexer_scores_mxfp8(const sia_page_table *pt, const sia_paged_cache *index_k,
                                const sia_queries *qs, const uint8_t *q_codes,
                                const uint8_t *q_scales, const float *w, int32_t heads,
                                float *scores, int64_t ld, void *workspace, size_t workspace_bytes,
                                void *stream);

/*
 * Quantize bf16 rows to MXFP8: every group of 32 consecutive elements of a row
 * gets the scale 2^e with e the smallest integer in [-127, 127] for which the
 * group's largest magnitude is at most 448 * 2^e (so no element is clipped),
 * stored as the E8M0 byte e + 127; each element becomes the e4m3 code nearest
 * to x / 2^e (ties to even). An all-zero group gets e = -127 and zero codes.
 *   x       device bf16 [rows, dim], finite values; dim a positive multiple of 32
 *   codes   device uint8 [rows, dim]
 *   scales  device uint8 [rows, dim / 32]
 */
int sia_quantize_mxfp8(const void *x, int64_t rows, int32_t dim, uint8_t *codes, uint8_t *scales,
                       void *stream);

/*
 * Test hook: sparse_indexer_topk with a record of where and when each
 * workgroup of the causal stream kernel (the prefill path) ran, to measure how
 * evenly a tile schedule loads the compute units. Results are those of
 * sparse_indexer_topk. wg_trace: device uint64 [trace_cap, 4]; record i of
 * workgroup i < trace_cap = {hardware ids (XCC_ID << 32 | HW_ID register:
 * shader engine, array, CU, SIMD, wave), start, end (a 100 MHz clock shared by
 * the whole GPU), query tiles the workgroup ran}. Calls that take the decode
 * path (score + selection passes) write no records.
 */
int sparse_indexer_topk_traced(const sia_page_table *pt, const sia_paged_cache *index_k,
                               const sia_queries *qs, const void *q_idx, const float *w,
                               int32_t heads, int32_t topk, int32_t *out_idx, float *out_score,
                               int32_t sched, void *workspace, size_t workspace_bytes, void *stream,
                               uint64_t *wg_trace, int32_t trace_cap);

/*
 * Test hook: the indexer's scores without selection, computed by the same device
 * code the fused pass uses, so that selection can be checked on identical
 * scores. scores: device fp32 [num_q, ld]; entry s of row j holds the score of
 * position s for s < min(t_j + 1, n_b), -inf for the rest of [0, ld).
 * Requires ld >= max_visible.
 */
int sparse_indexer_scores(const sia_page_table *pt, const sia_paged_cache *index_k,
                          const sia_queries *qs, const void *q_idx, const float *w,
                          int32_t heads, float *scores, int64_t ld, void *workspace,
                          size_t workspace_bytes, void *stream);

/* Bytes of workspace sparse_topk_from_scores needs. */
size_t sia_topk_workspace_size(int32_t num_q, int32_t max_row_len, int32_t topk);

/*
 * Test hook: Top-K of given score rows with the device selection the fused pass
 * uses. Row j has candidates 0..row_len[j]-1 (device int32 [num_q], each
 * <= max_row_len <= ld). Same output convention as sparse_indexer_topk.
 */
int sparse_topk_from_scores(const float *scores, int64_t ld, const int32_t *row_len,
                            int32_t num_q, int32_t max_row_len, int32_t topk,
                            int32_t *out_idx, float *out_score, void *workspace,
                            size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------ input preparation */

/*
 * Projection weights of the indexer's inputs (bf16, out x in like a linear
 * layer): the query heads from the query latent xq, the index key and the head
 * weights from the hidden state xh.
 */
typedef struct {
    const void *wq;        /* device bf16 [heads * dim, dq] */
    const void *wk;        /* device bf16 [dim, dh] */
    const float *k_gamma;  /* device fp32 [dim]: LayerNorm scale of the key */
    const float *k_beta;   /* device fp32 [dim]: LayerNorm shift of the key */
    const void *ww;        /* device bf16 [heads, dh] */
    int32_t dq, dh;        /* input widths, multiples of 16 */
    int32_t heads;         /* indexer heads, 1..64 */
    int32_t dim;           /* index dim, 128 */
    float eps;             /* LayerNorm epsilon */
} sia_indexer_weights;

/* Bytes of workspace sia_indexer_prepare needs for num_q tokens (0 if invalid). */
size_t sia_indexer_prepare_workspace_size(const sia_indexer_weights *W, int32_t num_q);

/*
 * Indexer input preparation for the MXFP8 index path, on three streams
 * ("Rapid Adaptation ...", section 4.3 "Multi-Stream Parallel Preparation";
 * "Day0 ... New-Architecture LLMs", section 3.2 "Three-Stream Coordination for
 * Indexer Input Preparation"). For the num_q tokens of qs (sequence q_seq[t],
 * position q_pos[t]):
 *   streams[0]: q = xq Wq^T (bf16), quantized to MXFP8 -> q_codes, q_scales
 *   streams[1]: k = LayerNorm(xh Wk^T) * gamma + beta, rounded to bf16, quantized
 *               to MXFP8 and written into index_k (dtype SIA_MXFP8_E4M3, dim 128)
 *               at row q_pos[t] of sequence q_seq[t] (the only input this call
 *               writes)
 *   streams[2]: w = xh Ww^T (fp32) -> w_out
 * The chains fork from streams[0] (events[0] recorded there first, so work
 * enqueued on streams[0] before the call is visible to all three) and join back
 * into streams[0] (events[1], events[2]), so the indexer enqueued on
 * streams[0] afterwards sees all its inputs. The same stream may be passed
 * three times (a serial chain). Streams and events are the caller's (hipStream_t,
 * hipEvent_t; NULL streams are the default stream).
 *   xq        device bf16 [num_q, dq];  xh device bf16 [num_q, dh]
 *   q_codes   device uint8 [num_q, heads, dim];  q_scales uint8 [num_q, heads, dim/32]
 *   w_out     device fp32 [num_q, heads]
 *   q_bf16    device bf16 [num_q, heads, dim] or NULL: the query before quantization
 *   k_bf16    device bf16 [num_q, dim] or NULL: the key before quantization
 * A token whose sequence, position or page is out of range writes no key row
 * and sets SIA_DEVSTATUS_BAD_PAGE in the workspace status word.
 */
int sia_indexer_prepare(const sia_indexer_weights *W, const void *xq, const void *xh,
                        const sia_page_table *pt, const sia_paged_cache *index_k,
                        const sia_queries *qs, uint8_t *q_codes, uint8_t *q_scales, float *w_out,
                        void *q_bf16, void *k_bf16, void *workspace, size_t workspace_bytes,
                        void *const *streams, void *const *events);

/* ------------------------------------------------------------------ stage 2 */

/* Bytes of workspace sparse_mla_attention needs (always >= 256). */
size_t sia_mla_workspace_size(const sia_queries *qs, int32_t heads, int32_t d_v, int32_t topk);

/*
 * Sparse MLA attention over the selected rows of the latent KV cache.
 *   kv        latent cache, dim 576 (512 latent + 64 rope), scale NULL, in one of two
 *             row formats:
 *               SIA_BF16: 576 bf16 values per row;
 *               SIA_FP8_E4M3FN: 656-byte rows: 512 e4m3 codes, four fp32 scales (one
 *               per 128 latent values: value = code * scale), then the 64 rope values
 *               as bf16 ("Rapid Adaptation ...", section 5.2 "Main Attention KV Cache
 *               Quantization": per token, blocks of 128 share one scale). The fp8
 *               path multiplies the bf16 query's latent part as two e4m3 terms (one
 *               exponent per head) against the codes on fp8 matrix cores, applies
 *               each row's block scales to its logits and folds them into the
 *               probabilities (bf16) of the value product.
 *   q         device bf16 [num_q, heads, 576]
 *   d_v       value width: the first d_v columns of each row (512)
 *   idx       device int32 [num_q, topk]; logical positions of sequence q_seq[j],
 *             entries < 0 are skipped (any order; duplicates count twice)
 *   sm_scale  softmax scale applied to q . c
 *   out       device bf16 [num_q, heads, d_v]: sum_i softmax_i(sm_scale q.c_i) c_i[0:d_v]
 *   lse       device fp32 [num_q, heads] or NULL: natural-log sum-exp of the logits
 * Only num_q and q_seq of `qs` are read (q_pos may be NULL).
 * An empty selection gives out = 0 and lse = -inf.
 * Supported: heads a multiple of 16 up to 128, kv dim 576, d_v 512.
 */
int sparse_mla_attention(const sia_page_table *pt, const sia_paged_cache *kv,
                         const sia_queries *qs, const void *q, int32_t heads, int32_t d_v,
                         const int32_t *idx, int32_t topk, float sm_scale, void *out,
                         float *lse, void *workspace, size_t workspace_bytes, void *stream);

/*
 * sparse_mla_attention without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Same arguments, results and validation as
 * sparse_mla_attention, minus the workspace: the scratch it needs (row-slice
 * partials, the device status word) lives in a static device array of
 * SIA_MLA_NOALLOC_MAX_BYTES bytes (64 MiB) that the library holds on each GPU
 * it runs on until the process ends. It allocates and frees nothing.
 *  - A call whose sparse_mla_attention workspace size (sia_mla_workspace_size)
 *    exceeds that maximum returns SIA_ERR_WORKSPACE and launches nothing.
 *  - Every call on one GPU shares that GPU's array: calls that may overlap on
 *    one GPU (different streams without ordering, other host threads) race and
 *    must be serialized by the caller.
 *  - The device status bits of these calls are not reported (use the workspace
 *    form to read them).
 */
int sparse_mla_attention_noalloc(const sia_page_table *pt, const sia_paged_cache *kv,
                                 const sia_queries *qs, const void *q, int32_t heads, int32_t d_v,
                                 const int32_t *idx, int32_t topk, float sm_scale, void *out,
                                 float *lse, void *stream);
#define SIA_MLA_NOALLOC_MAX_BYTES ((size_t)64 << 20)

/* ------------------------------------------------------------------ misc */

/*
 * Zigzag pairing of S equal shards over S/2 workers: worker i takes shards i and
 * S-1-i, so that with a cost growing linearly along a causal sequence every
 * worker carries the same load ("Day0 ... for a New Hybrid-Attention LLM
 * Architecture", section 4.3, Zigzag Load Balancing). Host function; the
 * prefill scheduler's SIA_SCHED_ZIGZAG mode uses the same mapping on the
 * device. out: host int32 [S]; out[2i], out[2i+1] = the shards of worker i (an
 * odd S leaves the middle shard alone on the last worker: out[S-1] = S/2).
 */
int sia_zigzag_assign(int32_t num_shards, int32_t *out);

/* Zero the device status word of a workspace (enqueued on stream). */
int sia_clear_device_status(void *workspace, void *stream);
/* Synchronize `stream` and read the device status word (SIA_DEVSTATUS_* bits). */
int sia_read_device_status(const void *workspace, void *stream, uint32_t *status);

/* Message for the last non-OK status returned on this thread. */
const char *sia_last_error(void);
/* Library version, major*10000 + minor*100 + patch. */
int sia_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SIA_H */
