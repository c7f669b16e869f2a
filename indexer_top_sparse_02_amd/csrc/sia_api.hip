// Host entry points of the C ABI declared in include/sia.h: argument
// validation (before anything touches the GPU), launch planning, workspace
// layout and dispatch to the gfx950 kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "sia.h"
#include "sia_kernels.h"
#include "sia_sched.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(SIA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kHeader = 256;   // status word at 0, work counter at 4
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int round_up_pow2(int64_t x) {
    int64_t p = 1;
    while (p < x) p <<= 1;
    return (int)p;
}

int env_int(const char* name, int dflt) {
    const char* v = getenv(name);
    return v && *v ? atoi(v) : dflt;
}

int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cus[dev]) {
        hipDeviceProp_t p;
        cus[dev] = hipGetDeviceProperties(&p, dev) == hipSuccess ? p.multiProcessorCount : 256;
    }
    return cus[dev];
}

// ------------------------------------------------------------ validation

int check_page_table(const sia_page_table* pt) {
    if (!pt) return fail(SIA_ERR_INVALID_ARG, "page table descriptor is NULL");
    if (!pt->page_table || !pt->seq_lens) return fail(SIA_ERR_INVALID_ARG, "page_table/seq_lens is NULL");
    if (pt->batch < 1 || pt->max_pages < 1)
        return fail(SIA_ERR_INVALID_ARG, "batch (%d) and max_pages (%d) must be >= 1", pt->batch, pt->max_pages);
    if (pt->page_size != 64) return fail(SIA_ERR_UNSUPPORTED, "page_size %d: only 64 is supported", pt->page_size);
    if ((int64_t)pt->max_pages * 64 > INT32_MAX)
        return fail(SIA_ERR_UNSUPPORTED, "max_pages %d too large", pt->max_pages);
    return SIA_OK;
}

int check_queries(const sia_queries* qs, const sia_page_table* pt) {
    if (!qs) return fail(SIA_ERR_INVALID_ARG, "query descriptor is NULL");
    if (qs->num_q < 0) return fail(SIA_ERR_INVALID_ARG, "num_q %d < 0", qs->num_q);
    if (qs->num_q > 0 && (!qs->q_seq || !qs->q_pos)) return fail(SIA_ERR_INVALID_ARG, "q_seq/q_pos is NULL");
    if (qs->group < 1) return fail(SIA_ERR_INVALID_ARG, "group %d < 1", qs->group);
    if (qs->max_visible < 0) return fail(SIA_ERR_INVALID_ARG, "max_visible %d < 0", qs->max_visible);
    if (pt && (int64_t)qs->max_visible > (int64_t)pt->max_pages * 64)
        return fail(SIA_ERR_INVALID_ARG, "max_visible %d exceeds max_pages*64 = %lld", qs->max_visible,
                    (long long)pt->max_pages * 64);
    return SIA_OK;
}

int check_index_cache(const sia_paged_cache* c) {
    if (!c) return fail(SIA_ERR_INVALID_ARG, "index cache descriptor is NULL");
    if (!c->rows) return fail(SIA_ERR_INVALID_ARG, "index cache rows is NULL");
    if (c->num_pages < 1) return fail(SIA_ERR_INVALID_ARG, "num_pages %lld < 1", (long long)c->num_pages);
    if (c->dtype != SIA_BF16 && c->dtype != SIA_FP8_E4M3FN && c->dtype != SIA_MXFP8_E4M3)
        return fail(SIA_ERR_UNSUPPORTED, "index cache dtype %d", c->dtype);
    if (c->dim != 64 && c->dim != 128) return fail(SIA_ERR_UNSUPPORTED, "index dim %d: supported 64, 128", c->dim);
    if (c->dtype == SIA_MXFP8_E4M3 && c->dim != 128)
        return fail(SIA_ERR_UNSUPPORTED, "MXFP8 index dim %d: supported 128", c->dim);
    if (c->dtype != SIA_BF16 && !c->scale) return fail(SIA_ERR_INVALID_ARG, "an fp8 index cache needs its scales");
    if (c->dtype == SIA_BF16 && c->scale) return fail(SIA_ERR_INVALID_ARG, "bf16 index cache takes no scale");
    return SIA_OK;
}

// ------------------------------------------------------------ indexer plan

struct IndexerPlan {
    bool stream = false;
    int group = 1;               // queries per score-pass workgroup (1 or 2)
    int part = 0, n_parts = 0;   // score-pass parts of each row
    int n_reg = 0;               // candidate regions per query
    int64_t ld = 0;              // row stride of the candidate and key rows
    size_t keys = 0, ckey = 0, cpos = 0, hist = 0, reg = 0, rlen = 0;   // workspace offsets
    size_t sbuf = 0;             // stream candidate buffers
    int cap = 0;                 // stream buffer capacity
    size_t total = kHeader;
};

// Score pass + selection pass. One score workgroup is resident per CU, so a row
// is cut into enough parts to give every CU one (parts of 2048 to 65536
// positions); each part has `regs_per_part` candidate regions (one per team or
// wave of the score pass). The selection pass reads the candidate regions and
// the per-part histograms; the dense key rows are its scratch for rows whose
// candidates do not fit in LDS. Every row holds room for all of its positions
// plus a spare tail of 64 entries that non-keeping lanes write to.
void plan_rows(IndexerPlan& p, int64_t num_q, int max_visible, int group, int regs_per_part) {
    p.group = group;
    const int64_t n_groups = std::max<int64_t>(1, ceil_div(num_q, group));
    const int64_t mv = std::max(max_visible, 1);
    const int forced = env_int("SIA_ROWS_PARTS", 0);
    int64_t np = forced > 0 ? forced : std::max<int64_t>(1, ceil_div(device_cus(), n_groups));
    if (forced <= 0) np = std::min<int64_t>(np, std::max<int64_t>(1, ceil_div(mv, 2048)));
    // (a pair part keeps 16-bit histogram counters: at most 32768 positions)
    const int64_t max_part = group == 2 ? 32768 : 64 * (int64_t)sia::kMaxPartPages;
    np = std::max<int64_t>(np, ceil_div(mv, max_part));
    p.part = (int)(ceil_div(ceil_div(mv, np), 64) * 64);
    p.n_parts = (int)ceil_div(mv, p.part);
    p.n_reg = p.n_parts * regs_per_part;
    p.ld = ceil_div(mv, 64) * 64 + 64;
    const size_t row_bytes = align_up((size_t)num_q * p.ld * 4);
    p.keys = p.total; p.total += row_bytes;
    p.ckey = p.total; p.total += row_bytes;
    p.cpos = p.total; p.total += row_bytes;
    p.hist = p.total; p.total += align_up((size_t)num_q * p.n_parts * sia::kCoarseBinsHost * 4);
    p.reg = p.total; p.total += align_up((size_t)num_q * p.n_reg * 8);
    p.rlen = p.total; p.total += align_up((size_t)num_q * 4);
}

// The pair kernel scores two queries of one sequence per workgroup; it needs
// the queries to come in pairs (group even) and an even count.
int score_group(const sia_queries* qs) {
    int g = qs->group % 2 == 0 && qs->num_q % 2 == 0 ? 2 : 1;
    if (env_int("SIA_ROWS_GROUP", 0) == 1) g = 1;
    return g;
}

IndexerPlan plan_indexer(const sia_queries* qs, int topk, int heads, int dim, bool eight_bit) {
    IndexerPlan p;
    const int mode = env_int("SIA_INDEXER_PATH", 0);   // 0 auto, 1 score + select passes, 2 stream
    const bool stream_ok = topk <= 2048 && qs->group % 4 == 0;
    bool stream = stream_ok && qs->num_q >= 256 && qs->max_visible > 2 * topk;
    if (mode == 1) stream = false;
    if (mode == 2) stream = stream_ok;
    if (stream && sia::indexer_stream_smem(qs->max_visible, dim, eight_bit) + 64 <= sia::kMaxLds) {
        // LDS holds the K ring, the staged page ids and the selection scratch;
        // each wave of the persistent grid (at most kStreamBlocksPerCu
        // workgroups per CU) has a candidate buffer of cap keys and positions
        // (+ a spare entry per lane) in the workspace
        p.stream = true;
        p.cap = std::min(4096, std::max(1024, 2 * topk));
        const int64_t waves = (int64_t)sia::kStreamBlocksPerCu * device_cus() * (sia::kStreamThreads / 64);
        p.sbuf = p.total;
        p.total += align_up((size_t)waves * 2 * (p.cap + 64) * 4);
        return p;
    }
    (void)heads;
    const int g = score_group(qs);
    plan_rows(p, qs->num_q, qs->max_visible, g, g == 2 ? sia::kPairRegions : sia::kRowsRegions);
    return p;
}

// The query of one indexer call: bf16 heads, or MXFP8 codes and block scales.
struct IdxQueryIn {
    const void* bf16 = nullptr;
    const uint8_t* codes = nullptr;
    const uint8_t* scales = nullptr;
};

sia::IdxArgs idx_args(const sia_page_table* pt, const sia_paged_cache* c, const sia_queries* qs,
                      const IdxQueryIn& qin, const float* w, int heads, void* ws) {
    sia::IdxArgs a;
    a.page_table = pt->page_table;
    a.seq_lens = pt->seq_lens;
    a.batch = pt->batch;
    a.max_pages = pt->max_pages;
    a.rows = static_cast<const uint8_t*>(c->rows);
    a.scale = static_cast<const float*>(c->scale);
    a.num_pages = c->num_pages;
    a.q_seq = qs->q_seq;
    a.q_pos = qs->q_pos;
    a.num_q = qs->num_q;
    a.max_visible = qs->max_visible;
    a.q_idx = static_cast<const uint16_t*>(qin.bf16);
    a.q8 = qin.codes;
    a.q8s = qin.scales;
    a.w = w;
    a.heads = heads;
    a.status = static_cast<uint32_t*>(ws);
    return a;
}

int check_workspace(void* ws, size_t have, size_t need) {
    if (!ws) return fail(SIA_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
    if (have < need) return fail(SIA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", have, need);
    if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(SIA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    return SIA_OK;
}

int check_indexer_common(const sia_page_table* pt, const sia_paged_cache* c, const sia_queries* qs,
                         const IdxQueryIn& qin, const float* w, int heads) {
    int rc;
    if ((rc = check_page_table(pt)) != SIA_OK) return rc;
    if ((rc = check_index_cache(c)) != SIA_OK) return rc;
    if ((rc = check_queries(qs, pt)) != SIA_OK) return rc;
    if (heads < 1 || heads > 64) return fail(SIA_ERR_UNSUPPORTED, "indexer heads %d: supported 1..64", heads);
    const bool mx = c->dtype == SIA_MXFP8_E4M3;
    if (mx && qin.bf16) return fail(SIA_ERR_INVALID_ARG, "an MXFP8 index cache takes an MXFP8 query (the _mxfp8 calls)");
    if (!mx && qin.codes) return fail(SIA_ERR_INVALID_ARG, "an MXFP8 query needs an MXFP8 index cache");
    if (qs->num_q > 0 && !w) return fail(SIA_ERR_INVALID_ARG, "w is NULL");
    if (qs->num_q > 0 && !mx && !qin.bf16) return fail(SIA_ERR_INVALID_ARG, "q_idx is NULL");
    if (qs->num_q > 0 && mx && (!qin.codes || !qin.scales))
        return fail(SIA_ERR_INVALID_ARG, "q_codes/q_scales is NULL");
    return SIA_OK;
}

}  // namespace

extern "C" {

size_t sia_indexer_workspace_size(const sia_page_table* pt, const sia_paged_cache* index_k,
                                  const sia_queries* qs, int32_t heads, int32_t topk) {
    if (check_page_table(pt) != SIA_OK || check_index_cache(index_k) != SIA_OK ||
        check_queries(qs, pt) != SIA_OK || heads < 1 || heads > 64 || topk < 1 || topk > 8192)
        return 0;
    return plan_indexer(qs, topk, heads, index_k->dim, index_k->dtype != SIA_BF16).total;
}

}  // extern "C"

namespace {

int indexer_topk(const sia_page_table* pt, const sia_paged_cache* index_k, const sia_queries* qs,
                 const IdxQueryIn& qin, const float* w, int32_t heads, int32_t topk, int32_t* out_idx,
                 float* out_score, int32_t sched, void* workspace, size_t workspace_bytes, void* stream,
                 uint64_t* trace, int32_t trace_cap) {
    int rc = check_indexer_common(pt, index_k, qs, qin, w, heads);
    if (rc != SIA_OK) return rc;
    if (topk < 1 || topk > 8192) return fail(SIA_ERR_UNSUPPORTED, "topk %d: supported 1..8192", topk);
    if (qs->num_q > 0 && !out_idx) return fail(SIA_ERR_INVALID_ARG, "out_idx is NULL");
    if (sched < -1 || sched > 2) return fail(SIA_ERR_INVALID_ARG, "sched %d", sched);
    const IndexerPlan p = plan_indexer(qs, topk, heads, index_k->dim, index_k->dtype != SIA_BF16);
    if ((rc = check_workspace(workspace, workspace_bytes, p.total)) != SIA_OK) return rc;
    if (qs->num_q == 0) return SIA_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    const sia::IdxArgs a = idx_args(pt, index_k, qs, qin, w, heads, workspace);
    const int mb = heads > 32 ? 2 : 1;
    const int kf = index_k->dtype;   // (sia_dtype values are the kernels' row formats)
    hipError_t e;
    if (p.stream) {
        sia::StreamArgs s;
        s.topk = topk;
        s.cap = p.cap;
        s.n_tiles = (int)ceil_div(qs->num_q, sia::kStreamThreads / 64);
        s.sched = sched < 0 ? env_int("SIA_SCHED", 1) : sched;
        if (s.sched < 0 || s.sched > 2) s.sched = 1;
        s.counter = reinterpret_cast<uint32_t*>(ws + 4);
        s.buf = reinterpret_cast<uint32_t*>(ws + p.sbuf);
        s.out_idx = out_idx;
        s.out_score = out_score;
        s.trace = trace;
        s.trace_cap = trace ? trace_cap : 0;
        // persistent workgroups, all resident, pulling work items from the counter
        e = sia::launch_fill_u32(s.counter, 0u, 1, st);
        if (e != hipSuccess) return hip_fail(e, "counter reset");
        const int items = s.sched == 2 ? sia::zigzag_workers(s.n_tiles) : s.n_tiles;
        const int occ = std::min(sia::kStreamBlocksPerCu,
                                 sia::indexer_stream_blocks_per_cu(mb, index_k->dim, kf, qs->max_visible));
        const int grid = (int)std::min<int64_t>(items, (int64_t)occ * device_cus());
        e = sia::launch_indexer_stream(a, s, mb, index_k->dim, kf, grid, st);
        if (e != hipSuccess) return hip_fail(e, "indexer stream launch");
        return SIA_OK;
    }
    sia::RowsArgs r{};
    r.part = p.part;
    r.n_parts = p.n_parts;
    r.topk = topk;
    r.n_reg = p.n_reg;
    r.ld = p.ld;
    r.cand_key = reinterpret_cast<uint32_t*>(ws + p.ckey);
    r.cand_pos = reinterpret_cast<int32_t*>(ws + p.cpos);
    r.reg = reinterpret_cast<int2*>(ws + p.reg);
    r.hist = reinterpret_cast<uint32_t*>(ws + p.hist);
    r.row_len = reinterpret_cast<int32_t*>(ws + p.rlen);
    e = sia::launch_indexer_rows(a, r, mb, index_k->dim, kf, p.group, false, st);
    if (e != hipSuccess) return hip_fail(e, "indexer score launch");
    const sia::SelectArgs sel{r.cand_key, r.cand_pos, r.reg, r.n_reg, r.ld,
                              reinterpret_cast<uint32_t*>(ws + p.keys), r.hist, r.n_parts, r.row_len,
                              qs->max_visible, qs->num_q, topk, out_idx, out_score};
    e = sia::launch_topk_rows(sel, st);
    if (e != hipSuccess) return hip_fail(e, "top-k selection launch");
    return SIA_OK;
}

}  // namespace

extern "C" {

int sparse_indexer_topk(const sia_page_table* pt, const sia_paged_cache* index_k, const sia_queries* qs,
                        const void* q_idx, const float* w, int32_t heads, int32_t topk,
                        int32_t* out_idx, float* out_score, int32_t sched, void* workspace,
                        size_t workspace_bytes, void* stream) {
    IdxQueryIn qin;
    qin.bf16 = q_idx;
    return indexer_topk(pt, index_k, qs, qin, w, heads, topk, out_idx, out_score, sched, workspace,
                        workspace_bytes, stream, nullptr, 0);
}

int sparse_indexer_topk_mxfp8(const sia_page_table* pt, const sia_paged_cache* index_k, const sia_queries* qs,
                              const uint8_t* q_codes, const uint8_t* q_scales, const float* w, int32_t heads,
                              int32_t topk, int32_t* out_idx, float* out_score, int32_t sched, void* workspace,
                              size_t workspace_bytes, void* stream) {
    IdxQueryIn qin;
    qin.codes = q_codes;
    qin.scales = q_scales;
    if (index_k && index_k->dtype != SIA_MXFP8_E4M3)
        return fail(SIA_ERR_INVALID_ARG, "sparse_indexer_topk_mxfp8 needs an MXFP8 index cache");
    return indexer_topk(pt, index_k, qs, qin, w, heads, topk, out_idx, out_score, sched, workspace,
                        workspace_bytes, stream, nullptr, 0);
}

int sparse_indexer_topk_traced(const sia_page_table* pt, const sia_paged_cache* index_k, const sia_queries* qs,
                               const void* q_idx, const float* w, int32_t heads, int32_t topk,
                               int32_t* out_idx, float* out_score, int32_t sched, void* workspace,
                               size_t workspace_bytes, void* stream, uint64_t* wg_trace, int32_t trace_cap) {
    if (!wg_trace || trace_cap < 1) return fail(SIA_ERR_INVALID_ARG, "wg_trace is NULL or trace_cap < 1");
    IdxQueryIn qin;
    qin.bf16 = q_idx;
    return indexer_topk(pt, index_k, qs, qin, w, heads, topk, out_idx, out_score, sched, workspace,
                        workspace_bytes, stream, wg_trace, trace_cap);
}

}  // extern "C"

namespace {

int indexer_scores(const sia_page_table* pt, const sia_paged_cache* index_k, const sia_queries* qs,
                   const IdxQueryIn& qin, const float* w, int32_t heads, float* scores, int64_t ld,
                   void* workspace, size_t workspace_bytes, void* stream) {
    int rc = check_indexer_common(pt, index_k, qs, qin, w, heads);
    if (rc != SIA_OK) return rc;
    if (qs->num_q > 0 && !scores) return fail(SIA_ERR_INVALID_ARG, "scores is NULL");
    if (ld < std::max(1, qs->max_visible)) return fail(SIA_ERR_INVALID_ARG, "ld %lld < max_visible %d", (long long)ld, qs->max_visible);
    if ((rc = check_workspace(workspace, workspace_bytes, kHeader)) != SIA_OK) return rc;
    if (qs->num_q == 0) return SIA_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = sia::launch_fill_u32(reinterpret_cast<uint32_t*>(scores), 0xff800000u,
                                        (int64_t)qs->num_q * ld, st);
    if (e != hipSuccess) return hip_fail(e, "scores fill");
    const sia::IdxArgs a = idx_args(pt, index_k, qs, qin, w, heads, workspace);
    IndexerPlan p;
    const int g = score_group(qs);
    plan_rows(p, qs->num_q, qs->max_visible, g, 1);
    sia::RowsArgs r{};
    r.part = p.part;
    r.n_parts = p.n_parts;
    r.ld = ld;
    r.scores = scores;
    e = sia::launch_indexer_rows(a, r, heads > 32 ? 2 : 1, index_k->dim, index_k->dtype, p.group, true, st);
    if (e != hipSuccess) return hip_fail(e, "indexer scores launch");
    return SIA_OK;
}

}  // namespace

extern "C" {

int sparse_indexer_scores(const sia_page_table* pt, const sia_paged_cache* index_k, const sia_queries* qs,
                          const void* q_idx, const float* w, int32_t heads, float* scores, int64_t ld,
                          void* workspace, size_t workspace_bytes, void* stream) {
    IdxQueryIn qin;
    qin.bf16 = q_idx;
    return indexer_scores(pt, index_k, qs, qin, w, heads, scores, ld, workspace, workspace_bytes, stream);
}

int sparse_indexer_scores_mxfp8(const sia_page_table* pt, const sia_paged_cache* index_k, const sia_queries* qs,
                                const uint8_t* q_codes, const uint8_t* q_scales, const float* w, int32_t heads,
                                float* scores, int64_t ld, void* workspace, size_t workspace_bytes, void* stream) {
    IdxQueryIn qin;
    qin.codes = q_codes;
    qin.scales = q_scales;
    if (index_k && index_k->dtype != SIA_MXFP8_E4M3)
        return fail(SIA_ERR_INVALID_ARG, "sparse_indexer_scores_mxfp8 needs an MXFP8 index cache");
    return indexer_scores(pt, index_k, qs, qin, w, heads, scores, ld, workspace, workspace_bytes, stream);
}

int sia_quantize_mxfp8(const void* x, int64_t rows, int32_t dim, uint8_t* codes, uint8_t* scales, void* stream) {
    if (rows < 0) return fail(SIA_ERR_INVALID_ARG, "rows %lld < 0", (long long)rows);
    if (dim < 32 || dim % 32) return fail(SIA_ERR_UNSUPPORTED, "dim %d: a positive multiple of 32", dim);
    if (rows > 0 && (!x || !codes || !scales)) return fail(SIA_ERR_INVALID_ARG, "x/codes/scales is NULL");
    if (rows == 0) return SIA_OK;
    hipError_t e = sia::launch_quantize_mxfp8(static_cast<const uint16_t*>(x), rows * (dim / 32), codes, scales,
                                              static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SIA_OK : hip_fail(e, "quantize launch");
}

size_t sia_topk_workspace_size(int32_t num_q, int32_t max_row_len, int32_t topk) {
    if (num_q < 0 || max_row_len < 0 || topk < 1 || topk > 8192) return 0;
    IndexerPlan p;
    plan_rows(p, num_q, max_row_len, 1, 1);
    return p.total;
}

int sparse_topk_from_scores(const float* scores, int64_t ld, const int32_t* row_len, int32_t num_q,
                            int32_t max_row_len, int32_t topk, int32_t* out_idx, float* out_score,
                            void* workspace, size_t workspace_bytes, void* stream) {
    if (num_q < 0) return fail(SIA_ERR_INVALID_ARG, "num_q %d < 0", num_q);
    if (num_q > 0 && (!scores || !row_len || !out_idx)) return fail(SIA_ERR_INVALID_ARG, "NULL pointer");
    if (topk < 1 || topk > 8192) return fail(SIA_ERR_UNSUPPORTED, "topk %d: supported 1..8192", topk);
    if (max_row_len < 0 || ld < max_row_len) return fail(SIA_ERR_INVALID_ARG, "need 0 <= max_row_len <= ld");
    IndexerPlan p;
    plan_rows(p, num_q, max_row_len, 1, 1);
    int rc = check_workspace(workspace, workspace_bytes, p.total);
    if (rc != SIA_OK) return rc;
    if (num_q == 0) return SIA_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    sia::KeysFromScoresArgs k{};
    k.scores = scores;
    k.ld_in = ld;
    k.row_len = row_len;
    k.num_q = num_q;
    k.max_len = max_row_len;
    k.part = p.part;
    k.n_parts = p.n_parts;
    k.ld = p.ld;
    k.cand_key = reinterpret_cast<uint32_t*>(ws + p.ckey);
    k.cand_pos = reinterpret_cast<int32_t*>(ws + p.cpos);
    k.reg = reinterpret_cast<int2*>(ws + p.reg);
    k.hist = reinterpret_cast<uint32_t*>(ws + p.hist);
    k.status = reinterpret_cast<uint32_t*>(ws);
    hipError_t e = sia::launch_keys_from_scores(k, st);
    if (e != hipSuccess) return hip_fail(e, "score keys launch");
    const sia::SelectArgs sel{k.cand_key, k.cand_pos, k.reg, p.n_reg, k.ld, reinterpret_cast<uint32_t*>(ws + p.keys),
                              k.hist, k.n_parts, row_len, max_row_len, num_q, topk, out_idx, out_score};
    e = sia::launch_topk_rows(sel, st);
    if (e != hipSuccess) return hip_fail(e, "top-k selection launch");
    return SIA_OK;
}

// ------------------------------------------------------------ input preparation

}  // extern "C"

namespace {

struct PrepPlan {
    int sq = 1, sk = 1, sw = 1;                   // K slices per projection
    size_t pq = 0, pk = 0, pw = 0, qb = 0;       // workspace offsets
    size_t total = kHeader;
};

// K slices: enough workgroups (64 x 64 tiles x slices) for about two per CU,
// each slice at least 256 wide and a multiple of 16.
int prep_slices(int64_t M, int64_t N, int64_t K) {
    const int64_t tiles = ceil_div(M, 64) * ceil_div(N, 64);
    int64_t sl = ceil_div(2 * (int64_t)device_cus(), tiles);
    sl = std::max<int64_t>(1, std::min<int64_t>(sl, K / 256));
    return (int)sl;
}
int64_t slice_width(int64_t K, int slices) { return ceil_div(ceil_div(K, slices), 16) * 16; }

PrepPlan plan_prepare(const sia_indexer_weights* W, int64_t M) {
    PrepPlan p;
    const int64_t nq = (int64_t)W->heads * W->dim;
    p.sq = prep_slices(M, nq, W->dq);
    p.sk = prep_slices(M, W->dim, W->dh);
    p.sw = prep_slices(M, W->heads, W->dh);
    p.pq = p.total; p.total += align_up((size_t)p.sq * M * nq * 4);
    p.pk = p.total; p.total += align_up((size_t)p.sk * M * W->dim * 4);
    p.pw = p.total; p.total += align_up((size_t)p.sw * M * W->heads * 4);
    p.qb = p.total; p.total += align_up((size_t)M * nq * 2);
    return p;
}

int check_prepare_weights(const sia_indexer_weights* W) {
    if (!W) return fail(SIA_ERR_INVALID_ARG, "weights descriptor is NULL");
    if (!W->wq || !W->wk || !W->ww || !W->k_gamma || !W->k_beta)
        return fail(SIA_ERR_INVALID_ARG, "a projection weight is NULL");
    if (W->dim != 128) return fail(SIA_ERR_UNSUPPORTED, "index dim %d: supported 128", W->dim);
    if (W->heads < 1 || W->heads > 64) return fail(SIA_ERR_UNSUPPORTED, "indexer heads %d: supported 1..64", W->heads);
    if (W->dq < 16 || W->dq % 16 || W->dh < 16 || W->dh % 16)
        return fail(SIA_ERR_UNSUPPORTED, "input widths %d, %d: positive multiples of 16", W->dq, W->dh);
    if (!(W->eps >= 0.f) || !std::isfinite(W->eps)) return fail(SIA_ERR_INVALID_ARG, "eps %g", (double)W->eps);
    return SIA_OK;
}

}  // namespace

extern "C" {

size_t sia_indexer_prepare_workspace_size(const sia_indexer_weights* W, int32_t num_q) {
    if (num_q < 0 || check_prepare_weights(W) != SIA_OK) return 0;
    return plan_prepare(W, num_q).total;
}

int sia_indexer_prepare(const sia_indexer_weights* W, const void* xq, const void* xh, const sia_page_table* pt,
                        const sia_paged_cache* index_k, const sia_queries* qs, uint8_t* q_codes, uint8_t* q_scales,
                        float* w_out, void* q_bf16, void* k_bf16, void* workspace, size_t workspace_bytes,
                        void* const* streams, void* const* events) {
    int rc;
    if ((rc = check_prepare_weights(W)) != SIA_OK) return rc;
    if ((rc = check_page_table(pt)) != SIA_OK) return rc;
    if ((rc = check_index_cache(index_k)) != SIA_OK) return rc;
    if (index_k->dtype != SIA_MXFP8_E4M3) return fail(SIA_ERR_UNSUPPORTED, "the prepared keys are MXFP8 index rows");
    if (!qs || qs->num_q < 0) return fail(SIA_ERR_INVALID_ARG, "query descriptor");
    if (!streams || !events) return fail(SIA_ERR_INVALID_ARG, "streams/events is NULL");
    if (!events[0] || !events[1] || !events[2]) return fail(SIA_ERR_INVALID_ARG, "an event is NULL");
    const int64_t M = qs->num_q;
    if (M > 0 && (!qs->q_seq || !qs->q_pos || !xq || !xh || !q_codes || !q_scales || !w_out))
        return fail(SIA_ERR_INVALID_ARG, "an input or output is NULL");
    const PrepPlan p = plan_prepare(W, M);
    if ((rc = check_workspace(workspace, workspace_bytes, p.total)) != SIA_OK) return rc;
    if (M == 0) return SIA_OK;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    hipStream_t s0 = static_cast<hipStream_t>(streams[0]), s1 = static_cast<hipStream_t>(streams[1]),
                s2 = static_cast<hipStream_t>(streams[2]);
    hipEvent_t e0 = static_cast<hipEvent_t>(events[0]), e1 = static_cast<hipEvent_t>(events[1]),
               e2 = static_cast<hipEvent_t>(events[2]);
    hipError_t e;
    // fork
    if ((e = hipEventRecord(e0, s0)) != hipSuccess) return hip_fail(e, "fork event");
    if ((e = hipStreamWaitEvent(s1, e0, 0)) != hipSuccess) return hip_fail(e, "fork wait");
    if ((e = hipStreamWaitEvent(s2, e0, 0)) != hipSuccess) return hip_fail(e, "fork wait");
    const int64_t nq = (int64_t)W->heads * W->dim;
    // chain 1: query projection, then MXFP8
    {
        sia::GemmArgs g{static_cast<const uint16_t*>(xq), static_cast<const uint16_t*>(W->wq),
                        reinterpret_cast<float*>(ws + p.pq), (int32_t)M, (int32_t)nq, W->dq,
                        (int32_t)slice_width(W->dq, p.sq)};
        if ((e = sia::launch_proj_gemm(g, s0)) != hipSuccess) return hip_fail(e, "query projection");
        uint16_t* qb = q_bf16 ? static_cast<uint16_t*>(q_bf16) : reinterpret_cast<uint16_t*>(ws + p.qb);
        if ((e = sia::launch_proj_reduce(g.part, (int)ceil_div(W->dq, g.k_slice), M * nq, qb, nullptr, s0)) != hipSuccess)
            return hip_fail(e, "query reduce");
        if ((e = sia::launch_quantize_mxfp8(qb, M * nq / 32, q_codes, q_scales, s0)) != hipSuccess)
            return hip_fail(e, "query quantize");
    }
    // chain 2: key projection, LayerNorm, MXFP8, cache rows
    {
        sia::GemmArgs g{static_cast<const uint16_t*>(xh), static_cast<const uint16_t*>(W->wk),
                        reinterpret_cast<float*>(ws + p.pk), (int32_t)M, W->dim, W->dh,
                        (int32_t)slice_width(W->dh, p.sk)};
        if ((e = sia::launch_proj_gemm(g, s1)) != hipSuccess) return hip_fail(e, "key projection");
        sia::KeyPrepArgs k{};
        k.part = g.part;
        k.splits = (int)ceil_div(W->dh, g.k_slice);
        k.M = (int32_t)M;
        k.eps = W->eps;
        k.gamma = W->k_gamma;
        k.beta = W->k_beta;
        k.k_out = static_cast<uint16_t*>(k_bf16);
        k.q_seq = qs->q_seq;
        k.q_pos = qs->q_pos;
        k.page_table = pt->page_table;
        k.batch = pt->batch;
        k.max_pages = pt->max_pages;
        k.num_pages = index_k->num_pages;
        k.codes = static_cast<uint8_t*>(const_cast<void*>(index_k->rows));
        k.scales = static_cast<uint8_t*>(const_cast<void*>(index_k->scale));
        k.status = reinterpret_cast<uint32_t*>(ws);
        if ((e = sia::launch_key_norm_quant(k, s1)) != hipSuccess) return hip_fail(e, "key normalize");
    }
    // chain 3: head-weight projection
    {
        sia::GemmArgs g{static_cast<const uint16_t*>(xh), static_cast<const uint16_t*>(W->ww),
                        reinterpret_cast<float*>(ws + p.pw), (int32_t)M, W->heads, W->dh,
                        (int32_t)slice_width(W->dh, p.sw)};
        if ((e = sia::launch_proj_gemm(g, s2)) != hipSuccess) return hip_fail(e, "weight projection");
        if ((e = sia::launch_proj_reduce(g.part, (int)ceil_div(W->dh, g.k_slice), M * W->heads, nullptr, w_out, s2)) !=
            hipSuccess)
            return hip_fail(e, "weight reduce");
    }
    // join
    if ((e = hipEventRecord(e1, s1)) != hipSuccess) return hip_fail(e, "join event");
    if ((e = hipEventRecord(e2, s2)) != hipSuccess) return hip_fail(e, "join event");
    if ((e = hipStreamWaitEvent(s0, e1, 0)) != hipSuccess) return hip_fail(e, "join wait");
    if ((e = hipStreamWaitEvent(s0, e2, 0)) != hipSuccess) return hip_fail(e, "join wait");
    return SIA_OK;
}

// ------------------------------------------------------------ attention

static int attn_plan(const sia_queries* qs, int heads, int topk, int& hb, int& n_split, int& rows_per_split,
                     size_t& total) {
    // bf16 rows take the whole-tile kernel (SIA_ATTN_WAVE=0 selects the
    // row-split one): 128 heads per workgroup where that alone gives every CU a
    // workgroup (each selected row is then gathered once per query), else 64
    int hb_max = 64;
    if (env_int("SIA_ATTN_WAVE", 1)) {
        const int forced = env_int("SIA_ATTN_HB", 0);
        if (forced > 0) hb_max = forced >= 128 ? 128 : 64;
        else if (heads % 128 == 0 && (int64_t)qs->num_q * (heads / 128) >= device_cus()) hb_max = 128;
    }
    hb = heads % hb_max == 0 ? hb_max : heads % 64 == 0 ? 64 : heads % 32 == 0 ? 32 : 16;
    const int64_t base = (int64_t)qs->num_q * (heads / hb);
    // one workgroup per CU is resident (LDS); split the rows only as far as it
    // takes to give every CU one, keeping at least two tiles per slice and at
    // most the slice length the kernel's row list holds
    int ns = env_int("SIA_ATTN_SPLIT", 0);
    if (ns <= 0) ns = (int)std::max<int64_t>(1, ceil_div(256, std::max<int64_t>(1, base)));
    const int max_split = std::max(1, (int)ceil_div(topk, 64));
    const int min_split = (int)ceil_div(topk, sia::kAttnMaxSliceRows);
    ns = std::max(min_split, std::min(ns, max_split));
    rows_per_split = (int)ceil_div(ceil_div(topk, ns), 32) * 32;
    n_split = (int)ceil_div(topk, rows_per_split);
    total = kHeader;
    if (n_split > 1) {
        total += align_up((size_t)qs->num_q * n_split * heads * 512 * 4);
        total += align_up((size_t)qs->num_q * n_split * heads * 4);
    }
    return SIA_OK;
}

static int check_attn(const sia_page_table* pt, const sia_paged_cache* kv, const sia_queries* qs, int heads,
                      int d_v, int topk) {
    int rc;
    if ((rc = check_page_table(pt)) != SIA_OK) return rc;
    if (!kv || !kv->rows) return fail(SIA_ERR_INVALID_ARG, "kv cache descriptor/rows is NULL");
    if (kv->num_pages < 1) return fail(SIA_ERR_INVALID_ARG, "kv num_pages < 1");
    if (kv->dtype != SIA_BF16 && kv->dtype != SIA_FP8_E4M3FN)
        return fail(SIA_ERR_UNSUPPORTED, "kv dtype %d: bf16 or fp8 e4m3fn rows", kv->dtype);
    if (kv->dim != 576) return fail(SIA_ERR_UNSUPPORTED, "kv dim %d: only 576", kv->dim);
    if (kv->scale) return fail(SIA_ERR_INVALID_ARG, "the latent cache takes no separate scale pool (fp8 rows hold their scales)");
    if (d_v != 512) return fail(SIA_ERR_UNSUPPORTED, "d_v %d: only 512", d_v);
    if (!qs) return fail(SIA_ERR_INVALID_ARG, "query descriptor is NULL");
    if (qs->num_q < 0) return fail(SIA_ERR_INVALID_ARG, "num_q %d < 0", qs->num_q);
    if (qs->num_q > 0 && !qs->q_seq) return fail(SIA_ERR_INVALID_ARG, "q_seq is NULL");
    if (heads < 16 || heads % 16 || heads > 128) return fail(SIA_ERR_UNSUPPORTED, "heads %d: multiple of 16 up to 128", heads);
    if (topk < 1) return fail(SIA_ERR_INVALID_ARG, "topk %d < 1", topk);
    return SIA_OK;
}

size_t sia_mla_workspace_size(const sia_queries* qs, int32_t heads, int32_t d_v, int32_t topk) {
    if (!qs || qs->num_q < 0 || heads < 16 || heads % 16 || heads > 128 || d_v != 512 || topk < 1) return 0;
    int hb, ns, rps;
    size_t total;
    attn_plan(qs, heads, topk, hb, ns, rps, total);
    return total;
}

}  // extern "C"

namespace {

// Launches the attention kernels with workspace `ws` (already checked to hold
// `total` bytes for this plan).
int mla_run(const sia_page_table* pt, const sia_paged_cache* kv, const sia_queries* qs, const void* q,
            int heads, int d_v, const int32_t* idx, int topk, float sm_scale, void* out, float* lse,
            uint8_t* ws, int hb, int ns, int rps, hipStream_t st) {
    sia::AttnArgs a;
    a.page_table = pt->page_table;
    a.seq_lens = pt->seq_lens;
    a.batch = pt->batch;
    a.max_pages = pt->max_pages;
    a.kv = static_cast<const uint16_t*>(kv->rows);
    a.kv8 = kv->dtype == SIA_FP8_E4M3FN;
    a.num_pages = kv->num_pages;
    a.q_seq = qs->q_seq;
    a.num_q = qs->num_q;
    a.q = static_cast<const uint16_t*>(q);
    a.heads = heads;
    a.d_v = d_v;
    a.idx = idx;
    a.topk = topk;
    a.sm_scale = sm_scale;
    a.n_split = ns;
    a.rows_per_split = rps;
    // bf16 rows: the whole-tile kernel where a block is 32 heads or more; fp8
    // rows: the row-split kernel, at most 64 heads per workgroup
    a.wave_heads = !a.kv8 && hb >= 32 && env_int("SIA_ATTN_WAVE", 1) ? 1 : 0;
    if (a.wave_heads && hb <= 64 && env_int("SIA_ATTN_RH", 1) == 2) a.wave_heads = 2;
    if (a.wave_heads && hb == 128 && env_int("SIA_ATTN_WIDE", 1)) a.wave_heads = 3;
    a.heads_per_block = a.kv8 ? std::min(hb, 64) : hb;
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse;
    a.part_o = ns > 1 ? reinterpret_cast<float*>(ws + kHeader) : nullptr;
    a.part_lse = ns > 1 ? reinterpret_cast<float*>(ws + kHeader + align_up((size_t)qs->num_q * ns * heads * 512 * 4))
                        : nullptr;
    a.status = reinterpret_cast<uint32_t*>(ws);
    hipError_t e = sia::launch_sparse_mla(a, st);
    if (e != hipSuccess) return hip_fail(e, "sparse attention launch");
    if (ns > 1) {
        e = sia::launch_mla_combine(a, st);
        if (e != hipSuccess) return hip_fail(e, "attention combine launch");
    }
    return SIA_OK;
}

int check_attn_call(const sia_page_table* pt, const sia_paged_cache* kv, const sia_queries* qs, const void* q,
                    int heads, int d_v, const int32_t* idx, int topk, float sm_scale, void* out) {
    int rc = check_attn(pt, kv, qs, heads, d_v, topk);
    if (rc != SIA_OK) return rc;
    if (qs->num_q > 0 && (!q || !idx || !out)) return fail(SIA_ERR_INVALID_ARG, "q/idx/out is NULL");
    if (!std::isfinite(sm_scale)) return fail(SIA_ERR_INVALID_ARG, "sm_scale is not finite");
    return SIA_OK;
}

// Scratch of sparse_mla_attention_noalloc: one copy per GPU, held until the
// process ends. Host code never uses the symbol's name as an address (on the
// host it is only a stand-in); the device address of each GPU's copy is
// looked up once per device with hipGetSymbolAddress, with that device
// current, and kept in g_scratch.
constexpr size_t kNoAllocScratch = SIA_MLA_NOALLOC_MAX_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch[kMaxDevices] = {};

}  // namespace

static __device__ __attribute__((aligned(256))) uint8_t scratch[kNoAllocScratch];

namespace {

// Device address of the current GPU's scratch (looked up on its first use).
int scratch_of_current_device(uint8_t** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(SIA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "scratch address");
        if (!p || reinterpret_cast<uintptr_t>(p) % 256) return fail(SIA_ERR_HIP, "scratch address is not 256-byte aligned");
        g_scratch[dev] = static_cast<uint8_t*>(p);
    }
    *out = g_scratch[dev];
    return SIA_OK;
}

}  // namespace

extern "C" {

int sparse_mla_attention(const sia_page_table* pt, const sia_paged_cache* kv, const sia_queries* qs,
                         const void* q, int32_t heads, int32_t d_v, const int32_t* idx, int32_t topk,
                         float sm_scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                         void* stream) {
    int rc = check_attn_call(pt, kv, qs, q, heads, d_v, idx, topk, sm_scale, out);
    if (rc != SIA_OK) return rc;
    int hb, ns, rps;
    size_t total;
    attn_plan(qs, heads, topk, hb, ns, rps, total);
    if ((rc = check_workspace(workspace, workspace_bytes, total)) != SIA_OK) return rc;
    if (qs->num_q == 0) return SIA_OK;
    return mla_run(pt, kv, qs, q, heads, d_v, idx, topk, sm_scale, out, lse, static_cast<uint8_t*>(workspace),
                   hb, ns, rps, static_cast<hipStream_t>(stream));
}

int sparse_mla_attention_noalloc(const sia_page_table* pt, const sia_paged_cache* kv, const sia_queries* qs,
                                 const void* q, int32_t heads, int32_t d_v, const int32_t* idx, int32_t topk,
                                 float sm_scale, void* out, float* lse, void* stream) {
    int rc = check_attn_call(pt, kv, qs, q, heads, d_v, idx, topk, sm_scale, out);
    if (rc != SIA_OK) return rc;
    int hb, ns, rps;
    size_t total;
    attn_plan(qs, heads, topk, hb, ns, rps, total);
    if (total > kNoAllocScratch)
        return fail(SIA_ERR_WORKSPACE,
                    "this call needs %zu bytes of scratch; the no-allocation entry point holds %zu "
                    "(use sparse_mla_attention with a workspace)", total, kNoAllocScratch);
    if (qs->num_q == 0) return SIA_OK;
    uint8_t* ws = nullptr;
    if ((rc = scratch_of_current_device(&ws)) != SIA_OK) return rc;
    return mla_run(pt, kv, qs, q, heads, d_v, idx, topk, sm_scale, out, lse, ws, hb, ns, rps,
                   static_cast<hipStream_t>(stream));
}

// ------------------------------------------------------------ misc

int sia_zigzag_assign(int32_t num_shards, int32_t* out) {
    if (num_shards < 1 || !out) return fail(SIA_ERR_INVALID_ARG, "num_shards %d / out", num_shards);
    const int workers = sia::zigzag_workers(num_shards);
    int k = 0;
    for (int i = 0; i < workers; i++)
        for (int s = 0; s < 2; s++) {
            const int v = sia::zigzag_shard(num_shards, i, s);
            if (v >= 0) out[k++] = v;
        }
    return SIA_OK;
}

int sia_clear_device_status(void* workspace, void* stream) {
    if (!workspace) return fail(SIA_ERR_INVALID_ARG, "workspace is NULL");
    hipError_t e = sia::launch_fill_u32(static_cast<uint32_t*>(workspace), 0u, 2, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SIA_OK : hip_fail(e, "status clear");
}

int sia_read_device_status(const void* workspace, void* stream, uint32_t* status) {
    if (!workspace || !status) return fail(SIA_ERR_INVALID_ARG, "workspace/status is NULL");
    hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "stream synchronize");
    e = hipMemcpy(status, workspace, 4, hipMemcpyDeviceToHost);
    return e == hipSuccess ? SIA_OK : hip_fail(e, "status read");
}

const char* sia_last_error(void) { return g_err.c_str(); }

int sia_version(void) { return 100; }

}  // extern "C"
