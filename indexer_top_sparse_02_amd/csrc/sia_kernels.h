// Launch interface between the host entry points (sia_api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sia {

// Index-row formats: bf16; OCP e4m3 with a per-token fp32 scale; MXFP8 (e4m3
// with one E8M0 scale per 32 elements of a row).
constexpr int kRowBf16 = 0, kRowFp8 = 1, kRowMx = 2;

// Everything the indexer kernels read. Device pointers unless noted.
struct IdxArgs {
    const int32_t* page_table;
    const int32_t* seq_lens;
    int32_t batch, max_pages;
    const uint8_t* rows;       // index-K pool [num_pages, 64, dim]
    const float* scale;        // [num_pages, 64] fp32 (fp8 rows), [num_pages, 64, dim/32] E8M0 bytes
                               // (MXFP8 rows; the same 4 bytes per row at dim 128), or null
    int64_t num_pages;
    const int32_t* q_seq;
    const int32_t* q_pos;
    int32_t num_q;
    int32_t max_visible;       // host bound on visible row length
    const uint16_t* q_idx;     // bf16 [num_q, heads, dim] (bf16 and fp8 rows)
    const uint8_t* q8;         // MXFP8 rows: e4m3 query codes [num_q, heads, dim]
    const uint8_t* q8s;        //             and E8M0 scales [num_q, heads, dim/32]
    const float* w;            // [num_q, heads]
    int32_t heads;
    uint32_t* status;          // device status word
};

// Score pass: a workgroup scores one part (`part` consecutive positions, a
// multiple of the page size) of the rows of one or two queries. A position's
// key is kept only while it reaches the running floor of the part (the coarse
// bin of its K-th largest key so far); kept keys and their positions are
// appended to the candidate list of the team (or wave) that scored them. The
// lists of a query, taken in region order, are in position order.
struct RowsArgs {
    int32_t part, n_parts;
    int32_t topk;
    int32_t n_reg;             // candidate regions per query (n_parts x teams per part)
    int64_t ld;                // row stride of cand_key / cand_pos / keys / scores
    uint32_t* cand_key;        // [num_q, ld] appended keys, region r from reg[r].x on
    int32_t* cand_pos;         // [num_q, ld] their positions
    int2* reg;                 // [num_q, n_reg] (first entry, count) of each region
    uint32_t* hist;            // [num_q, n_parts, kCoarseBins] per-part coarse histograms of kept keys
    int32_t* row_len;          // [num_q] visible row length (written by part 0)
    float* scores;             // scores mode: [num_q, ld]
};

// Candidates (every key, one region per part) and per-part histograms from a
// given score matrix (test hook).
struct KeysFromScoresArgs {
    const float* scores;
    int64_t ld_in;
    const int32_t* row_len;
    int32_t num_q, max_len, part, n_parts;
    int64_t ld;
    uint32_t* cand_key;
    int32_t* cand_pos;
    int2* reg;
    uint32_t* hist;
    uint32_t* status;
};

// Selection pass: exact Top-K of each query's candidate lists. `keys` is a
// dense [num_q, ld] scratch row used only when a row's candidates at the K-th
// coarse bin do not fit in LDS.
struct SelectArgs {
    const uint32_t* cand_key;
    const int32_t* cand_pos;
    const int2* reg;
    int32_t n_reg;
    int64_t ld;
    uint32_t* keys;
    const uint32_t* hist;
    int32_t n_parts;
    const int32_t* row_len;    // clamped to [0, max_len]
    int32_t max_len, num_q, topk;
    int32_t* out_idx;
    float* out_score;
};

struct StreamArgs {
    int32_t topk, cap, n_tiles, sched;
    uint32_t* counter;
    uint32_t* buf;             // candidate buffers: 2 * (cap + 64) words per wave of the grid
    int32_t* out_idx;
    float* out_score;
    uint64_t* trace;           // optional [trace_cap, 4] per-workgroup records (or null)
    int32_t trace_cap;
};

// Launchers; return hipSuccess or the launch error. `mb` = ceil(heads / 32),
// `kf` the index-row format.
hipError_t launch_indexer_rows(const IdxArgs& a, const RowsArgs& r, int mb, int dim, int kf, int group,
                               bool scores_mode, hipStream_t st);
hipError_t launch_keys_from_scores(const KeysFromScoresArgs& k, hipStream_t st);
hipError_t launch_topk_rows(const SelectArgs& s, hipStream_t st);
hipError_t launch_indexer_stream(const IdxArgs& a, const StreamArgs& s, int mb, int dim, int kf,
                                 int grid, hipStream_t st);
int indexer_stream_blocks_per_cu(int mb, int dim, int kf, int max_visible);
size_t indexer_stream_smem(int max_visible, int dim, bool fp8);
constexpr int kStreamBlocksPerCu = 2;   // (the kernel's launch bound)
constexpr size_t kMaxLds = 160 * 1024;
constexpr int kCoarseBinsHost = 2048;   // = kCoarseBins of the selection code
hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t st);
// MXFP8 quantization of n_groups groups of 32 consecutive bf16 values.
hipError_t launch_quantize_mxfp8(const uint16_t* x, int64_t n_groups, uint8_t* codes, uint8_t* scales,
                                 hipStream_t st);

constexpr int kRowsThreads = 512;      // eight waves: two per SIMD
constexpr int kRowsRegions = kRowsThreads / 64;   // candidate regions per part (one per wave)
constexpr int kPairThreads = 512;      // four teams of two waves (one team per SIMD) per query pair
constexpr int kPairRegions = kPairThreads / 128;  // candidate regions per part (one per team)
constexpr int kMaxPartPages = 1024;    // a score-pass part spans at most 65536 positions
constexpr int kSelThreads = 1024;
constexpr int kSelCap = 16384;         // candidates the selection pass holds in LDS
constexpr int kStreamThreads = 256;    // four waves, one query each

// Input preparation: projections out[M, N] = x[M, K] W[N, K]^T as fp32
// partials per K slice ([splits, M, N]), then reductions.
struct GemmArgs {
    const uint16_t* x;        // bf16 [M, K]
    const uint16_t* w;        // bf16 [N, K]
    float* part;              // [splits, M, N]
    int32_t M, N, K, k_slice; // K and k_slice multiples of 16
};
struct KeyPrepArgs {
    const float* part;        // [splits, M, 128] key projection partials
    int32_t splits, M;
    float eps;
    const float* gamma;       // [128]
    const float* beta;        // [128]
    uint16_t* k_out;          // bf16 [M, 128] or null
    const int32_t* q_seq;
    const int32_t* q_pos;
    const int32_t* page_table;
    int32_t batch, max_pages;
    int64_t num_pages;
    uint8_t* codes;           // MXFP8 index cache rows [num_pages, 64, 128]
    uint8_t* scales;          // [num_pages, 64, 4]
    uint32_t* status;
};
hipError_t launch_proj_gemm(const GemmArgs& g, hipStream_t st);
hipError_t launch_proj_reduce(const float* part, int splits, int64_t mn, uint16_t* out_bf16, float* out_f32,
                              hipStream_t st);
hipError_t launch_key_norm_quant(const KeyPrepArgs& k, hipStream_t st);

// Attention.
struct AttnArgs {
    const int32_t* page_table;
    const int32_t* seq_lens;
    int32_t batch, max_pages;
    const uint16_t* kv;       // bf16 [num_pages, 64, 576], or (kv8) 656-byte fp8 rows [num_pages, 64, 656]
    int32_t kv8;
    int64_t num_pages;
    const int32_t* q_seq;
    int32_t num_q;
    const uint16_t* q;        // bf16 [num_q, heads, 576]
    int32_t heads, d_v;
    const int32_t* idx;       // [num_q, topk]
    int32_t topk;
    float sm_scale;
    int32_t n_split, rows_per_split, heads_per_block;
    int32_t wave_heads;       // bf16 rows: 0 = row-split kernel; 1 = one wave per 16 heads over whole
                              // 32-row tiles (P in registers); 2 = two waves per 16 heads, each over
                              // one half of 64-row tiles
    uint16_t* out;            // bf16 [num_q, heads, d_v]  (n_split == 1)
    float* lse;               // [num_q, heads] or null
    float* part_o;            // [num_q, n_split, heads, d_v] fp32 (n_split > 1)
    float* part_lse;          // [num_q, n_split, heads]
    uint32_t* status;
};

hipError_t launch_sparse_mla(const AttnArgs& a, hipStream_t st);
constexpr int kAttnMaxSliceRows = 2048;   // selected rows one attention workgroup takes at most
hipError_t launch_mla_combine(const AttnArgs& a, hipStream_t st);

}  // namespace sia
