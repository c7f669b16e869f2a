// Launch interface between the host entry points (sia_api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sia {

// Everything the indexer kernels read. Device pointers unless noted.
struct IdxArgs {
    const int32_t* page_table;
    const int32_t* seq_lens;
    int32_t batch, max_pages;
    const uint8_t* rows;       // index-K pool [num_pages, 64, dim]
    const float* scale;        // [num_pages, 64] (fp8) or null
    int64_t num_pages;
    const int32_t* q_seq;
    const int32_t* q_pos;
    int32_t num_q;
    int32_t max_visible;       // host bound on visible row length
    const uint16_t* q_idx;     // bf16 [num_q, heads, dim]
    const float* w;            // [num_q, heads]
    int32_t heads;
    uint32_t* status;          // device status word
};

// Split-context pass: a workgroup scores `chunk` positions for `group` queries.
struct SplitArgs {
    int32_t chunk, n_chunks, topk, kc;   // kc = candidates kept per chunk
    int32_t* out_idx;                    // final output when n_chunks == 1
    float* out_score;
    uint32_t* cand_key;                  // [num_q, n_chunks, kc]
    int32_t* cand_pos;
    int32_t* cand_cnt;                   // [num_q, n_chunks]
    float* scores;                       // scores hook: [num_q, ld]
    int64_t ld;
};

// Selection directly from a score matrix (test hook).
struct FromScoresArgs {
    const float* scores;
    int64_t ld;
    const int32_t* row_len;
    int32_t num_q;
    uint32_t* status;
};

struct MergeArgs {
    int32_t num_q, n_in, kc_in, fan_in, n_out, topk;
    const uint32_t* in_key;
    const int32_t* in_pos;
    const int32_t* in_cnt;
    uint32_t* out_key;      // intermediate level (capacity topk per set)
    int32_t* out_pos;
    int32_t* out_cnt;
    int32_t* out_idx;       // final level
    float* out_score;
};

struct StreamArgs {
    int32_t topk, cap, n_tiles, sched;
    uint32_t* counter;
    int32_t* out_idx;
    float* out_score;
};

// Launchers; return hipSuccess or the launch error. `mb` = ceil(heads / 32).
hipError_t launch_indexer_split(const IdxArgs& a, const SplitArgs& s, int mb, int dim, bool fp8,
                                int group, bool scores_mode, hipStream_t st);
// Largest chunk the split kernel's LDS holds for this instantiation.
int indexer_split_chunk_cap(int mb, int dim, bool fp8, int group);
hipError_t launch_topk_from_scores(const FromScoresArgs& f, const SplitArgs& s, hipStream_t st);
hipError_t launch_topk_merge(const MergeArgs& m, hipStream_t st);
hipError_t launch_indexer_stream(const IdxArgs& a, const StreamArgs& s, int mb, int dim, bool fp8,
                                 int grid, hipStream_t st);
int indexer_stream_blocks_per_cu(int mb, int dim, bool fp8, int cap, int max_visible);
size_t indexer_stream_smem(int cap, int max_visible);
constexpr size_t kMaxLds = 160 * 1024;
constexpr int kCoarseBinsHost = 2048;   // = kCoarseBins of the selection code
hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t st);

constexpr int kSplitThreads = 512;   // eight waves: two per SIMD
constexpr int kMergeThreads = 512;
constexpr int kMergeCap = 32768;       // keys one merge workgroup holds in LDS (128 KB)
constexpr int kStreamThreads = 256;    // four waves, one query each

// Attention.
struct AttnArgs {
    const int32_t* page_table;
    const int32_t* seq_lens;
    int32_t batch, max_pages;
    const uint16_t* kv;       // bf16 [num_pages, 64, 576]
    int64_t num_pages;
    const int32_t* q_seq;
    int32_t num_q;
    const uint16_t* q;        // bf16 [num_q, heads, 576]
    int32_t heads, d_v;
    const int32_t* idx;       // [num_q, topk]
    int32_t topk;
    float sm_scale;
    int32_t n_split, rows_per_split, heads_per_block;
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
