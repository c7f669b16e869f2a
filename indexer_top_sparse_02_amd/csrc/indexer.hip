// Fused lightweight indexer + exact Top-K for gfx950.
//
// score[j,s] = sigma_s * sum_h w[j,h] * max(0, q[j,h,:] . k_s)
//
// The q . k products of one query against 32 positions are one MFMA tile:
// heads are the M dimension (32 per block), positions the N dimension, the
// index dim the K dimension. Queries sit in registers for the whole pass; each
// lane streams its position's half-row of index-K straight from the paged pool
// (fp8 rows are widened to bf16 exactly in registers). The accumulator puts 16
// heads of one position in each lane, so the ReLU, the head weights and the head
// sum stay in registers with a single cross-lane add, and sigma_s multiplies the
// sum. Only the selected positions ever reach memory ("Rapid Adaptation and
// Inference Optimization", section 4.1 "Indexer Fusion").
//
// Two launch shapes share that score code and the exact selection of
// sia_select.h, so they return identical indices:
//  * split: a workgroup scores a chunk of one sequence's positions for one or two
//    queries (decode, draft tokens), keeps the chunk's scores in LDS, selects the
//    chunk's Top-K and writes those candidates; a merge pass selects the final
//    Top-K from the candidates of all chunks. The global Top-K is a subset of the
//    union of per-chunk Top-Ks under the same total order, so this is exact.
//  * stream: one wave walks one query's whole causal row (prefill), appending
//    positions that beat the current threshold to an LDS buffer kept in position
//    order, and re-selecting the Top-K when the buffer fills. A position that
//    ties the threshold arrives after every kept one, so it can be dropped.
#include "sia_device.h"
#include "sia_kernels.h"
#include "sia_sched.h"
#include "sia_select.h"

namespace sia {

// ------------------------------------------------------------ score tile

template <int MB, int D>
struct IdxQuery {
    static constexpr int KS = D / 16;
    bf16x8 a[MB][KS];
    float w[MB][16];
};

template <int MB, int D>
__device__ __forceinline__ void load_query(const IdxArgs& A, int j, IdxQuery<MB, D>& q) {
    const int l = lane_id(), m = l & 31, half = l >> 5;
#pragma unroll
    for (int mb = 0; mb < MB; mb++) {
        const int head = mb * 32 + m;
#pragma unroll
        for (int ks = 0; ks < IdxQuery<MB, D>::KS; ks++) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (head < A.heads)
                v = *reinterpret_cast<const u32x4*>(
                    A.q_idx + ((int64_t)j * A.heads + head) * D + half * (D / 2) + ks * 8);
            q.a[mb][ks] = as_bf16x8(v);
        }
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int h = mb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            q.w[mb][r] = h < A.heads ? A.w[(int64_t)j * A.heads + h] : 0.f;
        }
    }
}

// One lane's share of a 32-position tile: half a row of index-K (+ its scale).
template <int D, bool FP8>
struct KTile {
    static constexpr int BYTES = (D / 2) * (FP8 ? 1 : 2);
    static constexpr int NV = BYTES / 16;
    u32x4 v[NV];
    float sc;
};

// Visible row length of query j (clamped; flags bad input).
__device__ __forceinline__ int visible_len(const IdxArgs& A, int j, int& b) {
    b = A.q_seq[j];
    if (b < 0 || b >= A.batch) {
        if (lane_id() == 0) atomicOr(A.status, kBadSeq);
        b = 0;
        return 0;
    }
    int64_t r = (int64_t)A.q_pos[j] + 1;
    const int64_t n = A.seq_lens[b];
    if (r > n) r = n;
    if (r < 0) r = 0;
    const int64_t cap_pages = (int64_t)A.max_pages * kPage;
    if (r > cap_pages) {
        if (lane_id() == 0) atomicOr(A.status, kBadPage);
        r = cap_pages;
    }
    if (r > A.max_visible) {
        if (lane_id() == 0) atomicOr(A.status, kRowTooLong);
        r = A.max_visible;
    }
    return (int)r;
}

// Loads the tile starting at pos0 (a multiple of 32). Lanes whose position is
// not visible, or whose page id is out of range, load zeros.
template <int D, bool FP8>
__device__ __forceinline__ void load_ktile(const IdxArgs& A, int b, int pos0, int row_len,
                                           KTile<D, FP8>& t) {
    const int l = lane_id(), half = l >> 5;
    const int p = pos0 + (l & 31);
    int page = A.page_table[(int64_t)b * A.max_pages + (pos0 >> 6)];
    page = __builtin_amdgcn_readfirstlane(page);
    const bool page_ok = page >= 0 && page < A.num_pages;
    if (!page_ok && pos0 < row_len && l == 0) atomicOr(A.status, kBadPage);
    const bool ok = page_ok && p < row_len;
    const int64_t row = (int64_t)page * kPage + (p & 63);
#pragma unroll
    for (int i = 0; i < KTile<D, FP8>::NV; i++) t.v[i] = u32x4{0u, 0u, 0u, 0u};
    t.sc = 1.f;
    if (ok) {
        const uint8_t* src = A.rows + row * (D * (FP8 ? 1 : 2)) + half * KTile<D, FP8>::BYTES;
#pragma unroll
        for (int i = 0; i < KTile<D, FP8>::NV; i++)
            t.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + i);
        if constexpr (FP8) t.sc = A.scale[row];
    }
}

// Scores of the tile's 32 positions; lanes l and l+32 both return the score of
// position pos0 + l%32. Fixed operation order, so every kernel that uses it
// produces the same bits.
template <int MB, int D, bool FP8>
__device__ __forceinline__ float tile_scores(const IdxQuery<MB, D>& q, const KTile<D, FP8>& t) {
    constexpr int KS = D / 16;
    f32x16 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; mb++) acc[mb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
        bf16x8 bk;
        if constexpr (FP8) {
            const u32x4 vv = t.v[ks >> 1];
            bk = e4m3x8_to_bf16x8(vv[(ks & 1) * 2], vv[(ks & 1) * 2 + 1]);
        } else {
            bk = as_bf16x8(t.v[ks]);
        }
#pragma unroll
        for (int mb = 0; mb < MB; mb++) acc[mb] = mfma32(q.a[mb][ks], bk, acc[mb]);
    }
    float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; mb++) {
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
            p0 = fmaf(q.w[mb][r + 0], fmaxf(acc[mb][r + 0], 0.f), p0);
            p1 = fmaf(q.w[mb][r + 1], fmaxf(acc[mb][r + 1], 0.f), p1);
            p2 = fmaf(q.w[mb][r + 2], fmaxf(acc[mb][r + 2], 0.f), p2);
            p3 = fmaf(q.w[mb][r + 3], fmaxf(acc[mb][r + 3], 0.f), p3);
        }
    }
    const float part = (p0 + p1) + (p2 + p3);
    float s = part + __shfl_xor(part, 32, kWave);
    if constexpr (FP8) s = s * t.sc;
    return s;
}

// ------------------------------------------------------------ emitters

struct EmitFinal {
    int32_t* idx;
    float* score;
    int base;        // position of key index 0
    __device__ void prefetch(int, u32x4) {}
    __device__ void operator()(int rank, int i, int, uint32_t k) const {
        idx[rank] = base + i;
        if (score) score[rank] = key_score(k);
    }
};

struct EmitCand {
    uint32_t* key;
    int32_t* pos;
    int base;
    __device__ void prefetch(int, u32x4) {}
    __device__ void operator()(int rank, int i, int, uint32_t k) const {
        key[rank] = k;
        pos[rank] = base + i;
    }
};

// Positions come from a parallel array (merge inputs).
struct EmitFinalPos {
    const int32_t* src_pos;
    int32_t* idx;
    float* score;
    __device__ void prefetch(int, u32x4) {}
    __device__ void operator()(int rank, int i, int, uint32_t k) const {
        idx[rank] = src_pos[i];
        if (score) score[rank] = key_score(k);
    }
};

struct EmitCandPos {
    const int32_t* src_pos;
    uint32_t* key;
    int32_t* pos;
    __device__ void prefetch(int, u32x4) {}
    __device__ void operator()(int rank, int i, int, uint32_t k) const {
        key[rank] = k;
        pos[rank] = src_pos[i];
    }
};

// In-place compaction of a wave's LDS buffer: positions of the round are read
// before any of the round's writes.
struct EmitInPlace {
    uint32_t* key;
    int32_t* pos;
    int32_t p4[4];
    __device__ void prefetch(int i, u32x4 k4) {
#pragma unroll
        for (int e = 0; e < 4; e++) p4[e] = k4[e] != 0u ? pos[i + e] : 0;
    }
    __device__ void operator()(int rank, int, int e, uint32_t k) const {
        key[rank] = k;
        pos[rank] = p4[e];
    }
};

struct EmitFinalBuf {
    const int32_t* pos;
    int32_t* idx;
    float* score;
    int32_t p4[4];
    __device__ void prefetch(int i, u32x4 k4) {
#pragma unroll
        for (int e = 0; e < 4; e++) p4[e] = k4[e] != 0u ? pos[i + e] : 0;
    }
    __device__ void operator()(int rank, int, int e, uint32_t k) const {
        idx[rank] = p4[e];
        if (score) score[rank] = key_score(k);
    }
};

// Select the top min(m_cap, nonzero) of keys[0..n) and emit them in index order.
template <int NT, typename Emit>
__device__ int select_emit(const uint32_t* keys, int n, int m_cap, SelScratch* s, Emit&& emit) {
    const int cnt = count_nonzero<NT>(keys, n, s);
    const int m = min(m_cap, cnt);
    if (m <= 0) return 0;
    if (m == cnt) {
        ordered_compact<NT>(keys, n, 0u, 0, s, emit);   // every nonzero key
    } else {
        int ties;
        const uint32_t T = radix_threshold<NT>(keys, n, m, s, ties);
        ordered_compact<NT>(keys, n, T, ties, s, emit);
    }
    return m;
}

// ------------------------------------------------------------ split kernel

template <int MB, int D, bool FP8, int G, bool SCORES>
__global__ __launch_bounds__(kSplitThreads) void indexer_split_kernel(IdxArgs A, SplitArgs S) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint32_t* keys_all = reinterpret_cast<uint32_t*>(smem);
    SelScratch* sel = reinterpret_cast<SelScratch*>(smem + (size_t)G * S.chunk * 4);

    constexpr int WPQ = 4 / G;   // waves per query
    const int g = blockIdx.x / S.n_chunks;
    const int c = blockIdx.x % S.n_chunks;
    const int w = threadIdx.x / kWave, l = lane_id();
    const int qi = w / WPQ, sub = w % WPQ;
    const int j = g * G + qi;
    const int chunk0 = c * S.chunk;

    // ---- scores of this chunk
    if (j < A.num_q) {
        int b;
        const int rl = visible_len(A, j, b);
        const int nvalid = max(0, min(S.chunk, rl - chunk0));
        uint32_t* keys = keys_all + qi * S.chunk;
        const int ntiles = (nvalid + 31) / 32;
        if (sub < ntiles) {
            IdxQuery<MB, D> q;
            load_query<MB, D>(A, j, q);
            KTile<D, FP8> cur, nxt;
            load_ktile<D, FP8>(A, b, chunk0 + sub * 32, rl, cur);
            for (int t = sub; t < ntiles; t += WPQ) {
                if (t + WPQ < ntiles) load_ktile<D, FP8>(A, b, chunk0 + (t + WPQ) * 32, rl, nxt);
                const float s = tile_scores<MB, D, FP8>(q, cur);
                const int i = t * 32 + (l & 31);
                if constexpr (SCORES) {
                    if (l < 32 && i < nvalid) S.scores[(int64_t)j * S.ld + chunk0 + i] = s;
                } else {
                    if (l < 32) keys[i] = i < nvalid ? score_key(s) : 0u;
                }
                cur = nxt;
            }
        }
        if constexpr (!SCORES) {
            // zero the keys past the last tile so that groups of four are clean
            for (int i = ntiles * 32 + threadIdx.x % (WPQ * kWave); i < S.chunk && i < ntiles * 32 + 4;
                 i += WPQ * kWave)
                if (sub == 0 || true) keys[i] = 0u;
        }
    }
    if constexpr (SCORES) return;
    else {
        __syncthreads();
        // ---- per-query selection over the chunk
        for (int q2 = 0; q2 < G; q2++) {
            const int j2 = g * G + q2;
            if (j2 >= A.num_q) break;
            int b2;
            const int rl = visible_len(A, j2, b2);
            const int nvalid = max(0, min(S.chunk, rl - chunk0));
            const int nscan = (nvalid + 31) / 32 * 32;
            const uint32_t* keys = keys_all + q2 * S.chunk;
            if (S.n_chunks == 1) {
                int32_t* oi = S.out_idx + (int64_t)j2 * S.topk;
                float* os = S.out_score ? S.out_score + (int64_t)j2 * S.topk : nullptr;
                const int m = select_emit<kSplitThreads>(keys, nscan, S.topk, sel,
                                                         EmitFinal{oi, os, chunk0});
                for (int r = m + threadIdx.x; r < S.topk; r += kSplitThreads) {
                    oi[r] = -1;
                    if (os) os[r] = -INFINITY;
                }
            } else {
                const int64_t slot = (int64_t)j2 * S.n_chunks + c;
                const int m = select_emit<kSplitThreads>(
                    keys, nscan, S.kc, sel,
                    EmitCand{S.cand_key + slot * S.kc, S.cand_pos + slot * S.kc, chunk0});
                if (threadIdx.x == 0) S.cand_cnt[slot] = m;
            }
            __syncthreads();
        }
    }
}

// ------------------------------------------------------------ selection from given scores

__global__ __launch_bounds__(kSplitThreads) void topk_from_scores_kernel(FromScoresArgs F, SplitArgs S) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint32_t* keys = reinterpret_cast<uint32_t*>(smem);
    SelScratch* sel = reinterpret_cast<SelScratch*>(smem + (size_t)S.chunk * 4);
    const int j = blockIdx.x / S.n_chunks;
    const int c = blockIdx.x % S.n_chunks;
    const int chunk0 = c * S.chunk;
    const int rl = F.row_len[j];
    const int nvalid = max(0, min(S.chunk, rl - chunk0));
    const int nscan = (nvalid + 3) / 4 * 4;
    for (int i = threadIdx.x; i < nscan; i += kSplitThreads)
        keys[i] = i < nvalid ? score_key(F.scores[(int64_t)j * F.ld + chunk0 + i]) : 0u;
    __syncthreads();
    if (S.n_chunks == 1) {
        int32_t* oi = S.out_idx + (int64_t)j * S.topk;
        float* os = S.out_score ? S.out_score + (int64_t)j * S.topk : nullptr;
        const int m = select_emit<kSplitThreads>(keys, nscan, S.topk, sel, EmitFinal{oi, os, chunk0});
        for (int r = m + threadIdx.x; r < S.topk; r += kSplitThreads) {
            oi[r] = -1;
            if (os) os[r] = -INFINITY;
        }
    } else {
        const int64_t slot = (int64_t)j * S.n_chunks + c;
        const int m = select_emit<kSplitThreads>(
            keys, nscan, S.kc, sel,
            EmitCand{S.cand_key + slot * S.kc, S.cand_pos + slot * S.kc, chunk0});
        if (threadIdx.x == 0) S.cand_cnt[slot] = m;
    }
}

// ------------------------------------------------------------ merge

__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(MergeArgs M) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint32_t* keys = reinterpret_cast<uint32_t*>(smem);
    const int q = blockIdx.x / M.n_out;
    const int o = blockIdx.x % M.n_out;
    const int s0 = o * M.fan_in;
    const int nsets = min(M.fan_in, M.n_in - s0);
    const int n = nsets * M.kc_in;
    SelScratch* sel = reinterpret_cast<SelScratch*>(smem + (size_t)M.fan_in * M.kc_in * 4);
    const int64_t set0 = (int64_t)q * M.n_in + s0;
    for (int i = threadIdx.x; i < n; i += kMergeThreads) {
        const int set = i / M.kc_in, off = i - set * M.kc_in;
        keys[i] = off < M.in_cnt[set0 + set] ? M.in_key[set0 * M.kc_in + i] : 0u;
    }
    __syncthreads();
    const int32_t* src_pos = M.in_pos + set0 * M.kc_in;
    if (M.out_idx) {
        int32_t* oi = M.out_idx + (int64_t)q * M.topk;
        float* os = M.out_score ? M.out_score + (int64_t)q * M.topk : nullptr;
        const int m = select_emit<kMergeThreads>(keys, n, M.topk, sel, EmitFinalPos{src_pos, oi, os});
        for (int r = m + threadIdx.x; r < M.topk; r += kMergeThreads) {
            oi[r] = -1;
            if (os) os[r] = -INFINITY;
        }
    } else {
        const int64_t slot = (int64_t)q * M.n_out + o;
        const int m = select_emit<kMergeThreads>(
            keys, n, M.topk, sel,
            EmitCandPos{src_pos, M.out_key + slot * M.topk, M.out_pos + slot * M.topk});
        if (threadIdx.x == 0) M.out_cnt[slot] = m;
    }
}

// ------------------------------------------------------------ stream kernel

struct WaveBuf {
    uint32_t* key;
    int32_t* pos;
    SelScratch* sel;
};

template <int MB, int D, bool FP8>
__device__ void stream_query(const IdxArgs& A, const StreamArgs& S, int j, WaveBuf B) {
    const int l = lane_id();
    int b;
    const int rl = visible_len(A, j, b);
    int32_t* oi = S.out_idx + (int64_t)j * S.topk;
    float* os = S.out_score ? S.out_score + (int64_t)j * S.topk : nullptr;
    int cnt = 0;
    uint32_t tau = 0u;
    const int ntiles = (rl + 31) / 32;
    if (ntiles > 0) {
        IdxQuery<MB, D> q;
        load_query<MB, D>(A, j, q);
        KTile<D, FP8> cur, nxt;
        load_ktile<D, FP8>(A, b, 0, rl, cur);
        for (int t = 0; t < ntiles; t++) {
            if (t + 1 < ntiles) load_ktile<D, FP8>(A, b, (t + 1) * 32, rl, nxt);
            const float s = tile_scores<MB, D, FP8>(q, cur);
            const int p = t * 32 + (l & 31);
            const uint32_t k = (l < 32 && p < rl) ? score_key(s) : 0u;
            const bool take = k > tau;
            const uint64_t mask = __ballot(take);
            if (take) {
                const int at = cnt + lanes_below(mask);
                B.key[at] = k;
                B.pos[at] = p;
            }
            cnt += __popcll(mask);
            cur = nxt;
            if (cnt > S.cap - 32) {
                // keep exactly the Top-K seen so far; later ties of T lose to them
                wave_sync();
                int ties;
                const int n4 = (cnt + 3) & ~3;
                for (int i = cnt + l; i < n4; i += kWave) B.key[i] = 0u;
                wave_sync();
                const uint32_t T = radix_threshold<kWave>(B.key, n4, S.topk, B.sel, ties);
                ordered_compact<kWave>(B.key, n4, T, ties, B.sel, EmitInPlace{B.key, B.pos, {}});
                cnt = S.topk;
                tau = T;
                wave_sync();
            }
        }
    }
    wave_sync();
    const int n4 = (cnt + 3) & ~3;
    for (int i = cnt + l; i < n4; i += kWave) B.key[i] = 0u;
    wave_sync();
    const int m = select_emit<kWave>(B.key, n4, S.topk, B.sel, EmitFinalBuf{B.pos, oi, os, {}});
    for (int r = m + l; r < S.topk; r += kWave) {
        oi[r] = -1;
        if (os) os[r] = -INFINITY;
    }
    wave_sync();
}

template <int MB, int D, bool FP8>
__global__ __launch_bounds__(kStreamThreads) void indexer_stream_kernel(IdxArgs A, StreamArgs S) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ int next_tile;
    const int w = threadIdx.x / kWave;
    const size_t per_wave = (size_t)S.cap * 8 + sizeof(SelScratch);
    uint8_t* base = smem + w * per_wave;
    WaveBuf B{reinterpret_cast<uint32_t*>(base), reinterpret_cast<int32_t*>(base + (size_t)S.cap * 4),
              reinterpret_cast<SelScratch*>(base + (size_t)S.cap * 8)};
    constexpr int QPT = kStreamThreads / kWave;   // queries per tile
    auto run_tile = [&](int tile) {
        const int j = tile * QPT + w;
        if (j < A.num_q) stream_query<MB, D, FP8>(A, S, j, B);
    };
    if (S.sched == 0) {
        run_tile(blockIdx.x);
    } else if (S.sched == 2) {
        const int t0 = zigzag_shard(S.n_tiles, blockIdx.x, 0);
        const int t1 = zigzag_shard(S.n_tiles, blockIdx.x, 1);
        if (t1 >= 0) run_tile(t1);   // heavier one first
        if (t0 >= 0) run_tile(t0);
    } else {
        for (;;) {
            if (threadIdx.x == 0) next_tile = (int)atomicAdd(S.counter, 1u);
            __syncthreads();
            const int n = next_tile;
            __syncthreads();
            if (n >= S.n_tiles) break;
            run_tile(heavy_first_tile(S.n_tiles, n));
        }
    }
}

__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// ------------------------------------------------------------ launchers

template <typename K>
static hipError_t set_smem(K kernel, size_t bytes) {
    if (bytes > 64 * 1024)
        return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    return hipSuccess;
}

template <int MB, int D, bool FP8, int G, bool SC>
static hipError_t split_launch(const IdxArgs& a, const SplitArgs& s, hipStream_t st) {
    const int groups = (a.num_q + G - 1) / G;
    const size_t smem = SC ? 16 : (size_t)G * s.chunk * 4 + sizeof(SelScratch);
    auto k = indexer_split_kernel<MB, D, FP8, G, SC>;
    hipError_t e = set_smem(k, smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(groups * s.n_chunks), dim3(kSplitThreads), smem, st, a, s);
    return hipGetLastError();
}

template <int MB, int D, bool FP8, int G>
static hipError_t split_launch2(const IdxArgs& a, const SplitArgs& s, bool sc, hipStream_t st) {
    return sc ? split_launch<MB, D, FP8, G, true>(a, s, st) : split_launch<MB, D, FP8, G, false>(a, s, st);
}

template <int MB, int D, bool FP8>
static hipError_t split_launch3(const IdxArgs& a, const SplitArgs& s, int g, bool sc, hipStream_t st) {
    return g == 2 ? split_launch2<MB, D, FP8, 2>(a, s, sc, st) : split_launch2<MB, D, FP8, 1>(a, s, sc, st);
}

hipError_t launch_indexer_split(const IdxArgs& a, const SplitArgs& s, int mb, int dim, bool fp8,
                                int group, bool scores_mode, hipStream_t st) {
#define SIA_SPLIT(MBv, Dv, F8)                                                  \
    if (mb == MBv && dim == Dv && fp8 == F8)                                   \
        return split_launch3<MBv, Dv, F8>(a, s, group, scores_mode, st);
    SIA_SPLIT(1, 64, false) SIA_SPLIT(1, 64, true) SIA_SPLIT(1, 128, false) SIA_SPLIT(1, 128, true)
    SIA_SPLIT(2, 64, false) SIA_SPLIT(2, 64, true) SIA_SPLIT(2, 128, false) SIA_SPLIT(2, 128, true)
#undef SIA_SPLIT
    return hipErrorInvalidValue;
}

hipError_t launch_topk_from_scores(const FromScoresArgs& f, const SplitArgs& s, hipStream_t st) {
    const size_t smem = (size_t)s.chunk * 4 + sizeof(SelScratch);
    hipError_t e = set_smem(topk_from_scores_kernel, smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_from_scores_kernel, dim3(f.num_q * s.n_chunks), dim3(kSplitThreads), smem,
                       st, f, s);
    return hipGetLastError();
}

hipError_t launch_topk_merge(const MergeArgs& m, hipStream_t st) {
    const size_t smem = (size_t)m.fan_in * m.kc_in * 4 + sizeof(SelScratch);
    hipError_t e = set_smem(topk_merge_kernel, smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_merge_kernel, dim3(m.num_q * m.n_out), dim3(kMergeThreads), smem, st, m);
    return hipGetLastError();
}

static size_t stream_smem(int cap) { return 4 * ((size_t)cap * 8 + sizeof(SelScratch)); }

template <int MB, int D, bool FP8>
static hipError_t stream_launch(const IdxArgs& a, const StreamArgs& s, int grid, hipStream_t st) {
    auto k = indexer_stream_kernel<MB, D, FP8>;
    const size_t smem = stream_smem(s.cap);
    hipError_t e = set_smem(k, smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(grid), dim3(kStreamThreads), smem, st, a, s);
    return hipGetLastError();
}

template <int MB, int D, bool FP8>
static int stream_occupancy(int cap) {
    auto k = indexer_stream_kernel<MB, D, FP8>;
    const size_t smem = stream_smem(cap);
    if (set_smem(k, smem) != hipSuccess) return 1;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(k),
                                                     kStreamThreads, smem) != hipSuccess || n < 1)
        return 1;
    return n;
}

hipError_t launch_indexer_stream(const IdxArgs& a, const StreamArgs& s, int mb, int dim, bool fp8,
                                 int grid, hipStream_t st) {
#define SIA_STREAM(MBv, Dv, F8) \
    if (mb == MBv && dim == Dv && fp8 == F8) return stream_launch<MBv, Dv, F8>(a, s, grid, st);
    SIA_STREAM(1, 64, false) SIA_STREAM(1, 64, true) SIA_STREAM(1, 128, false) SIA_STREAM(1, 128, true)
    SIA_STREAM(2, 64, false) SIA_STREAM(2, 64, true) SIA_STREAM(2, 128, false) SIA_STREAM(2, 128, true)
#undef SIA_STREAM
    return hipErrorInvalidValue;
}

int indexer_stream_blocks_per_cu(int mb, int dim, bool fp8, int cap) {
#define SIA_OCC(MBv, Dv, F8) \
    if (mb == MBv && dim == Dv && fp8 == F8) return stream_occupancy<MBv, Dv, F8>(cap);
    SIA_OCC(1, 64, false) SIA_OCC(1, 64, true) SIA_OCC(1, 128, false) SIA_OCC(1, 128, true)
    SIA_OCC(2, 64, false) SIA_OCC(2, 64, true) SIA_OCC(2, 128, false) SIA_OCC(2, 128, true)
#undef SIA_OCC
    return 1;
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, v, n);
    return hipGetLastError();
}

}  // namespace sia
