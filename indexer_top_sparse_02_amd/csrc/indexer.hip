// Fused lightweight indexer + exact Top-K for gfx950.
//
// score[j,s] = sigma_s * sum_h w[j,h] * max(0, q[j,h,:] . k_s)
//
// The q . k products of one query against 32 positions are one MFMA tile:
// heads are the M dimension (32 per block), positions the N dimension, the
// index dim the K dimension. Queries sit in registers for the whole pass; a
// lane supplies its position's half-row of index-K (fp8 rows are widened to bf16
// exactly in registers), staged through LDS by the split kernel and loaded
// straight from the paged pool by the stream kernel. The accumulator puts 16
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

static_assert(kCoarseBins == kCoarseBinsHost, "host and device histogram sizes differ");

// ------------------------------------------------------------ score tile

// A query's indexer heads in MFMA operand layout. The bf16 form feeds
// 32x32x16 bf16 MFMAs (fp8 keys are widened to bf16). The fp8 form feeds
// 32x32x64 fp8 MFMAs on the raw e4m3 key bytes: q * 2^s is split into an e4m3
// high part and an e4m3 residual times 2^4 (one exponent s per query, chosen so
// that max|q| * 2^s < 256), and the two products are summed with MFMA scales
// 2^-s and 2^-(s+4). The split is exact for every element above 2^-21 of the
// query's largest element (below that the residual underflows), so the scores
// equal those of the bf16 form up to rounding order.
template <int MB, int D, bool FP8>
struct IdxQuery;

template <int MB, int D>
struct IdxQuery<MB, D, false> {
    static constexpr int KS = D / 16;
    bf16x8 a[MB][KS];
    float w[MB][16];
};

template <int MB, int D>
struct IdxQuery<MB, D, true> {
    static constexpr int KS = D / 64;
    i32x8 hi[MB][KS], lo[MB][KS];
    int sh, sl;   // E8M0 scales of the two parts
    float w[MB][16];
};

template <int MB, int D>
__device__ __forceinline__ void load_weights(const IdxArgs& A, int j, float (&w)[MB][16]) {
    const int half = lane_id() >> 5;
#pragma unroll
    for (int mb = 0; mb < MB; mb++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int h = mb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            w[mb][r] = h < A.heads ? A.w[(int64_t)j * A.heads + h] : 0.f;
        }
}

template <int MB, int D>
__device__ __forceinline__ void load_query(const IdxArgs& A, int j, IdxQuery<MB, D, false>& q) {
    const int l = lane_id(), m = l & 31, half = l >> 5;
#pragma unroll
    for (int mb = 0; mb < MB; mb++) {
        const int head = mb * 32 + m;
#pragma unroll
        for (int ks = 0; ks < IdxQuery<MB, D, false>::KS; ks++) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (head < A.heads)
                v = *reinterpret_cast<const u32x4*>(
                    A.q_idx + ((int64_t)j * A.heads + head) * D + half * (D / 2) + ks * 8);
            q.a[mb][ks] = as_bf16x8(v);
        }
    }
    load_weights<MB, D>(A, j, q.w);
}

template <int MB, int D>
__device__ __forceinline__ void load_query(const IdxArgs& A, int j, IdxQuery<MB, D, true>& q) {
    constexpr int KS = IdxQuery<MB, D, true>::KS;
    const int l = lane_id(), m = l & 31, half = l >> 5;
    // lane l holds head mb*32 + l%32 and dims 64 ks + 32 (l/32) .. +31 of each step;
    // the query is read twice (the second time from cache): once for its largest
    // magnitude, once to split it
    auto ld = [&](int mb, int ks, int c) -> u32x4 {
        const int head = mb * 32 + m;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (head < A.heads)
            v = *reinterpret_cast<const u32x4*>(
                A.q_idx + ((int64_t)j * A.heads + head) * D + ks * 64 + half * 32 + c * 8);
        return v;
    };
    float amax = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; mb++)
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const u32x4 v = ld(mb, ks, c);
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    amax = fmaxf(amax, fabsf(__uint_as_float(v[e] << 16)));
                    amax = fmaxf(amax, fabsf(__uint_as_float(v[e] & 0xffff0000u)));
                }
            }
    amax = wave_max_f(amax);
    // exponent s with amax * 2^s in [128, 256) (0 for an all-zero query)
    int s = 0;
    if (amax > 0.f) {
        int e;
        frexpf(amax, &e);   // amax = f * 2^e, f in [0.5, 1)
        s = min(max(8 - e, -120), 120);
    }
    const float f = ldexpf(1.f, s);
    q.sh = 127 - s;
    q.sl = 127 - s - 4;
#pragma unroll
    for (int mb = 0; mb < MB; mb++)
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const u32x4 v = ld(mb, ks, c);
#pragma unroll
                for (int e = 0; e < 4; e += 2) {
                    // four bf16 -> one dword of e4m3 (high part) and one of e4m3 (residual)
                    float x[4];
                    x[0] = __uint_as_float(v[e] << 16) * f;
                    x[1] = __uint_as_float(v[e] & 0xffff0000u) * f;
                    x[2] = __uint_as_float(v[e + 1] << 16) * f;
                    x[3] = __uint_as_float(v[e + 1] & 0xffff0000u) * f;
                    int h = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
                    h = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], h, true);
                    float r[4];
                    r[0] = (x[0] - __builtin_amdgcn_cvt_f32_fp8(h, 0)) * 16.f;
                    r[1] = (x[1] - __builtin_amdgcn_cvt_f32_fp8(h, 1)) * 16.f;
                    r[2] = (x[2] - __builtin_amdgcn_cvt_f32_fp8(h, 2)) * 16.f;
                    r[3] = (x[3] - __builtin_amdgcn_cvt_f32_fp8(h, 3)) * 16.f;
                    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
                    lo = __builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], lo, true);
                    q.hi[mb][ks][c * 2 + e / 2] = h;
                    q.lo[mb][ks][c * 2 + e / 2] = lo;
                }
            }
        }
    load_weights<MB, D>(A, j, q.w);
}

// One lane's share of a 32-position tile: half a row of index-K (+ its scale).
// bf16: lane half h holds the row's chunks h*CPR/2 .. (16-byte chunks, the
// 32x32x16 operand layout); fp8: for each 64-byte MFMA step ks it holds the 32
// bytes 64 ks + 32 h .. (chunks 4 ks + 2 h and 4 ks + 2 h + 1).
template <int D, bool FP8>
struct KTile {
    static constexpr int BYTES = (D / 2) * (FP8 ? 1 : 2);
    static constexpr int NV = BYTES / 16;
    u32x4 v[NV];
    float sc;
    bool ok;      // this lane's position is visible and its page id valid
    // 16-byte chunk of the row held in v[i] by lane half h
    static __device__ __forceinline__ int chunk(int i, int h) {
        if constexpr (FP8) return 4 * (i >> 1) + 2 * h + (i & 1);
        else return h * NV + i;
    }
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

// Physical page of logical page `lp` of sequence b, or -1 (and a status bit)
// if the table holds an id outside [0, num_pages).
__device__ __forceinline__ int page_of(const IdxArgs& A, int b, int lp) {
    const int page = A.page_table[(int64_t)b * A.max_pages + lp];
    if (page >= 0 && page < A.num_pages) return page;
    atomicOr(A.status, kBadPage);
    return -1;
}

// Loads the tile starting at pos0 (a multiple of 32) that lives on physical
// page `page` (wave-uniform). Branch-free: a lane whose position is not visible,
// or whose page is invalid, reads row 0 of the pool instead (always in bounds)
// and is marked not ok, so that its score is discarded. Keeping loads out of
// branches lets the compiler wait for exactly the tile being consumed.
template <int D, bool FP8>
__device__ __forceinline__ void load_ktile(const IdxArgs& A, int page, int pos0, int row_len,
                                           KTile<D, FP8>& t) {
    const int l = lane_id(), half = l >> 5;
    const int p = pos0 + (l & 31);
    t.ok = page >= 0 && p < row_len;
    const int64_t row = t.ok ? (int64_t)page * kPage + (p & 63) : 0;
    const uint8_t* src = A.rows + row * (D * (FP8 ? 1 : 2));
#pragma unroll
    for (int i = 0; i < KTile<D, FP8>::NV; i++)
        t.v[i] = reinterpret_cast<const u32x4*>(src)[KTile<D, FP8>::chunk(i, half)];
    if constexpr (FP8) t.sc = A.scale[row];
    else t.sc = 1.f;
}

// max(0, x) in one integer instruction: a negative float is a negative int,
// -0.0 maps to +0.0.
__device__ __forceinline__ float relu(float x) {
    return __int_as_float(max(__float_as_int(x), 0));
}

// x[lane] + x[lane ^ 32], as (lower-half value) + (upper-half value) in every lane.
__device__ __forceinline__ float add_halves(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// MFMA half of a tile: the raw q.k products of one query against 32
// positions (heads x positions accumulators).
template <int MB, int D, bool FP8>
__device__ __forceinline__ void tile_mfma(const IdxQuery<MB, D, FP8>& q, const KTile<D, FP8>& t,
                                          f32x16 (&acc)[MB]) {
#pragma unroll
    for (int mb = 0; mb < MB; mb++) acc[mb] = f32x16{};
    if constexpr (FP8) {
        constexpr int KS = D / 64;
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            const u32x4 v0 = t.v[2 * ks], v1 = t.v[2 * ks + 1];
            const i32x8 b = {(int)v0[0], (int)v0[1], (int)v0[2], (int)v0[3],
                             (int)v1[0], (int)v1[1], (int)v1[2], (int)v1[3]};
#pragma unroll
            for (int mb = 0; mb < MB; mb++) {
                acc[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(q.hi[mb][ks], b, acc[mb], 0, 0, 0,
                                                                          q.sh, 0, 127);
                acc[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(q.lo[mb][ks], b, acc[mb], 0, 0, 0,
                                                                          q.sl, 0, 127);
            }
        }
    } else {
        constexpr int KS = D / 16;
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            const bf16x8 bk = as_bf16x8(t.v[ks]);
#pragma unroll
            for (int mb = 0; mb < MB; mb++) acc[mb] = mfma32(q.a[mb][ks], bk, acc[mb]);
        }
    }
}

// Vector half: ReLU, head weights, head sum, token scale.
template <int MB, int D, bool FP8>
__device__ __forceinline__ float tile_epilogue(const IdxQuery<MB, D, FP8>& q, const f32x16 (&acc)[MB],
                                               float tsc) {
    float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; mb++) {
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
            p0 = fmaf(q.w[mb][r + 0], relu(acc[mb][r + 0]), p0);
            p1 = fmaf(q.w[mb][r + 1], relu(acc[mb][r + 1]), p1);
            p2 = fmaf(q.w[mb][r + 2], relu(acc[mb][r + 2]), p2);
            p3 = fmaf(q.w[mb][r + 3], relu(acc[mb][r + 3]), p3);
        }
    }
    float v = add_halves((p0 + p1) + (p2 + p3));
    if constexpr (FP8) v = v * tsc;
    return v;
}

// Scores of the tile's 32 positions for one query; lanes l and l+32 both get
// the score of position pos0 + l%32 (undefined where the tile lane is not ok).
// Every kernel scores through tile_mfma + tile_epilogue, so a query and position
// give the same bits in each of them.
template <int MB, int D, bool FP8>
__device__ __forceinline__ float tile_scores(const IdxQuery<MB, D, FP8>& q, const KTile<D, FP8>& t) {
    f32x16 acc[MB];
    tile_mfma<MB, D, FP8>(q, t, acc);
    return tile_epilogue<MB, D, FP8>(q, acc, t.sc);
}

// ------------------------------------------------------------ emitters

struct EmitFinal {
    int32_t* idx;
    float* score;
    int base;        // position of key index 0
    __device__ void prefetch(int, u32x4, uint32_t) {}
    __device__ void prefetch2(int, u32x4, uint32_t) {}
    __device__ void operator()(int rank, int i, int, uint32_t k) const {
        idx[rank] = base + i;
        if (score) score[rank] = key_score(k);
    }
};

struct EmitCand {
    uint32_t* key;
    int32_t* pos;
    int base;
    __device__ void prefetch(int, u32x4, uint32_t) {}
    __device__ void prefetch2(int, u32x4, uint32_t) {}
    __device__ void operator()(int rank, int i, int, uint32_t k) const {
        key[rank] = k;
        pos[rank] = base + i;
    }
};

// Positions come from a parallel array in global memory (merge inputs).
struct EmitFinalPos {
    const int32_t* src_pos;
    int32_t* idx;
    float* score;
    int32_t p4[8];
    __device__ void prefetch(int i, u32x4 k4, uint32_t T) {
#pragma unroll
        for (int e = 0; e < 4; e++) p4[e] = (k4[e] != 0u && k4[e] >= T) ? src_pos[i + e] : 0;
    }
    __device__ void prefetch2(int i, u32x4 k4, uint32_t T) {
#pragma unroll
        for (int e = 0; e < 4; e++) p4[4 + e] = (k4[e] != 0u && k4[e] >= T) ? src_pos[i + e] : 0;
    }
    __device__ void operator()(int rank, int, int e, uint32_t k) const {
        idx[rank] = p4[e];
        if (score) score[rank] = key_score(k);
    }
};

struct EmitCandPos {
    const int32_t* src_pos;
    uint32_t* key;
    int32_t* pos;
    int32_t p4[8];
    __device__ void prefetch(int i, u32x4 k4, uint32_t T) {
#pragma unroll
        for (int e = 0; e < 4; e++) p4[e] = (k4[e] != 0u && k4[e] >= T) ? src_pos[i + e] : 0;
    }
    __device__ void prefetch2(int i, u32x4 k4, uint32_t T) {
#pragma unroll
        for (int e = 0; e < 4; e++) p4[4 + e] = (k4[e] != 0u && k4[e] >= T) ? src_pos[i + e] : 0;
    }
    __device__ void operator()(int rank, int, int e, uint32_t k) const {
        key[rank] = k;
        pos[rank] = p4[e];
    }
};

// In-place compaction of a wave's LDS buffer: positions of the round are read
// before any of the round's writes.
struct EmitInPlace {
    uint32_t* key;
    int32_t* pos;
    int32_t p4[8];
    __device__ void prefetch(int i, u32x4 k4, uint32_t T) {
#pragma unroll
        for (int e = 0; e < 4; e++) p4[e] = (k4[e] != 0u && k4[e] >= T) ? pos[i + e] : 0;
    }
    __device__ void prefetch2(int i, u32x4 k4, uint32_t T) {
#pragma unroll
        for (int e = 0; e < 4; e++) p4[4 + e] = (k4[e] != 0u && k4[e] >= T) ? pos[i + e] : 0;
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
    int32_t p4[8];
    __device__ void prefetch(int i, u32x4 k4, uint32_t T) {
#pragma unroll
        for (int e = 0; e < 4; e++) p4[e] = (k4[e] != 0u && k4[e] >= T) ? pos[i + e] : 0;
    }
    __device__ void prefetch2(int i, u32x4 k4, uint32_t T) {
#pragma unroll
        for (int e = 0; e < 4; e++) p4[4 + e] = (k4[e] != 0u && k4[e] >= T) ? pos[i + e] : 0;
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

// Geometry of the split kernel. Eight waves; wave w scores query w / (8/G)
// against its tiles sub, sub + 8/G, ... (sub = w % (8/G)) of 32 positions.
// Each wave streams its tiles through a private ring of NS LDS slots filled by
// direct global -> LDS copies, 16 bytes per lane and eight lanes per 128-byte
// row (coalesced), with the 16-byte chunks of a row XOR-swizzled by the row
// index so that the MFMA operand reads spread over the LDS banks. A wave only
// waits on its own copies (no barrier in the streaming loop), and issues the
// MFMAs of tile k before the vector epilogue of tile k-1, so both pipes stay
// busy. With two queries the waves of a pair copy the same rows; the second
// copy is served from L2.
template <int D, bool FP8, int G>
struct SplitGeom {
    static constexpr int R = D * (FP8 ? 1 : 2);          // bytes per row
    static constexpr int CPR = R / 16;                   // 16-byte chunks per row
    static constexpr int SWZ = (CPR < 8 ? CPR : 8) - 1;  // chunk swizzle mask
    // two queries: eight waves and most of the LDS (one workgroup per CU); one
    // query: four waves and at most half the LDS, so that two workgroups share a
    // CU and one's setup and selection overlap the other's streaming
    static constexpr int NWV = G == 2 ? 8 : 4;           // waves per workgroup
    static constexpr int NT = NWV * kWave;
    static constexpr int WPQ = NWV / G;                  // waves per query
    static constexpr int TILE = 32 * R;                  // bytes of one tile
    static constexpr size_t LDS_BUDGET = G == 2 ? kMaxLds : kMaxLds / 2;
    static constexpr int NRING = NWV;                    // one ring per wave
    static constexpr int NS_RAW = (G == 2 ? 98304 : 49152) / (NRING * TILE);
    static constexpr int NS = NS_RAW < 2 ? 2 : (NS_RAW > 4 ? 4 : NS_RAW);   // ring depth
    static constexpr int DMA = TILE / 1024;              // 1 KB copies per tile
    static constexpr int PER_TILE = DMA + (FP8 ? 1 : 0); // copies per tile (+ scales)
    static constexpr size_t STATIC_LDS = (size_t)NS * NRING * (TILE + (FP8 ? 128 : 0));
};

__host__ __device__ inline size_t split_pages_bytes(int chunk) {
    return ((size_t)(chunk / kPage) * 4 + 15) / 16 * 16;
}

template <int MB, int D, bool FP8, int G, bool SCORES>
__global__ __launch_bounds__(512) void indexer_split_kernel(IdxArgs A, SplitArgs S) {
    using GM = SplitGeom<D, FP8, G>;
    constexpr int NS = GM::NS, R = GM::R, CPR = GM::CPR, NT = GM::NT, WPQ = GM::WPQ;
    constexpr int NRING = GM::NRING, RB = NRING * GM::TILE, SB = FP8 ? NRING * 32 : 4;
    // one static array per ring slot: every LDS access names its slot, which lets
    // the compiler wait for exactly the copies that wrote it
    __shared__ __attribute__((aligned(16))) uint8_t ring0[RB];
    __shared__ __attribute__((aligned(16))) uint8_t ring1[RB];
    __shared__ __attribute__((aligned(16))) uint8_t ring2[NS > 2 ? RB : 16];
    __shared__ __attribute__((aligned(16))) uint8_t ring3[NS > 3 ? RB : 16];
    __shared__ __attribute__((aligned(16))) float scl0[SB];
    __shared__ __attribute__((aligned(16))) float scl1[SB];
    __shared__ __attribute__((aligned(16))) float scl2[NS > 2 ? SB : 4];
    __shared__ __attribute__((aligned(16))) float scl3[NS > 3 ? SB : 4];
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    int* pages = reinterpret_cast<int*>(smem);
    uint32_t* keys_all = reinterpret_cast<uint32_t*>(smem + split_pages_bytes(S.chunk));
    uint32_t* hist_all = keys_all + (size_t)G * S.chunk;          // [G][kCoarseBins]
    SelScratch* sel = reinterpret_cast<SelScratch*>(hist_all + (SCORES ? 0 : G * kCoarseBins));

    const int g = blockIdx.x / S.n_chunks;
    const int c = blockIdx.x % S.n_chunks;
    const int w = threadIdx.x / kWave, l = lane_id(), half = l >> 5;
    const int qi = w / WPQ, sub = w % WPQ;
    const int chunk0 = c * S.chunk;

    // The group's queries share one sequence; a query naming another sequence is
    // dropped (status bit) rather than scored against the wrong cache.
    int rl[G];
    int b0 = 0, rlmax = 0;
#pragma unroll
    for (int i = 0; i < G; i++) {
        const int j = g * G + i;
        rl[i] = 0;
        if (j < A.num_q) {
            int b;
            rl[i] = visible_len(A, j, b);
            if (i == 0) b0 = b;
            else if (b != b0) {
                if (threadIdx.x == 0) atomicOr(A.status, kBadSeq);
                rl[i] = 0;
            }
        }
        rlmax = max(rlmax, rl[i]);
    }
    const int nvalid = max(0, min(S.chunk, rlmax - chunk0));
    const int ntiles = (nvalid + 31) / 32;
    const int npg = (nvalid + kPage - 1) / kPage;
    const int row_end = chunk0 + nvalid;
    for (int i = threadIdx.x; i < npg; i += NT) pages[i] = page_of(A, b0, chunk0 / kPage + i);
    if constexpr (!SCORES)
        for (int i = threadIdx.x; i < G * kCoarseBins; i += NT) hist_all[i] = 0u;
    __syncthreads();
    if (ntiles == 0) {
        // nothing of this chunk is visible to any query of the group: an empty
        // candidate set, or (single chunk) an all-padding output row
        if constexpr (!SCORES) {
            for (int i = 0; i < G; i++) {
                const int jj = g * G + i;
                if (jj >= A.num_q) break;
                if (S.n_chunks == 1) {
                    for (int r = threadIdx.x; r < S.topk; r += NT) {
                        S.out_idx[(int64_t)jj * S.topk + r] = -1;
                        if (S.out_score) S.out_score[(int64_t)jj * S.topk + r] = -INFINITY;
                    }
                } else if (threadIdx.x == 0) {
                    S.cand_cnt[(int64_t)jj * S.n_chunks + c] = 0;
                }
            }
        }
        return;   // uniform over the workgroup
    }

    const int my_rl = rl[qi];
    const int j = g * G + qi;
    // query registers first (unconditionally: a clamped index keeps the load in
    // bounds), and all of them in before the copy pipeline starts, so that the
    // only vector-memory operations in flight in the loop are the ring copies
    IdxQuery<MB, D, FP8> q;
    load_query<MB, D>(A, min(j, A.num_q - 1), q);
    wait_vmcnt<0>();

    auto ring = [&](int u) -> uint8_t* {
        return (u == 0 ? ring0 : u == 1 ? ring1 : u == 2 ? ring2 : ring3) + w * GM::TILE;
    };
    auto scl = [&](int u) -> float* { return (u == 0 ? scl0 : u == 1 ? scl1 : u == 2 ? scl2 : scl3) + w * 32; };
    // Loop-invariant per-lane offsets. A tile (32 positions, 32-aligned) lies in
    // one page, so its rows are contiguous: copy r of a tile moves the 16-byte
    // piece gi = 64 r + lane, i.e. row gi / CPR, chunk gi % CPR, stored at the
    // chunk's swizzled place in the slot.
    const int frow = l & 31;   // the tile row (position) this lane reads
    int lds_off[KTile<D, FP8>::NV];
#pragma unroll
    for (int i = 0; i < KTile<D, FP8>::NV; i++) {
        const int cc = KTile<D, FP8>::chunk(i, half);
        lds_off[i] = frow * R + ((cc ^ (frow & GM::SWZ)) << 4);
    }
    // positions [0, lim) of the chunk are visible to this wave's query
    const int lim = min(row_end, my_rl) - chunk0;

    // copy tile ti into this wave's slot (a tile past the end repeats the last
    // page; rows past the visible end are read from the same, valid, page and
    // masked out when scored)
    auto issue = [&](int ti, uint8_t* slot, float* sslot) {
        int page = __builtin_amdgcn_readfirstlane(pages[min(ti >> 1, npg - 1)]);
        page = page < 0 ? 0 : page;
        const int64_t row0 = (int64_t)page * kPage + (ti & 1) * 32;
        const uint8_t* base = A.rows + row0 * R;
#pragma unroll
        for (int r = 0; r < GM::DMA; r++) {
            const int gi = r * kWave + l;
            const int row = gi / CPR, cc = gi % CPR;
            // (the source goes through a named pointer: written inline in the call,
            // the host compile drops the kernel's launch stub)
            const uint8_t* src = base + row * R + ((cc ^ (row & GM::SWZ)) << 4);
            __builtin_amdgcn_global_load_lds(src, (SIA_LDS void*)(slot + r * 1024), 16, 0, 0);
        }
        if constexpr (FP8) {
            const float* ssrc = A.scale + row0 + 4 * l;
            if (l < 8) __builtin_amdgcn_global_load_lds(ssrc, (SIA_LDS void*)sslot, 16, 0, 0);
        }
    };
    // operand reads of tile ti from its slot
    auto fetch = [&](int ti, const uint8_t* slot, const float* sslot, KTile<D, FP8>& t) {
        // the scale is read first: the wait for the row data that the MFMAs need
        // then also covers it, before the slot is refilled
        if constexpr (FP8) t.sc = sslot[frow];
        else t.sc = 1.f;
#pragma unroll
        for (int i = 0; i < KTile<D, FP8>::NV; i++) t.v[i] = *reinterpret_cast<const u32x4*>(slot + lds_off[i]);
        t.ok = frow < lim - ti * 32;   // a tile whose page id is invalid has no visible position
    };
    auto finish = [&](int ti, const f32x16 (&acc)[MB], float tsc, bool tok) {
        const float sc = tile_epilogue<MB, D, FP8>(q, acc, tsc);
        const int i = ti * 32 + frow;
        if constexpr (SCORES) {
            if (l < 32 && tok) S.scores[(int64_t)j * S.ld + chunk0 + i] = sc;
        } else {
            // the key goes to LDS (both lane halves hold the same key and store
            // it to the same place) and into the coarse histogram of its query
            const uint32_t k = tok ? score_key(sc) : 0u;
            keys_all[qi * S.chunk + i] = k;
            if (l < 32 && k != 0u) atomicAdd(&hist_all[qi * kCoarseBins + coarse_bin(k)], 1u);
        }
    };

    const bool active = my_rl > chunk0 && sub < ntiles;
    if (active) {
        // this wave's tiles: sub + k * WPQ; slot of the k-th: k % NS
#pragma unroll
        for (int u = 0; u < NS - 1; u++) issue(sub + u * WPQ, ring(u), scl(u));
        f32x16 acc0[MB], acc1[MB];
        float sc0 = 0.f, sc1 = 0.f;
        bool ok0 = false, ok1 = false;
        int prev = -1;
        for (int k0 = 0; sub + k0 * WPQ < ntiles; k0 += 2 * NS) {
#pragma unroll
            for (int u = 0; u < 2 * NS; u++) {
                const int ti = sub + (k0 + u) * WPQ;
                if (ti < ntiles) {
                    issue(ti + (NS - 1) * WPQ, ring((u + NS - 1) % NS), scl((u + NS - 1) % NS));
                    wait_vmcnt<(NS - 1) * GM::PER_TILE>();   // this tile's copies have landed
                    KTile<D, FP8> t;
                    fetch(ti, ring(u % NS), scl(u % NS), t);
                    // MFMAs of this tile, then the vector epilogue of the previous one
                    if (u % 2 == 0) {
                        tile_mfma<MB, D, FP8>(q, t, acc0);
                        sc0 = t.sc; ok0 = t.ok;
                        if (prev >= 0) finish(prev, acc1, sc1, ok1);
                    } else {
                        tile_mfma<MB, D, FP8>(q, t, acc1);
                        sc1 = t.sc; ok1 = t.ok;
                        finish(prev, acc0, sc0, ok0);
                    }
                    prev = ti;
                }
            }
        }
        // epilogue of the last tile: its parity is the count of tiles of this wave
        const int count = (ntiles - sub + WPQ - 1) / WPQ;
        if (count % 2 == 1) finish(prev, acc0, sc0, ok0);
        else finish(prev, acc1, sc1, ok1);
    } else if constexpr (!SCORES) {
        // a query that sees nothing of this chunk still needs zero keys
        for (int i = sub * kWave + l; i < ntiles * 32; i += WPQ * kWave) keys_all[qi * S.chunk + i] = 0u;
    }
    wait_vmcnt<0>();
    if constexpr (SCORES) return;
    else {
        __syncthreads();
        // ---- per-query selection over the chunk
        const int nscan = ntiles * 32;
#pragma unroll
        for (int i = 0; i < G; i++) {
            const int jj = g * G + i;
            if (jj >= A.num_q) break;
            const uint32_t* keys = keys_all + i * S.chunk;
            const uint32_t* hist = hist_all + i * kCoarseBins;
            if (S.n_chunks == 1) {
                int32_t* oi = S.out_idx + (int64_t)jj * S.topk;
                float* os = S.out_score ? S.out_score + (int64_t)jj * S.topk : nullptr;
                const int m = select_emit_coarse<NT>(keys, nscan, hist, S.topk, sel, EmitFinal{oi, os, chunk0});
                for (int r = m + threadIdx.x; r < S.topk; r += NT) {
                    oi[r] = -1;
                    if (os) os[r] = -INFINITY;
                }
            } else {
                const int64_t slot = (int64_t)jj * S.n_chunks + c;
                const int m = select_emit_coarse<NT>(
                    keys, nscan, hist, S.kc, sel,
                    EmitCand{S.cand_key + slot * S.kc, S.cand_pos + slot * S.kc, chunk0});
                if (threadIdx.x == 0) S.cand_cnt[slot] = m;
            }
            __syncthreads();
        }
    }
}

// Largest chunk (power of two, <= 16384) whose LDS fits next to the ring.
template <int MB, int D, bool FP8, int G>
static int split_chunk_cap() {
    using GM = SplitGeom<D, FP8, G>;
    for (int chunk = 16384; chunk >= 64; chunk >>= 1) {
        const size_t dyn = split_pages_bytes(chunk) + (size_t)G * (chunk + kCoarseBins) * 4 + sizeof(SelScratch);
        if (GM::STATIC_LDS + dyn + 256 <= GM::LDS_BUDGET) return chunk;
    }
    return 64;
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

// Rank -> candidate index, kept in LDS; positions are gathered afterwards in
// one parallel pass instead of one dependent load per compaction round.
struct EmitRank {
    int32_t* rank_idx;
    __device__ void prefetch(int, u32x4, uint32_t) {}
    __device__ void prefetch2(int, u32x4, uint32_t) {}
    __device__ void operator()(int rank, int i, int, uint32_t) const { rank_idx[rank] = i; }
};

__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(MergeArgs M) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint32_t* keys = reinterpret_cast<uint32_t*>(smem);
    const int q = blockIdx.x / M.n_out;
    const int o = blockIdx.x % M.n_out;
    const int s0 = o * M.fan_in;
    const int nsets = min(M.fan_in, M.n_in - s0);
    const int n = nsets * M.kc_in;
    uint32_t* hist = keys + (size_t)M.fan_in * M.kc_in;
    int32_t* rank_idx = reinterpret_cast<int32_t*>(hist + kCoarseBins);     // [topk]
    int* cnt = rank_idx + M.topk;                                          // [fan_in]
    SelScratch* sel = reinterpret_cast<SelScratch*>(cnt + (M.fan_in + 3) / 4 * 4);
    const int64_t set0 = (int64_t)q * M.n_in + s0;
    for (int i = threadIdx.x; i < kCoarseBins; i += kMergeThreads) hist[i] = 0u;
    for (int i = threadIdx.x; i < nsets; i += kMergeThreads) cnt[i] = M.in_cnt[set0 + i];
    __syncthreads();
    // candidate keys: independent loads, several in flight per thread
    const uint32_t* src = M.in_key + set0 * M.kc_in;
    constexpr int U = 32;
    for (int i0 = threadIdx.x; i0 < n; i0 += kMergeThreads * U) {
        uint32_t k[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int i = i0 + u * kMergeThreads;
            const int set = i / M.kc_in;
            k[u] = (i < n && i - set * M.kc_in < cnt[min(set, nsets - 1)]) ? src[i] : 0u;
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int i = i0 + u * kMergeThreads;
            if (i < n) keys[i] = k[u];
        }
    }
    __syncthreads();
    for (int i = threadIdx.x * 4; i < n; i += kMergeThreads * 4) {
        const u32x4 k4 = *reinterpret_cast<const u32x4*>(keys + i);
#pragma unroll
        for (int e = 0; e < 4; e++) hist_add(hist, coarse_bin(k4[e]), i + e < n && k4[e] != 0u);
    }
    __syncthreads();
    const int m = select_emit_coarse<kMergeThreads>(keys, n, hist, M.topk, sel, EmitRank{rank_idx});
    __syncthreads();
    const int32_t* src_pos = M.in_pos + set0 * M.kc_in;
    if (M.out_idx) {
        int32_t* oi = M.out_idx + (int64_t)q * M.topk;
        float* os = M.out_score ? M.out_score + (int64_t)q * M.topk : nullptr;
        for (int r = threadIdx.x; r < M.topk; r += kMergeThreads) {
            if (r < m) {
                const int i = rank_idx[r];
                oi[r] = src_pos[i];
                if (os) os[r] = key_score(keys[i]);
            } else {
                oi[r] = -1;
                if (os) os[r] = -INFINITY;
            }
        }
    } else {
        const int64_t slot = (int64_t)q * M.n_out + o;
        uint32_t* ok = M.out_key + slot * M.topk;
        int32_t* op = M.out_pos + slot * M.topk;
        for (int r = threadIdx.x; r < m; r += kMergeThreads) {
            const int i = rank_idx[r];
            ok[r] = keys[i];
            op[r] = src_pos[i];
        }
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
__device__ void stream_query(const IdxArgs& A, const StreamArgs& S, int j, int rl, const int* pages,
                             WaveBuf B) {
    const int l = lane_id();
    int32_t* oi = S.out_idx + (int64_t)j * S.topk;
    float* os = S.out_score ? S.out_score + (int64_t)j * S.topk : nullptr;
    int cnt = 0;
    uint32_t tau = 0u;
    const int ntiles = (rl + 31) / 32;
    if (ntiles > 0) {
        IdxQuery<MB, D, FP8> q;
        load_query<MB, D>(A, j, q);
        const int npages = (rl + kPage - 1) / kPage;
        auto fetch = [&](KTile<D, FP8>& t, int ti) {   // ti past the end: dummy row
            const int page = __builtin_amdgcn_readfirstlane(pages[min(ti >> 1, npages - 1)]);
            load_ktile<D, FP8>(A, page, ti * 32, ti < ntiles ? rl : 0, t);
        };
        auto consume = [&](const KTile<D, FP8>& t, int ti) {
            const float sc = tile_scores<MB, D, FP8>(q, t);
            const int p = ti * 32 + (l & 31);
            const uint32_t k = (l < 32 && t.ok) ? score_key(sc) : 0u;
            const bool take = k > tau;
            const uint64_t mask = __ballot(take);
            if (take) {
                const int at = cnt + lanes_below(mask);
                B.key[at] = k;
                B.pos[at] = p;
            }
            cnt += __popcll(mask);
            if (cnt > S.cap - 32) {
                // keep exactly the Top-K seen so far; later ties of T lose to them
                wave_sync();
                int ties;
                const int n4 = (cnt + 3) & ~3;
                for (int i = cnt + l; i < n4; i += kWave) B.key[i] = 0u;
                wave_sync();
                const uint32_t T = radix_threshold<kWave>(B.key, n4, S.topk, B.sel, ties);
                ordered_compact<kWave, true>(B.key, n4, T, ties, B.sel, EmitInPlace{B.key, B.pos, {}});
                cnt = S.topk;
                tau = T;
                wave_sync();
            }
        };
        constexpr int kPrefetch = 4;   // K tiles in flight per wave
        KTile<D, FP8> buf[kPrefetch];
#pragma unroll
        for (int d = 0; d < kPrefetch; d++) fetch(buf[d], d);
        int t = 0;
        for (; t + kPrefetch - 1 < ntiles; t += kPrefetch) {
#pragma unroll
            for (int d = 0; d < kPrefetch; d++) {
                consume(buf[d], t + d);
                fetch(buf[d], t + d + kPrefetch);
            }
        }
#pragma unroll
        for (int d = 0; d < kPrefetch - 1; d++)
            if (t + d < ntiles) consume(buf[d], t + d);
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

__host__ __device__ inline size_t stream_wave_bytes(int cap) { return (size_t)cap * 8 + sizeof(SelScratch); }
__host__ __device__ inline size_t stream_smem_bytes(int cap, int max_visible) {
    return 4 * stream_wave_bytes(cap) + ((size_t)(max_visible + kPage - 1) / kPage * 4 + 15) / 16 * 16;
}

template <int MB, int D, bool FP8>
__global__ __launch_bounds__(kStreamThreads) void indexer_stream_kernel(IdxArgs A, StreamArgs S) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ int next_tile;
    __shared__ int tile_seq, tile_rows;
    constexpr int QPT = kStreamThreads / kWave;   // queries per tile, one per wave
    const int w = threadIdx.x / kWave;
    uint8_t* base = smem + w * stream_wave_bytes(S.cap);
    WaveBuf B{reinterpret_cast<uint32_t*>(base), reinterpret_cast<int32_t*>(base + (size_t)S.cap * 4),
              reinterpret_cast<SelScratch*>(base + (size_t)S.cap * 8)};
    int* pages = reinterpret_cast<int*>(smem + QPT * stream_wave_bytes(S.cap));

    // One tile: four consecutive queries of one sequence. Their page ids are staged
    // once in LDS; a query of another sequence is dropped (status bit).
    auto run_tile = [&](int tile) {
        const int j = tile * QPT + w;
        int b = 0, rl = 0;
        if (j < A.num_q) rl = visible_len(A, j, b);
        if (w == 0 && lane_id() == 0) tile_seq = b;
        __syncthreads();
        const int b0 = tile_seq;
        if (j < A.num_q && b != b0) {
            if (lane_id() == 0) atomicOr(A.status, kBadSeq);
            rl = 0;
        }
        // longest row of the tile
        if (w == 0 && lane_id() == 0) tile_rows = 0;
        __syncthreads();
        if (lane_id() == 0) atomicMax(&tile_rows, rl);
        __syncthreads();
        const int npg = (tile_rows + kPage - 1) / kPage;
        for (int i = threadIdx.x; i < npg; i += kStreamThreads) pages[i] = page_of(A, b0, i);
        __syncthreads();
        if (j < A.num_q) stream_query<MB, D, FP8>(A, S, j, rl, pages, B);
        __syncthreads();
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
    constexpr int NT = SplitGeom<D, FP8, G>::NT;
    const int groups = (a.num_q + G - 1) / G;
    const size_t smem = split_pages_bytes(s.chunk) +
                        (SC ? 0 : (size_t)G * (s.chunk + kCoarseBins) * 4 + sizeof(SelScratch));
    auto k = indexer_split_kernel<MB, D, FP8, G, SC>;
    hipError_t e = set_smem(k, smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(groups * s.n_chunks), dim3(NT), smem, st, a, s);
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

int indexer_split_chunk_cap(int mb, int dim, bool fp8, int group) {
#define SIA_CAP(MBv, Dv, F8)                                                              \
    if (mb == MBv && dim == Dv && fp8 == F8)                                              \
        return group == 2 ? split_chunk_cap<MBv, Dv, F8, 2>() : split_chunk_cap<MBv, Dv, F8, 1>();
    SIA_CAP(1, 64, false) SIA_CAP(1, 64, true) SIA_CAP(1, 128, false) SIA_CAP(1, 128, true)
    SIA_CAP(2, 64, false) SIA_CAP(2, 64, true) SIA_CAP(2, 128, false) SIA_CAP(2, 128, true)
#undef SIA_CAP
    return 2048;
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
    const size_t smem = ((size_t)m.fan_in * m.kc_in + kCoarseBins + m.topk + (m.fan_in + 3) / 4 * 4) * 4 +
                        sizeof(SelScratch);
    hipError_t e = set_smem(topk_merge_kernel, smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_merge_kernel, dim3(m.num_q * m.n_out), dim3(kMergeThreads), smem, st, m);
    return hipGetLastError();
}

template <int MB, int D, bool FP8>
static hipError_t stream_launch(const IdxArgs& a, const StreamArgs& s, int grid, hipStream_t st) {
    auto k = indexer_stream_kernel<MB, D, FP8>;
    const size_t smem = stream_smem_bytes(s.cap, a.max_visible);
    hipError_t e = set_smem(k, smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(grid), dim3(kStreamThreads), smem, st, a, s);
    return hipGetLastError();
}

template <int MB, int D, bool FP8>
static int stream_occupancy(int cap, int max_visible) {
    auto k = indexer_stream_kernel<MB, D, FP8>;
    const size_t smem = stream_smem_bytes(cap, max_visible);
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

size_t indexer_stream_smem(int cap, int max_visible) { return stream_smem_bytes(cap, max_visible); }

int indexer_stream_blocks_per_cu(int mb, int dim, bool fp8, int cap, int max_visible) {
#define SIA_OCC(MBv, Dv, F8) \
    if (mb == MBv && dim == Dv && fp8 == F8) return stream_occupancy<MBv, Dv, F8>(cap, max_visible);
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
