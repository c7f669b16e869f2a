// Lightweight indexer + exact Top-K for gfx950.
//
// score[j,s] = sigma_s * sum_h w[j,h] * max(0, q[j,h,:] . k_s)
//
// The q . k products of one query against 32 positions are one MFMA tile:
// heads are the M dimension (32 per block), positions the N dimension, the
// index dim the K dimension. Queries sit in registers for the whole pass; a
// lane supplies its position's half-row of index-K, staged through LDS by
// direct global -> LDS copies (a private ring per team in the decode score pass,
// one ring shared by the four queries of a workgroup in the stream kernel). The
// accumulator puts 16 heads of one position in each lane, so the
// ReLU, the head weights and the head sum stay in registers with a single
// cross-lane add, and sigma_s multiplies the sum ("Rapid Adaptation and
// Inference Optimization", section 4.1 "Indexer Fusion": the indexer reads the
// paged K cache directly and hands on only the selection).
//
// Launch shapes (all score through tile_mfma + tile_epilogue, so a query and a
// position give the same bits everywhere, and all select with sia_select.h):
//  * decode, score pass + selection pass: the score pass streams parts of the
//    rows (two draft tokens of a sequence share every copy). A position's
//    order-preserving key is kept only if it reaches the part's running floor
//    (the coarse bin of the part's K-th largest kept key, raised as the pass
//    goes); kept keys and positions are appended to per-team candidate lists,
//    with a coarse histogram per part. No per-position score or key is
//    written. The selection pass takes each row's exact Top-K from its lists.
//  * prefill, stream: one wave walks one query's whole causal row (the four
//    waves of a workgroup walk four consecutive queries over one shared ring of
//    K tiles), appending positions that beat the current threshold to an LDS
//    buffer kept in position order, and re-selecting the Top-K when the buffer
//    fills. A position that ties the threshold arrives after every kept one, so
//    it can be dropped.
#include "sia_device.h"
#include "sia_kernels.h"
#include "sia_sched.h"
#include "sia_select.h"

namespace sia {

static_assert(kCoarseBins == kCoarseBinsHost, "host and device histogram sizes differ");

// XOR applied to the 16-byte chunk index of row `row` of a tile of rows with
// CPR chunks each, staged in LDS. The operand reads take one chunk of 16
// consecutive rows per 16 lanes; with 64 banks of 4 bytes, rows of CPR chunks
// repeat their bank pattern every 16 / CPR rows, so the XOR takes the row
// index divided by that (8 chunks: (row / 2) % 8), which puts the 16 reads on
// 16 distinct bank groups. The XOR stays inside the row.
template <int CPR>
__device__ __forceinline__ int row_swz(int row) {
    static_assert(CPR == 4 || CPR == 8 || CPR == 16, "rows of 64, 128 or 256 bytes");
    return (row / (16 / CPR)) & (CPR - 1);
}

// ------------------------------------------------------------ score tile

// A query's indexer heads in MFMA operand layout, one form per index-row
// format KF.
//  * bf16 rows (kRowBf16): 32x32x16 bf16 MFMAs on the bf16 query.
//  * fp8 rows with a per-token scale (kRowFp8): 32x32x64 fp8 MFMAs on the raw
//    e4m3 key bytes. X = q * 2^s is split into an e4m3 high part hi = e4m3(X)
//    and an e4m3 residual lo = e4m3(16 (X - hi)) (one exponent s per query,
//    chosen so that max|q| * 2^s lies in [128, 256)), and the two products are
//    summed with MFMA scales 2^-s and 2^-(s+4). The split is exact wherever
//    |X| >= 2^-6 (e4m3's smallest normal), which covers every element with
//    |q| >= 2^-13 max|q|; below that the residual falls into e4m3's subnormal
//    steps and the element is represented to within 2^-14 2^-s <=
//    2^-21 max|q|. The scores therefore equal those of the bf16 form up to
//    rounding order and that error on the smallest elements.
//  * MXFP8 rows (kRowMx): the query is MXFP8 too (e4m3 elements, one E8M0
//    scale per 32 consecutive elements of a head), so one 32x32x64 fp8 MFMA per
//    64-wide step takes both operands' block scales per lane: lane half h
//    holds the h-th 16 bytes of each of the step's two blocks and supplies the
//    scale of block h, which the MFMA applies to both halves of that block
//    (A: the head's query, B: the position's row). Products of the dequantized
//    values are exact in fp32.
template <int MB, int D, int KF>
struct IdxQuery;

template <int MB, int D>
struct IdxQuery<MB, D, kRowBf16> {
    static constexpr int KS = D / 16;
    bf16x8 a[MB][KS];
    float w[MB][16];
};

template <int MB, int D>
struct IdxQuery<MB, D, kRowFp8> {
    static constexpr int KS = D / 64;
    i32x8 hi[MB][KS], lo[MB][KS];
    int sh, sl;   // E8M0 scales of the two parts
    float w[MB][16];
};

template <int MB, int D>
struct IdxQuery<MB, D, kRowMx> {
    static constexpr int KS = D / 64;
    i32x8 a[MB][KS];
    int sa[MB][KS];   // this lane's E8M0 block scale per step
    float w[MB][16];
};

// MFMAs per query, 32-position tile and 32-head block.
template <int D, int KF>
__host__ __device__ constexpr int mfmas_per_block() {
    return KF == kRowBf16 ? D / 16 : KF == kRowFp8 ? 2 * (D / 64) : D / 64;
}

// hb0: first head block (of 32 heads) held, for waves that split a query's heads.
template <int MB, int D>
__device__ __forceinline__ void load_weights(const IdxArgs& A, int j, float (&w)[MB][16], int hb0 = 0) {
    const int half = lane_id() >> 5;
#pragma unroll
    for (int mb = 0; mb < MB; mb++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int h = (hb0 + mb) * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            w[mb][r] = h < A.heads ? A.w[(int64_t)j * A.heads + h] : 0.f;
        }
}

template <int MB, int D>
__device__ __forceinline__ void load_query(const IdxArgs& A, int j, IdxQuery<MB, D, kRowMx>& q, int hb0 = 0) {
    constexpr int KS = IdxQuery<MB, D, kRowMx>::KS;
    const int l = lane_id(), m = l & 31, half = l >> 5;
    // lane l: head (hb0 + mb)*32 + l%32; of step ks, the (l/32)-th 16 bytes of
    // block 2 ks (operand bytes 0-15) and of block 2 ks + 1 (bytes 16-31), and
    // the scale of block 2 ks + l/32 (the MFMA applies lane half h's scale to
    // k 32h .. 32h + 31 of both halves); heads past the count give zero codes
#pragma unroll
    for (int mb = 0; mb < MB; mb++) {
        const int head = (hb0 + mb) * 32 + m;
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
            int sc = 127;
            if (head < A.heads) {
                const uint8_t* src = A.q8 + ((int64_t)j * A.heads + head) * D + ks * 64 + half * 16;
                v0 = *reinterpret_cast<const u32x4*>(src);
                v1 = *reinterpret_cast<const u32x4*>(src + 32);
                sc = A.q8s[((int64_t)j * A.heads + head) * (D / 32) + 2 * ks + half];
            }
            q.a[mb][ks] = i32x8{(int)v0[0], (int)v0[1], (int)v0[2], (int)v0[3],
                                (int)v1[0], (int)v1[1], (int)v1[2], (int)v1[3]};
            q.sa[mb][ks] = sc;
        }
    }
    load_weights<MB, D>(A, j, q.w, hb0);
}

template <int MB, int D>
__device__ __forceinline__ void load_query(const IdxArgs& A, int j, IdxQuery<MB, D, kRowBf16>& q, int hb0 = 0) {
    const int l = lane_id(), m = l & 31, half = l >> 5;
#pragma unroll
    for (int mb = 0; mb < MB; mb++) {
        const int head = (hb0 + mb) * 32 + m;
#pragma unroll
        for (int ks = 0; ks < IdxQuery<MB, D, kRowBf16>::KS; ks++) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (head < A.heads)
                v = *reinterpret_cast<const u32x4*>(
                    A.q_idx + ((int64_t)j * A.heads + head) * D + half * (D / 2) + ks * 8);
            q.a[mb][ks] = as_bf16x8(v);
        }
    }
    load_weights<MB, D>(A, j, q.w, hb0);
}

template <int MB, int D>
__device__ __forceinline__ void load_query(const IdxArgs& A, int j, IdxQuery<MB, D, kRowFp8>& q, int hb0 = 0) {
    constexpr int KS = IdxQuery<MB, D, kRowFp8>::KS;
    const int l = lane_id(), m = l & 31, half = l >> 5;
    // lane l holds head (hb0 + mb)*32 + l%32 and dims 64 ks + 32 (l/32) .. +31 of
    // each step; the query is read twice (the second time from cache): once for
    // the largest magnitude over all its heads (one exponent per query, whatever
    // share of the heads a wave holds), once to split it
    auto ld = [&](int blk, int ks, int c) -> u32x4 {
        const int head = blk * 32 + m;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (head < A.heads)
            v = *reinterpret_cast<const u32x4*>(
                A.q_idx + ((int64_t)j * A.heads + head) * D + ks * 64 + half * 32 + c * 8);
        return v;
    };
    float amax = 0.f;
#pragma unroll
    for (int blk = 0; blk < 2; blk++)   // every head block (64 heads at most)
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const u32x4 v = ld(blk, ks, c);
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
                const u32x4 v = ld(hb0 + mb, ks, c);
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
    load_weights<MB, D>(A, j, q.w, hb0);
}

// One lane's share of a 32-position tile: half a row of index-K (+ its scale).
// bf16: lane half h holds the row's chunks h*CPR/2 .. (16-byte chunks, the
// 32x32x16 operand layout); fp8: for each 64-byte MFMA step ks it holds the 32
// bytes 64 ks + 32 h .. (chunks 4 ks + 2 h and 4 ks + 2 h + 1).
template <int D, int KF>
struct KTile {
    static constexpr int BYTES = (D / 2) * ((KF != kRowBf16) ? 1 : 2);
    static constexpr int NV = BYTES / 16;
    u32x4 v[NV];
    float sc;     // fp8 rows: the token scale; MXFP8 rows: the row's E8M0 block scales (bytes, as bits)
    bool ok;      // this lane's position is visible and its page id valid
    // 16-byte chunk of the row held in v[i] by lane half h. In a 64-element
    // step of the fp8 MFMA, lane half h holds bytes 0-15 at k 16h.. and bytes
    // 16-31 at k 32 + 16h..; a block scale covers k 0..31 (from lane half 0)
    // or 32..63 (from lane half 1). MXFP8 rows follow that layout (chunks
    // 4 ks + h and 4 ks + 2 + h); fp8 rows with one scale per token may use
    // any order shared with the query, and take 32 contiguous bytes.
    static __device__ __forceinline__ int chunk(int i, int h) {
        if constexpr (KF == kRowMx) return 4 * (i >> 1) + 2 * (i & 1) + h;
        else if constexpr (KF != kRowBf16) return 4 * (i >> 1) + 2 * h + (i & 1);
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
template <int D, int KF>
__device__ __forceinline__ void load_ktile(const IdxArgs& A, int page, int pos0, int row_len,
                                           KTile<D, KF>& t) {
    const int l = lane_id(), half = l >> 5;
    const int p = pos0 + (l & 31);
    t.ok = page >= 0 && p < row_len;
    const int64_t row = t.ok ? (int64_t)page * kPage + (p & 63) : 0;
    const uint8_t* src = A.rows + row * (D * ((KF != kRowBf16) ? 1 : 2));
#pragma unroll
    for (int i = 0; i < KTile<D, KF>::NV; i++)
        t.v[i] = reinterpret_cast<const u32x4*>(src)[KTile<D, KF>::chunk(i, half)];
    if constexpr (KF != kRowBf16) t.sc = A.scale[row];
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
template <int MB, int D, int KF>
__device__ __forceinline__ void tile_mfma(const IdxQuery<MB, D, KF>& q, const KTile<D, KF>& t,
                                          f32x16 (&acc)[MB]) {
#pragma unroll
    for (int mb = 0; mb < MB; mb++) acc[mb] = f32x16{};
    if constexpr (KF == kRowMx) {
        constexpr int KS = D / 64;
        // the row's four E8M0 bytes; this lane's block of step ks is 2 ks + lane/32
        const uint32_t rs = __float_as_uint(t.sc) >> (8 * (lane_id() >> 5));
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            const u32x4 v0 = t.v[2 * ks], v1 = t.v[2 * ks + 1];
            const i32x8 b = {(int)v0[0], (int)v0[1], (int)v0[2], (int)v0[3],
                             (int)v1[0], (int)v1[1], (int)v1[2], (int)v1[3]};
            const int sb = (int)((rs >> (16 * ks)) & 0xffu);
#pragma unroll
            for (int mb = 0; mb < MB; mb++)
                acc[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(q.a[mb][ks], b, acc[mb], 0, 0, 0,
                                                                          q.sa[mb][ks], 0, sb);
        }
    } else if constexpr (KF == kRowFp8) {
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

// Vector half: ReLU, head weights and head sum, block by block: each block of 32
// heads is summed on its own and the block sums are added in block order, so a
// wave holding one block of a query gives the same bits once its partner's block
// sum is added.
template <int MB, int D, int KF>
__device__ __forceinline__ float tile_head_sum(const IdxQuery<MB, D, KF>& q, const f32x16 (&acc)[MB]) {
    float v = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; mb++) {
        float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
            p0 = fmaf(q.w[mb][r + 0], relu(acc[mb][r + 0]), p0);
            p1 = fmaf(q.w[mb][r + 1], relu(acc[mb][r + 1]), p1);
            p2 = fmaf(q.w[mb][r + 2], relu(acc[mb][r + 2]), p2);
            p3 = fmaf(q.w[mb][r + 3], relu(acc[mb][r + 3]), p3);
        }
        const float b = add_halves((p0 + p1) + (p2 + p3));
        v = mb == 0 ? b : v + b;
    }
    return v;
}

// ... times the token scale.
template <int MB, int D, int KF>
__device__ __forceinline__ float tile_epilogue(const IdxQuery<MB, D, KF>& q, const f32x16 (&acc)[MB],
                                               float tsc) {
    const float v = tile_head_sum<MB, D, KF>(q, acc);
    return KF == kRowFp8 ? v * tsc : v;
}

// Scores of the tile's 32 positions for one query; lanes l and l+32 both get
// the score of position pos0 + l%32 (undefined where the tile lane is not ok).
// Every kernel scores through tile_mfma + tile_epilogue, so a query and position
// give the same bits in each of them.
template <int MB, int D, int KF>
__device__ __forceinline__ float tile_scores(const IdxQuery<MB, D, KF>& q, const KTile<D, KF>& t) {
    f32x16 acc[MB];
    tile_mfma<MB, D, KF>(q, t, acc);
    return tile_epilogue<MB, D, KF>(q, acc, t.sc);
}

// ------------------------------------------------------------ emitters

// Output rows hold `cap` entries; a rank past them (only possible if a row's
// histogram and keys disagreed) is dropped rather than written out of bounds.
struct EmitFinal {
    int32_t* idx;
    float* score;
    int base;        // position of key index 0
    int cap;
    __device__ void prefetch(int, u32x4, uint32_t) {}
    __device__ void prefetch2(int, u32x4, uint32_t) {}
    __device__ void operator()(int rank, int i, int, uint32_t k) const {
        if (rank >= cap) return;
        idx[rank] = base + i;
        if (score) score[rank] = key_score(k);
    }
};

// In-place compaction of a stream wave's candidate buffer (global memory):
// positions of the round are read before any of the round's writes, as two
// 16-byte groups issued together with the keys (the buffer holds cap + 64
// entries, so the groups stay inside it), so that a round costs one memory
// round trip.
struct EmitInPlace {
    uint32_t* key;
    int32_t* pos;
    int32_t p4[8];
    __device__ void prefetch(int i, u32x4, uint32_t) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(pos + i);
#pragma unroll
        for (int e = 0; e < 4; e++) p4[e] = (int32_t)v[e];
    }
    __device__ void prefetch2(int i, u32x4, uint32_t) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(pos + i);
#pragma unroll
        for (int e = 0; e < 4; e++) p4[4 + e] = (int32_t)v[e];
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
    int cap;
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
        if (rank >= cap) return;
        idx[rank] = p4[e];
        if (score) score[rank] = key_score(k);
    }
};

// The stream kernel's final emission from a wave's candidate buffer (global
// memory, cap + 64 entries): positions read as 16-byte groups beside the keys.
struct EmitFinalStream {
    const int32_t* pos;
    int32_t* idx;
    float* score;
    int cap;
    int32_t p4[8];
    __device__ void prefetch(int i, u32x4, uint32_t) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(pos + i);
#pragma unroll
        for (int e = 0; e < 4; e++) p4[e] = (int32_t)v[e];
    }
    __device__ void prefetch2(int i, u32x4, uint32_t) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(pos + i);
#pragma unroll
        for (int e = 0; e < 4; e++) p4[4 + e] = (int32_t)v[e];
    }
    __device__ void operator()(int rank, int, int e, uint32_t k) const {
        if (rank >= cap) return;
        idx[rank] = p4[e];
        if (score) score[rank] = key_score(k);
    }
};

// Select the top min(m_cap, cnt) of keys[0..n) and emit them in index order;
// cnt = the number of nonzero keys, known to the caller.
template <int NT, typename Emit>
__device__ int select_emit(const uint32_t* keys, int n, int cnt, int m_cap, SelScratch* s, Emit&& emit,
                           uint32_t* spare = nullptr) {
    const int m = min(m_cap, cnt);
    if (m <= 0) return 0;
    if (m == cnt) {
        ordered_compact<NT>(keys, n, 0u, 0, s, emit);   // every nonzero key
    } else {
        int ties;
        const uint32_t T = radix_threshold<NT>(keys, n, m, s, ties, spare);
        ordered_compact<NT>(keys, n, T, ties, s, emit);
    }
    return m;
}

// ------------------------------------------------------------ score pass (decode)

// Geometry of the score pass. Eight waves; the waves of query qi (8/G of them)
// split the part's tiles of 32 positions into contiguous runs, one run per
// wave. Each wave streams its run through a private ring of NS LDS slots filled
// by direct global -> LDS copies, 16 bytes per lane and eight lanes per
// 128-byte row (coalesced), with the 16-byte chunks of a row XOR-swizzled by
// the row index so that the MFMA operand reads spread over the LDS banks. The
// copies are addressed from scalar registers (page base) plus a loop-invariant
// lane offset. A wave only waits on its own copies (no barrier in the loop);
// it issues the MFMAs of tile k, the copy of tile k + NS - 1, the vector
// epilogue of tile k - 1, then reads tile k + 1's operands, so the matrix pipe,
// the vector pipe and the copies overlap. With two queries the waves of a pair
// copy the same rows at about the same time; the second copy is served from L2.
template <int D, int KF, int G>
struct RowsGeom {
    static constexpr int R = D * ((KF != kRowBf16) ? 1 : 2);          // bytes per row
    static constexpr int CPR = R / 16;                   // 16-byte chunks per row
    static constexpr int NWV = kRowsThreads / kWave;
    static constexpr int WPQ = NWV / G;                  // waves per query
    static constexpr int TILE = 32 * R;                  // bytes of one tile
    static constexpr int DMA = TILE / 1024;              // 1 KB copies per tile
    static constexpr int PER_TILE = DMA + ((KF != kRowBf16) ? 1 : 0); // copies per tile (+ scales)
    static constexpr int SLOT = TILE + ((KF != kRowBf16) ? 256 : 0);  // (+ the scales of the tile's page)
    static constexpr size_t FIXED = (size_t)G * kCoarseBins * 4 + kMaxPartPages * 4 + 512;
    static constexpr int NS_FIT = (int)((kMaxLds - FIXED) / ((size_t)NWV * SLOT));
    static constexpr int NS = NS_FIT > 4 ? 4 : NS_FIT;   // ring depth
    static constexpr int U = NS % 2 == 0 ? NS : 2 * NS;  // unroll: static slot and accumulator
    static_assert(NS >= 2, "the ring needs two slots per wave");
};

template <int MB, int D, int KF, int G, bool SCORES>
__global__ __launch_bounds__(kRowsThreads) void indexer_rows_kernel(IdxArgs A, RowsArgs S) {
    using GM = RowsGeom<D, KF, G>;
    constexpr int NS = GM::NS, R = GM::R, CPR = GM::CPR, NWV = GM::NWV, WPQ = GM::WPQ, U = GM::U;
    constexpr int SLOT = GM::SLOT, NV = KTile<D, KF>::NV;
    __shared__ __attribute__((aligned(16))) uint8_t ring[NS * NWV * SLOT];
    __shared__ int pages[kMaxPartPages];
    __shared__ __attribute__((aligned(16))) uint32_t hist[SCORES ? 4 : G * kCoarseBins];
    __shared__ uint32_t floor_key[G];   // keys below it are not kept (>= 1)

    const int g = blockIdx.x / S.n_parts;
    const int part = blockIdx.x % S.n_parts;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int l = lane_id(), half = l >> 5, frow = l & 31;
    const int qi = w / WPQ, sub = w % WPQ;
    const int pos0 = part * S.part;

    // The group's queries share one sequence; a query naming another sequence is
    // dropped (status bit) rather than scored against the wrong cache.
    int b0 = 0, rlmax = 0, my_rl = 0;
#pragma unroll
    for (int i = 0; i < G; i++) {
        const int jj = g * G + i;
        int r = 0;
        if (jj < A.num_q) {
            int b;
            r = visible_len(A, jj, b);
            if (i == 0) b0 = b;
            else if (b != b0) {
                if (threadIdx.x == 0) atomicOr(A.status, kBadSeq);
                r = 0;
            }
            if (!SCORES && part == 0 && threadIdx.x == 0) S.row_len[jj] = r;
        }
        rlmax = max(rlmax, r);
        if (i == qi) my_rl = r;
    }
    // wave-uniform (the copies are addressed from scalar registers)
    b0 = __builtin_amdgcn_readfirstlane(b0);
    rlmax = __builtin_amdgcn_readfirstlane(rlmax);
    my_rl = __builtin_amdgcn_readfirstlane(my_rl);
    const int nvalid = max(0, min(S.part, rlmax - pos0));
    const int npg = (nvalid + kPage - 1) / kPage;
    for (int i = threadIdx.x; i < npg; i += kRowsThreads) pages[i] = page_of(A, b0, pos0 / kPage + i);
    if constexpr (!SCORES) {
        for (int i = threadIdx.x; i < G * kCoarseBins; i += kRowsThreads) hist[i] = 0u;
        if (threadIdx.x < G) floor_key[threadIdx.x] = 1u;
    }
    __syncthreads();

    // this wave's run: tiles t0 .. t0 + n - 1 of the part (an even count per wave,
    // so that a run starts on a page)
    const int j = g * G + qi;
    const int my_valid = max(0, min(S.part, my_rl - pos0));
    const int my_tiles = (my_valid + 31) / 32;
    const int tpw = ((my_tiles + WPQ - 1) / WPQ + 1) & ~1;
    const int t0 = sub * tpw;
    const int n = max(0, min(tpw, my_tiles - t0));
    const int64_t rowbase = (int64_t)j * S.ld + pos0;
    const int rbase = pos0 + t0 * 32;   // first entry of this wave's candidate region
    int cnt = 0;                        // candidates appended

    if (n > 0) {
        // copy r of a tile moves the 16-byte piece gi = 64 r + lane: row gi / CPR,
        // chunk gi % CPR, stored at the chunk's swizzled place in the slot
        uint32_t voff[GM::DMA];
#pragma unroll
        for (int r = 0; r < GM::DMA; r++) {
            const int gi = r * kWave + l;
            const int row = gi / CPR, cc = gi % CPR;
            voff[r] = row * R + ((cc ^ row_swz<CPR>(row)) << 4);
        }
        // operand reads: lane half `half` of row frow
        uint32_t roff[NV];
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const int cc = KTile<D, KF>::chunk(i, half);
            roff[i] = w * SLOT + frow * R + ((cc ^ row_swz<CPR>(frow)) << 4);
        }
        const uint32_t ring_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((SIA_LDS uint8_t*)ring)) +
                                  w * SLOT;
        // copy the wave's k-th tile (clamped to its last) into slot s
        auto issue = [&](int k, int s) {
            const int t = t0 + min(k, n - 1);
            const int page = max(__builtin_amdgcn_readfirstlane(pages[t >> 1]), 0);
            const int64_t row0 = (int64_t)page * kPage + (t & 1) * 32;
            const uint8_t* base = A.rows + row0 * R;
            const uint32_t dst = ring_lds + s * (NWV * SLOT);
#pragma unroll
            for (int r = 0; r < GM::DMA; r++) dma16_s_nt(base, voff[r], dst + r * 1024);
            if constexpr (KF != kRowBf16) {
                // the 64 scales of the page, 4 bytes per lane (no lane mask, so
                // that the loop body stays one basic block)
                const float* sbase = A.scale + (int64_t)page * kPage;
                dma4_s(sbase, 4 * l, dst + GM::TILE);
            }
        };
        // operand reads of the wave's k-th tile from slot s
        auto fetch = [&](int k, int s, KTile<D, KF>& t) {
            const uint8_t* slot = ring + s * (NWV * SLOT);
#pragma unroll
            for (int i = 0; i < NV; i++) t.v[i] = *reinterpret_cast<const u32x4*>(slot + roff[i]);
            if constexpr (KF != kRowBf16)
                t.sc = *reinterpret_cast<const float*>(slot + w * SLOT + GM::TILE + 4 * (((t0 + k) & 1) * 32 + frow));
            else t.sc = 1.f;
            // (a position on a page whose id is out of range was copied from page 0;
            // it is not visible, and the call reports the bad id in the status word)
            t.ok = (t0 + k) * 32 + frow < my_valid && pages[(t0 + k) >> 1] >= 0;
        };
        // Epilogue of the wave's kk-th tile. kk outside [0, n) is a padding step
        // (the last tile again, or the step before the first): its keys go to the
        // row's spare tail and count nowhere. Without branches, so that the
        // compiler keeps the MFMAs where they are issued instead of sinking them
        // into a store branch next to this epilogue.
        auto finish = [&](int kk, const f32x16 (&acc)[MB], float tsc, bool tok, const IdxQuery<MB, D, KF>& q) {
            const float sc = tile_epilogue<MB, D, KF>(q, acc, tsc);
            const bool valid = kk >= 0 && kk < n;
            if constexpr (SCORES) {
                asm volatile("" ::"v"(sc));
                if (l < 32 && tok && valid) S.scores[rowbase + (t0 + kk) * 32 + frow] = sc;
            } else {
                // lanes 0..31 keep their position's key if it reaches the floor
                // (lanes 32..63 hold the same keys and keep none); a lane that
                // keeps nothing writes to the row's spare tail (no branch in the
                // loop body)
                const uint32_t key = score_key(sc) & (0u - (uint32_t)(tok && valid && l < 32));
                const bool take = key >= floor_key[qi];
                const uint64_t mask = __ballot(take);
                const int64_t at = take ? (int64_t)j * S.ld + rbase + cnt + lanes_below(mask)
                                        : (int64_t)j * S.ld + S.ld - 64 + frow;
                S.cand_key[at] = key;
                S.cand_pos[at] = pos0 + (t0 + kk) * 32 + frow;
                // lanes that keep nothing add 0 to distinct bins (no conflicts)
                atomicAdd(&hist[qi * kCoarseBins + (take ? coarse_bin(key) : (uint32_t)l)], take ? 1u : 0u);
                cnt += __popcll(mask);
            }
        };

        // the first copies go out before the query is read, so that both latencies overlap
#pragma unroll
        for (int u = 0; u < NS - 1; u++) issue(u, u);
        IdxQuery<MB, D, KF> q;
        load_query<MB, D>(A, j, q);
        wait_vmcnt_mem<0>();
        KTile<D, KF> t;
        fetch(0, 0, t);
        f32x16 acc0[MB], acc1[MB];
#pragma unroll
        for (int mb = 0; mb < MB; mb++) acc1[mb] = f32x16{};
        float sc0 = 0.f, sc1 = 0.f;
        bool ok0 = false, ok1 = false;
        // the run is padded to a multiple of the unroll with repeats of its last
        // tile (scored, never stored), so the loop body has no branches
        for (int k0 = 0; k0 < n; k0 += U) {
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int k = k0 + u;
                if (u % 2 == 0) {
                    tile_mfma<MB, D, KF>(q, t, acc0);
                    sc0 = t.sc; ok0 = t.ok;
                } else {
                    tile_mfma<MB, D, KF>(q, t, acc1);
                    sc1 = t.sc; ok1 = t.ok;
                }
                __builtin_amdgcn_sched_barrier(0);   // the MFMAs go out before the epilogue below
                issue(k + NS - 1, (u + NS - 1) % NS);   // refills the slot of tile k - 1
                if (u % 2 == 0) finish(k - 1, acc1, sc1, ok1, q);
                else finish(k - 1, acc0, sc0, ok0, q);
                wait_vmcnt_mem<(NS - 2) * GM::PER_TILE>();   // tile k + 1 has landed
                fetch(min(k + 1, n - 1), (u + 1) % NS, t);
            }
            if constexpr (!SCORES) {
                // the waves take turns raising the floor from the part's histogram
                if ((k0 / U) % WPQ == sub) {
                    int b0, b1;
                    coarse_floor<false>(hist + qi * kCoarseBins, S.topk, b0, b1);
                    if (l == 0) floor_key[qi] = max((uint32_t)b0 << (32 - kCoarseBits), 1u);
                }
            }
        }
        // last step of the padded run: its parity is that of U (even)
        finish(((n + U - 1) / U) * U - 1, acc1, sc1, ok1, q);
        wait_vmcnt_mem<0>();
    }
    if constexpr (!SCORES) {
        if (j < A.num_q && l == 0) S.reg[(int64_t)j * S.n_reg + part * WPQ + sub] = make_int2(rbase, cnt);
        __syncthreads();
        for (int i = 0; i < G; i++) {
            const int jj = g * G + i;
            if (jj >= A.num_q) break;
            uint32_t* dst = S.hist + ((int64_t)jj * S.n_parts + part) * kCoarseBins;
            for (int b = threadIdx.x; b < kCoarseBins; b += kRowsThreads) dst[b] = hist[i * kCoarseBins + b];
        }
    }
}

// ------------------------------------------------------------ score pass, query pairs

// Two queries of one sequence (draft tokens) read the same index-K rows, so a
// workgroup scores a part of both rows and copies every row once for the pair.
// Eight waves form four teams; a team is the two waves of one SIMD (w and w + 4)
// with one ring of LDS slots and one contiguous run of tiles:
//   copier (w < 4):    copies the team's tiles, scores heads 0..31 of both
//                      queries and hands its block sums over through LDS;
//   finisher (w >= 4): scores heads 32..63 of both queries, adds the copier's
//                      block sums (block order kept), applies the token scale,
//                      writes keys and histogram counts.
// Each wave holds one head block of both queries (about 200 registers), so two
// waves share a SIMD and each hides the other's vector work behind its MFMAs.
// One workgroup barrier per tile orders the copies, the hand-over and the reuse
// of ring slots. Within a wave the MFMAs of one query are interleaved with the
// vector epilogue of the other, whose accumulators were issued a group earlier.
constexpr int kPairUnroll = 8;          // loop unroll (ring slots are static per step)
constexpr int kPairPartPages = 512;     // a pair part spans at most 32768 positions

template <int D, int KF>
struct PairGeom {
    static constexpr int R = D * ((KF != kRowBf16) ? 1 : 2);
    static constexpr int CPR = R / 16;
    static constexpr int NTEAM = kPairThreads / kWave / 2;
    static constexpr int TILE = 32 * R;
    static constexpr int DMA = TILE / 1024;
    static constexpr int PER_TILE = DMA + ((KF != kRowBf16) ? 1 : 0);
    static constexpr int SLOT = TILE + ((KF != kRowBf16) ? 256 : 0);
    static constexpr size_t FIXED = kCoarseBins * 4 + kPairPartPages * 4 + 2 * NTEAM * kWave * 4 + 512;
    static constexpr int NS_FIT = (int)((kMaxLds - FIXED) / ((size_t)NTEAM * SLOT));
    static constexpr int NS = NS_FIT >= 8 ? 8 : (NS_FIT >= 4 ? 4 : 2);   // divides the unroll
    static_assert(NS_FIT >= 4, "the pair ring needs four slots per team at least");
};

// Scheduling hint for a step: each of the query's MFMAs followed by up to NVALU
// vector instructions. NVALU spreads the group's vector work over all of its
// MFMAs, so that some of it still follows the last one: the head sums of the
// next group read this group's results, which are ready only a full MFMA after
// its last issue (the wait states otherwise become s_nop stalls).
// (The spreads below were measured per key format: MXFP8 tiles take half the
// MFMAs of fp8 tiles with the query's two terms, for the same vector work.)
template <int NMFMA, int NVALU = 16>
__device__ __forceinline__ void interleave_mfma_valu() {
#pragma unroll
    for (int i = 0; i < NMFMA; i++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, NVALU, 0);   // then up to NVALU VALU (its shadow)
    }
}


template <int D, int KF, bool SCORES>
__global__ __launch_bounds__(kPairThreads) void indexer_pair_kernel(IdxArgs A, RowsArgs S) {
    using GM = PairGeom<D, KF>;
    constexpr int NS = GM::NS, R = GM::R, CPR = GM::CPR, NTEAM = GM::NTEAM, U = kPairUnroll;
    constexpr int SLOT = GM::SLOT, NV = KTile<D, KF>::NV;
    constexpr int NMFMA = mfmas_per_block<D, KF>();   // MFMAs per query, tile and head block
    __shared__ __attribute__((aligned(16))) uint8_t ring[NS * NTEAM * SLOT];
    __shared__ int pages[kPairPartPages];
    // the part's coarse histograms, query 0 in the low and query 1 in the high
    // 16 bits of each counter (a part has at most 32768 positions)
    __shared__ __attribute__((aligned(16))) uint32_t hist[SCORES ? 4 : kCoarseBins];
    __shared__ float xch[2][NTEAM][kWave];   // copier block sums, by step parity
    __shared__ uint32_t floor_key[2];        // per query: keys below it are not kept (>= 1)

    const int g = blockIdx.x / S.n_parts;
    const int part = blockIdx.x % S.n_parts;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int team = w % NTEAM, hb = w / NTEAM;   // hb = 0: copier, 1: finisher
    const int l = lane_id(), half = l >> 5, frow = l & 31;
    const int pos0 = part * S.part;
    const int j0 = 2 * g, j1 = 2 * g + 1;
    const int j1s = j1 < A.num_q ? j1 : j0;   // (an odd last query has no partner: its
                                              // half of the work keeps nothing)

    // both queries must name one sequence; a second query naming another is
    // dropped (status bit)
    int b0 = 0, rl0 = 0, rl1 = 0;
    if (j0 < A.num_q) rl0 = visible_len(A, j0, b0);
    if (j1 < A.num_q) {
        int b1;
        rl1 = visible_len(A, j1, b1);
        if (b1 != b0) {
            if (threadIdx.x == 0) atomicOr(A.status, kBadSeq);
            rl1 = 0;
        }
    }
    if (!SCORES && part == 0 && threadIdx.x == 0) {
        if (j0 < A.num_q) S.row_len[j0] = rl0;
        if (j1 < A.num_q) S.row_len[j1] = rl1;
    }
    b0 = __builtin_amdgcn_readfirstlane(b0);
    rl0 = __builtin_amdgcn_readfirstlane(rl0);
    rl1 = __builtin_amdgcn_readfirstlane(rl1);
    const int valid0 = max(0, min(S.part, rl0 - pos0));
    const int valid1 = max(0, min(S.part, rl1 - pos0));
    const int nvalid = max(valid0, valid1);
    const int npg = (nvalid + kPage - 1) / kPage;
    for (int i = threadIdx.x; i < npg; i += kPairThreads) pages[i] = page_of(A, b0, pos0 / kPage + i);
    if constexpr (!SCORES) {
        for (int i = threadIdx.x; i < kCoarseBins; i += kPairThreads) hist[i] = 0u;
        if (threadIdx.x < 2) floor_key[threadIdx.x] = 1u;
    }
    __syncthreads();

    // the team's run of tiles (an even count, so that a run starts on a page);
    // every wave takes the same number of steps (the longest run, padded to the
    // unroll), so that the barriers match
    const int ntiles = (nvalid + 31) / 32;
    const int tpw = ((ntiles + NTEAM - 1) / NTEAM + 1) & ~1;
    const int t0 = team * tpw;
    const int n = max(0, min(tpw, ntiles - t0));
    const int nloop = (min(tpw, ntiles) + U - 1) / U * U;
    const int rbase = pos0 + t0 * 32;   // first entry of the team's candidate regions
    int cnt0 = 0, cnt1 = 0;             // candidates appended per query (finisher)

    if (nloop > 0) {
        uint32_t voff[GM::DMA];
#pragma unroll
        for (int r = 0; r < GM::DMA; r++) {
            const int gi = r * kWave + l;
            const int row = gi / CPR, cc = gi % CPR;
            voff[r] = row * R + ((cc ^ row_swz<CPR>(row)) << 4);
        }
        uint32_t roff[NV];
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const int cc = KTile<D, KF>::chunk(i, half);
            roff[i] = team * SLOT + frow * R + ((cc ^ row_swz<CPR>(frow)) << 4);
        }
        const uint32_t ring_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((SIA_LDS uint8_t*)ring)) +
                                  team * SLOT;
        // tile of the team's k-th step: clamped into the run (a padding step
        // repeats the last tile; a team without tiles reads the part's last one)
        auto tile_of = [&](int k) { return min(t0 + max(min(k, n - 1), 0), ntiles - 1); };
        auto issue = [&](int k, int s, int pg) {   // copier only; pg: the tile's page id
            const int t = tile_of(k);
            const int page = max(__builtin_amdgcn_readfirstlane(pg), 0);
            const int64_t row0 = (int64_t)page * kPage + (t & 1) * 32;
            const uint8_t* base = A.rows + row0 * R;
            const uint32_t dst = ring_lds + s * (NTEAM * SLOT);
#pragma unroll
            for (int r = 0; r < GM::DMA; r++) dma16_s_nt(base, voff[r], dst + r * 1024);
            if constexpr (KF != kRowBf16) {
                // the 64 scales of the page, 4 bytes per lane (no lane mask)
                const float* sbase = A.scale + (int64_t)page * kPage;
                dma4_s(sbase, 4 * l, dst + GM::TILE);
            }
        };
        auto fetch = [&](int k, int s, KTile<D, KF>& t) {
            const uint8_t* slot = ring + s * (NTEAM * SLOT);
#pragma unroll
            for (int i = 0; i < NV; i++) t.v[i] = *reinterpret_cast<const u32x4*>(slot + roff[i]);
            if constexpr (KF != kRowBf16)
                t.sc = *reinterpret_cast<const float*>(slot + team * SLOT + GM::TILE +
                                                       4 * ((tile_of(k) & 1) * 32 + frow));
            else t.sc = 1.f;
        };
        // finisher: lanes 0..31 hold query 0 of step kq, lanes 32..63 query 1 of
        // step kq - 1 (pg: the page id of this lane's tile). finish_prep (vector
        // work, beside the MFMAs) decides which
        // keys reach their query's floor `fk` and where they go in the query's
        // candidate list of this team; finish_commit (after them) writes only
        // those. Positions on a page whose id is out of range were copied from
        // page 0 and are dropped.
        struct Fin {
            int64_t at;      // candidate slot (scores: score index)
            uint32_t key;
            float sc;
            bool take;
        };
        auto finish_prep = [&](int kq, float v, float tsc, uint32_t fk, int pg) -> Fin {
            Fin f;
            f.sc = KF == kRowFp8 ? v * tsc : v;
            const int kk = half ? kq - 1 : kq;
            const bool in_run = (kk >= 0) & (kk < n);
            const int tpos = (t0 + kk) * 32 + frow;   // position within the part
            const bool tok = in_run & (tpos < (half ? valid1 : valid0)) & (pg >= 0);
            const int64_t row = (int64_t)(half ? j1s : j0) * S.ld;
            if constexpr (SCORES) {
                f.take = tok;
                f.at = row + pos0 + tpos;
                f.key = 0u;
            } else {
                f.key = score_key(f.sc) & (0u - (uint32_t)tok);
                f.take = f.key >= fk;
                const uint64_t mask = __ballot(f.take);
                const uint32_t m0 = (uint32_t)mask, m1 = (uint32_t)(mask >> 32);
                const int rank = (half ? cnt1 : cnt0) + __popc((half ? m1 : m0) & ((1u << frow) - 1u));
                f.at = row + rbase + rank;
                cnt0 += __popc(m0);
                cnt1 += __popc(m1);
            }
            return f;
        };
        auto finish_commit = [&](const Fin& f, int kq) {
            if (f.take) {
                if constexpr (SCORES) {
                    S.scores[f.at] = f.sc;
                } else {
                    const int kk = half ? kq - 1 : kq;
                    S.cand_key[f.at] = f.key;
                    S.cand_pos[f.at] = pos0 + (t0 + kk) * 32 + frow;
                    atomicAdd(&hist[coarse_bin(f.key)], half ? 0x10000u : 1u);
                }
            }
        };

        if (hb == 0) {
#pragma unroll
            for (int u = 0; u < NS - 1; u++) issue(u, u, pages[tile_of(u) >> 1]);
        }
        // copier: page id of the tile that step k copies, read a step ahead
        int pg_next = pages[tile_of(NS - 1) >> 1];
        IdxQuery<1, D, KF> q0, q1;
        load_query<1, D>(A, min(j0, A.num_q - 1), q0, hb);
        load_query<1, D>(A, min(j1, A.num_q - 1), q1, hb);
        wait_vmcnt_mem<0>();
        __syncthreads();   // the first copies have landed
        // tile k is in registers at the top of step k: each step reads the next
        // tile from LDS before its barrier (the tile was published one barrier
        // earlier), so that the read completes behind the barrier and the next
        // step's MFMAs find their operands
        KTile<D, KF> tc;
        fetch(0, 0, tc);
        f32x16 a0[1], a1[1];
        a1[0] = f32x16{};
        float mine_p = 0.f;                 // finisher: own block sums of step k - 1
        float xv = 0.f;                     // finisher: the copier's block sums of step k - 1
        int pgv = 0;                        // finisher: page id of its lanes' tile of step k - 1
        uint32_t fk = SCORES ? 0u : floor_key[half];   // finisher: this lane's query's floor
        float sc_p1 = 0.f, sc_p2 = 0.f;     // token scales of the tiles of steps k - 1, k - 2
        // page id of the tile whose completion finish_prep takes at step j + 1
        auto page_for = [&](int j) { return pages[tile_of(half ? j - 1 : j) >> 1]; };
        // One step of a role: query 0's MFMAs on tile k beside query 1's block
        // sums of tile k - 1 and (finisher) the vector half of completing step
        // k - 1, whose copier block sums were read after the previous barrier;
        // then query 1's MFMAs on tile k beside query 0's block sums of tile k.
        // Then the copier hands its block sums over, reads tile k + 1, refills
        // the slot of tile k - 1 and waits until tile k + 2 has landed; the
        // finisher reads tile k + 1 and writes the kept candidates. After the
        // barrier the finisher reads what the next completion needs.
        auto step = [&](auto fin_tag, int k, int u) {
            constexpr bool FIN = decltype(fin_tag)::value;
            // scheduling fences keep each group of vector work beside the MFMAs
            // it is meant to hide behind (without them the block sums are
            // hoisted to right behind their own MFMAs)
            __builtin_amdgcn_sched_barrier(0);
            tile_mfma<1, D, KF>(q0, tc, a0);
            const float h1 = tile_head_sum<1, D, KF>(q1, a1);
            Fin fin{};
            if constexpr (FIN) fin = finish_prep(k - 1, xv + mine_p, half ? sc_p2 : sc_p1, fk, pgv);
            interleave_mfma_valu<NMFMA, KF == kRowMx ? (FIN ? 36 : 18) : (FIN ? 12 : 6)>();
            __builtin_amdgcn_sched_barrier(0);
            tile_mfma<1, D, KF>(q1, tc, a1);
            const float h0 = tile_head_sum<1, D, KF>(q0, a0);
            interleave_mfma_valu<NMFMA, KF == kRowMx ? 40 : 16>();
            __builtin_amdgcn_sched_barrier(0);
            const float mine = half ? h1 : h0;
            sc_p2 = sc_p1;
            sc_p1 = tc.sc;
            if constexpr (!FIN) {
                xch[k & 1][team][l] = mine;
                const int pg = pg_next;
                pg_next = pages[tile_of(k + NS) >> 1];
                lds_wait_all();                                // the block sums are written
                fetch(k + 1, (u + 1) % NS, tc);
                issue(k + NS - 1, (u + NS - 1) % NS, pg);      // refills the slot of tile k - 1
                if constexpr (!SCORES) {
                    // once per unrolled round, team 0's copier (which waits at
                    // the barrier for its finisher anyway) raises both queries'
                    // floors from the part's histogram (a snapshot taken while
                    // the finishers add to it undercounts, so the floor stays a
                    // lower bound)
                    if (u == U - 1 && team == 0) {
                        int b0, b1;
                        coarse_floor<true>(hist, S.topk, b0, b1);
                        if (l == 0) {
                            floor_key[0] = max((uint32_t)b0 << (32 - kCoarseBits), 1u);
                            floor_key[1] = max((uint32_t)b1 << (32 - kCoarseBits), 1u);
                        }
                        lds_wait_all();                        // the floors are written
                    }
                }
                wait_vmcnt_mem<(NS - 3) * GM::PER_TILE>();    // tile k + 2 has landed

            } else {
                mine_p = mine;
                fetch(k + 1, (u + 1) % NS, tc);
                finish_commit(fin, k - 1);

            }
            barrier_only();
            if constexpr (FIN) {
                xv = xch[k & 1][team][l];
                pgv = page_for(k);
                if constexpr (!SCORES) {
                    if (u == U - 1) fk = floor_key[half];      // the floors move once per round
                }
            }
        };
        // the two roles run separate, branch-free loop bodies with the same
        // barriers
        auto run = [&](auto fin_tag) {
            for (int k0 = 0; k0 < nloop; k0 += U) {
#pragma unroll
                for (int u = 0; u < U; u++) step(fin_tag, k0 + u, u);
            }
        };
        if (hb == 0) run(std::integral_constant<bool, false>{});
        else run(std::integral_constant<bool, true>{});
        // drain: query 1's block sums of the last tile; the finisher completes
        // the last two steps
        {
            const float h1 = tile_head_sum<1, D, KF>(q1, a1);
            if (hb == 0) {
                xch[nloop & 1][team][l] = h1;
            } else {
                finish_commit(finish_prep(nloop - 1, xv + mine_p, half ? sc_p2 : sc_p1, fk, pgv), nloop - 1);
            }
            lds_barrier();
            if (hb == 1)
                finish_commit(finish_prep(nloop, xch[nloop & 1][team][l] + h1, sc_p1, fk, page_for(nloop)), nloop);
        }
        wait_vmcnt_mem<0>();
    }
    if constexpr (!SCORES) {
        if (hb == 1 && l == 0) {
            S.reg[(int64_t)j0 * S.n_reg + part * NTEAM + team] = make_int2(rbase, cnt0);
            if (j1 < A.num_q) S.reg[(int64_t)j1 * S.n_reg + part * NTEAM + team] = make_int2(rbase, cnt1);
        }
        __syncthreads();
        for (int i = 0; i < 2; i++) {
            const int jj = 2 * g + i;
            if (jj >= A.num_q) break;
            uint32_t* dst = S.hist + ((int64_t)jj * S.n_parts + part) * kCoarseBins;
            for (int b = threadIdx.x; b < kCoarseBins; b += kPairThreads)
                dst[b] = i ? hist[b] >> 16 : hist[b] & 0xffffu;
        }
    }
}

// ------------------------------------------------------------ keys from given scores

// Every key of a given score row becomes a candidate: part p of query j is one
// region holding positions p * part .. in order.
__global__ __launch_bounds__(kRowsThreads) void keys_from_scores_kernel(KeysFromScoresArgs K) {
    __shared__ uint32_t hist[kCoarseBins];
    const int j = blockIdx.x / K.n_parts;
    const int part = blockIdx.x % K.n_parts;
    for (int b = threadIdx.x; b < kCoarseBins; b += kRowsThreads) hist[b] = 0u;
    __syncthreads();
    int rl = K.row_len[j];
    if (rl < 0 || rl > K.max_len) {
        if (threadIdx.x == 0) atomicOr(K.status, kRowTooLong);
        rl = max(0, min(rl, K.max_len));
    }
    const int p0 = part * K.part;
    const int p1 = min(p0 + K.part, rl);
    for (int p = p0 + threadIdx.x; p < p1; p += kRowsThreads) {
        const uint32_t key = score_key(K.scores[(int64_t)j * K.ld_in + p]);
        K.cand_key[(int64_t)j * K.ld + p] = key;
        K.cand_pos[(int64_t)j * K.ld + p] = p;
        atomicAdd(&hist[coarse_bin(key)], 1u);
    }
    if (threadIdx.x == 0) K.reg[(int64_t)j * K.n_parts + part] = make_int2(p0, max(0, p1 - p0));
    __syncthreads();
    uint32_t* dst = K.hist + ((int64_t)j * K.n_parts + part) * kCoarseBins;
    for (int b = threadIdx.x; b < kCoarseBins; b += kRowsThreads) dst[b] = hist[b];
}

// ------------------------------------------------------------ selection pass

// Gathers every candidate key >= lo of query j and its position into the LDS
// arrays ckey / cpos, in position order (the regions are taken in order; wave w
// takes a contiguous range of them). Two passes over the candidate keys: count
// per wave, then place at the wave's offset. The caller knows that the count
// fits (at most kSelCap). Returns the count.
__device__ int gather_candidates(const SelectArgs& S, int j, uint32_t lo, uint32_t* ckey, int32_t* cpos,
                                 int* wtot) {
    constexpr int NW = kSelThreads / kWave, STEPS = 4;
    const int w = threadIdx.x / kWave, l = lane_id();
    const int r0 = (int)((int64_t)w * S.n_reg / NW), r1 = (int)((int64_t)(w + 1) * S.n_reg / NW);
    const int2* reg = S.reg + (int64_t)j * S.n_reg;
    const uint32_t* krow = S.cand_key + (int64_t)j * S.ld;
    const int32_t* prow = S.cand_pos + (int64_t)j * S.ld;
    // keys e .. e+3 of chunk s of a region starting at entry `base` with `c` entries
    auto load4 = [&](int base, int c, int i) -> u32x4 {
        u32x4 k4 = {0u, 0u, 0u, 0u};
        if (i < c) k4 = *reinterpret_cast<const u32x4*>(krow + base + i);
#pragma unroll
        for (int e = 0; e < 4; e++)
            if (i + e >= c) k4[e] = 0u;
        return k4;
    };
    int cnt = 0;
    for (int r = r0; r < r1; r++) {
        const int2 rc = reg[r];
        for (int b = 0; b < rc.y; b += STEPS * 256) {
            u32x4 k4[STEPS];
#pragma unroll
            for (int s = 0; s < STEPS; s++) k4[s] = load4(rc.x, rc.y, b + s * 256 + 4 * l);
#pragma unroll
            for (int s = 0; s < STEPS; s++)
#pragma unroll
                for (int e = 0; e < 4; e++) cnt += k4[s][e] >= lo;
        }
    }
    cnt = wave_sum(cnt);
    if (l == 0) wtot[w] = cnt;
    __syncthreads();
    int off = 0, total = 0;
    for (int i = 0; i < NW; i++) {
        const int c = wtot[i];
        off += i < w ? c : 0;
        total += c;
    }
    for (int r = r0; r < r1; r++) {
        const int2 rc = reg[r];
        for (int b = 0; b < rc.y; b += STEPS * 256) {
            u32x4 k4[STEPS];
#pragma unroll
            for (int s = 0; s < STEPS; s++) k4[s] = load4(rc.x, rc.y, b + s * 256 + 4 * l);
#pragma unroll
            for (int s = 0; s < STEPS; s++) {
                const int i = b + s * 256 + 4 * l;
                int c = 0;
#pragma unroll
                for (int e = 0; e < 4; e++) c += k4[s][e] >= lo;
                // (positions of the four entries, read only where one is taken)
                u32x4 p4 = {0u, 0u, 0u, 0u};
                if (c > 0) p4 = *reinterpret_cast<const u32x4*>(prow + rc.x + i);
                const int inc = wave_incl_scan(c);
                int at = off + inc - c;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    if (k4[s][e] >= lo) {
                        if (at < kSelCap) {   // (the caller checked the count; this only guards LDS)
                            ckey[at] = k4[s][e];
                            cpos[at] = (int32_t)p4[e];
                        }
                        at++;
                    }
                }
                off += __shfl(inc, kWave - 1, kWave);
            }
        }
    }
    __syncthreads();
    return total;
}

// One workgroup per query: the coarse histogram (sum of the parts') gives the
// bin of the K-th largest key; every candidate at or above that bin is gathered
// into LDS in position order, the exact threshold is refined there, and the
// ordered compaction emits the Top-K ascending in position. A row whose
// candidates at that bin do not fit in LDS (many equal scores) is first spread
// into a dense key row in global memory (key 0 where there is none) and
// selected there.
__global__ __launch_bounds__(kSelThreads) void topk_rows_kernel(SelectArgs S) {
    __shared__ uint32_t hist[kCoarseBins];
    __shared__ __attribute__((aligned(16))) uint32_t ckey[kSelCap];
    __shared__ __attribute__((aligned(16))) int32_t cpos[kSelCap];
    __shared__ SelScratch sel;
    __shared__ int wtot[kSelThreads / kWave];
    const int j = blockIdx.x;
    const int tid = threadIdx.x;
    const int rl = max(0, min(S.row_len[j], S.max_len));
    int32_t* oi = S.out_idx + (int64_t)j * S.topk;
    float* os = S.out_score ? S.out_score + (int64_t)j * S.topk : nullptr;
    // the row's coarse histogram: the sum of its parts' (both bins of a thread,
    // four parts at a time, so that the loads go out together)
    static_assert(kCoarseBins == 2 * kSelThreads, "two coarse bins per thread");
    {
        const uint32_t* h = S.hist + (int64_t)j * S.n_parts * kCoarseBins + tid;
        uint32_t c0 = 0, c1 = 0;
        int p = 0;
        for (; p + 4 <= S.n_parts; p += 4) {
            uint32_t v[8];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                v[2 * i] = h[(int64_t)(p + i) * kCoarseBins];
                v[2 * i + 1] = h[(int64_t)(p + i) * kCoarseBins + kSelThreads];
            }
#pragma unroll
            for (int i = 0; i < 4; i++) {
                c0 += v[2 * i];
                c1 += v[2 * i + 1];
            }
        }
        for (; p < S.n_parts; p++) {
            c0 += h[(int64_t)p * kCoarseBins];
            c1 += h[(int64_t)p * kCoarseBins + kSelThreads];
        }
        hist[tid] = c0;
        hist[tid + kSelThreads] = c1;
    }
    __syncthreads();
    // (every key in the K-th bin or above was kept by the score pass: its floor
    // never passes the row's K-th bin, so these counts are exact there)
    int above, total;
    const int bin = coarse_select<kSelThreads>(hist, S.topk, &sel, above, total);
    const int m = min(S.topk, total);
    if (m > 0) {
        const bool all = m == total;
        const uint32_t bin_lo = (uint32_t)bin << (32 - kCoarseBits);
        const uint32_t lo = all ? 1u : max(bin_lo, 1u);
        const int ncand = all ? total : above + (int)hist[bin];
        if (ncand <= kSelCap) {
            const int got = gather_candidates(S, j, lo, ckey, cpos, wtot);
            const int nc = min(got, kSelCap);
            for (int i = nc + tid; i < (nc + 7) / 8 * 8; i += kSelThreads) ckey[i] = 0u;
            __syncthreads();
            if (all) {
                ordered_compact<kSelThreads>(ckey, nc, 0u, 0, &sel, EmitFinalBuf{cpos, oi, os, S.topk, {}});
            } else {
                // the remaining 21 bits in two passes of 11 and 10 bits, over
                // the counters of the coarse histogram (free once its bin is
                // known; fewer block-wide rounds than passes of 8 bits)
                uint32_t T = bin_lo, tmask = ~0u << (32 - kCoarseBits);
                int ties = m - above;
#pragma unroll
                for (int pass = 0; pass < 2; pass++) {
                    const int width = pass == 0 ? 11 : 32 - kCoarseBits - 11;
                    const int shift = pass == 0 ? 32 - kCoarseBits - 11 : 0;
                    const uint32_t dmask = (1u << width) - 1u;
                    for (int i = tid; i < kCoarseBins; i += kSelThreads) hist[i] = 0u;
                    __syncthreads();
                    for (int i = tid; i < nc; i += kSelThreads) {
                        const uint32_t k = ckey[i];
                        if ((k & tmask) == T) atomicAdd(&hist[(k >> shift) & dmask], 1u);
                    }
                    __syncthreads();
                    int ab, tot;
                    const int d = coarse_select<kSelThreads>(hist, ties, &sel, ab, tot);
                    T |= (uint32_t)d << shift;
                    tmask |= dmask << shift;
                    ties -= ab;
                }
                ordered_compact<kSelThreads>(ckey, nc, T, ties, &sel, EmitFinalBuf{cpos, oi, os, S.topk, {}});
            }
        } else {
            // dense key row: clear it, spread the candidates at or above lo to
            // their positions (distinct, below rl), then select in global memory
            uint32_t* keys = S.keys + (int64_t)j * S.ld;
            const int n8 = (rl + 7) / 8 * 8;   // (ld >= n8: the row has a spare tail)
            for (int p = tid; p < n8; p += kSelThreads) keys[p] = 0u;
            __threadfence();
            __syncthreads();
            const int2* reg = S.reg + (int64_t)j * S.n_reg;
            const uint32_t* krow = S.cand_key + (int64_t)j * S.ld;
            const int32_t* prow = S.cand_pos + (int64_t)j * S.ld;
            for (int r = 0; r < S.n_reg; r++) {
                const int2 rc = reg[r];
                for (int i = tid; i < rc.y; i += kSelThreads) {
                    const uint32_t k = krow[rc.x + i];
                    const int p = prow[rc.x + i];
                    if (k >= lo && p >= 0 && p < rl) keys[p] = k;
                }
            }
            __threadfence();
            __syncthreads();
            if (all) {
                ordered_compact<kSelThreads>(keys, rl, 0u, 0, &sel, EmitFinal{oi, os, 0, S.topk});
            } else {
                int ties;
                const uint32_t T = radix_refine<kSelThreads>(keys, rl, bin_lo, ~0u << (32 - kCoarseBits),
                                                             m - above, 32 - kCoarseBits, &sel, ties);
                ordered_compact<kSelThreads>(keys, rl, T, ties, &sel, EmitFinal{oi, os, 0, S.topk});
            }
        }
    }
    for (int r = m + tid; r < S.topk; r += kSelThreads) {
        oi[r] = -1;
        if (os) os[r] = -INFINITY;
    }
}

// ------------------------------------------------------------ stream kernel

// A wave's candidate buffer: keys and positions in the workspace (global
// memory, cap entries each plus one spare entry per lane for the branch-free
// append), its selection scratch and the 64 spare counters of the selection's
// branch-free histogram adds in LDS.
struct WaveBuf {
    uint32_t* key;
    int32_t* pos;
    SelScratch* sel;
    uint32_t* spare;
};

// Orders a wave's global stores to its candidate buffer before its later loads
// of the buffer in other lanes (all lanes of a wave run on one CU, whose L1 the
// stores write through), then waits for every vector memory access in flight
// (vmcnt 0; expcnt and lgkmcnt left open) as a compiler-visible wait: the
// compiler's own tracking then knows that nothing of the selection is pending
// where its path joins the scoring loop again, and does not make the loop's
// next MFMA wait for all outstanding memory accesses (the ring copies among
// them) there.
__device__ __forceinline__ void buffer_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Geometry of the K ring the four waves of a stream workgroup share: every
// 32-position tile of index-K is copied once from global memory into LDS and
// read there by all four queries of the workgroup (consecutive positions of one
// sequence walk almost the same causal rows).
template <int D, int KF>
struct StreamGeom {
    static constexpr int R = D * ((KF != kRowBf16) ? 1 : 2);            // bytes per row
    static constexpr int CPR = R / 16;                      // 16-byte chunks per row
    static constexpr int TILE = 32 * R;
    static constexpr int DMA = TILE / 1024;                 // 1 KB copies per tile
    static constexpr int QPT = kStreamThreads / kWave;      // waves (= queries) per workgroup
    static constexpr int CPW = (DMA + QPT - 1) / QPT;       // copies per wave and tile
    static constexpr int PER_TILE = CPW + ((KF != kRowBf16) ? 1 : 0);    // (+ the page's 64 scales)
    static constexpr int SLOT = TILE + ((KF != kRowBf16) ? 256 : 0);
    static constexpr int NS = TILE <= 4096 ? 8 : 4;         // ring slots
    static constexpr int RING = NS * SLOT;
    static_assert(DMA >= 1 && (NS == 4 || NS == 8) && (NS - 1) * PER_TILE < 64 &&
                  (NS - 4) * PER_TILE + 2 * (NS - 2) < 64, "stream ring geometry");
};

__host__ __device__ inline size_t stream_ring_bytes(int dim, bool fp8) {
    const size_t tile = 32 * (size_t)dim * (fp8 ? 1 : 2);
    return (tile <= 4096 ? 8 : 4) * (tile + (fp8 ? 256 : 0));
}

// One workgroup's four queries j (one per wave; rl = its visible length, rl_max
// the longest of the four) walked tile by tile over the shared K ring. Each
// wave keeps the keys that beat its threshold tau in its own LDS candidate
// buffer and re-selects inside it when the buffer fills, then emits its Top-K.
// Called by all four waves (the ring needs one barrier per tile).
template <int MB, int D, int KF>
__device__ void stream_group(const IdxArgs& A, const StreamArgs& S, int j, int rl, int rl_max,
                             const int* pages, WaveBuf B, uint8_t* ring, int* votes) {
    using SG = StreamGeom<D, KF>;
    constexpr int NS = SG::NS, R = SG::R, NV = KTile<D, KF>::NV;
    const int l = lane_id(), half = l >> 5, frow = l & 31;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const bool live = j < A.num_q;
    int cnt = 0;
    uint32_t tau = 0u;
    const int nt = (rl_max + 31) / 32;
    if (nt > 0) {
        IdxQuery<MB, D, KF> q;
        load_query<MB, D>(A, live ? j : A.num_q - 1, q);
        // this wave's copies of a tile: tile bytes [1024 r, 1024 r + 1024) land
        // linearly in the slot; lane l fetches the source chunk that belongs at
        // slot byte 1024 r + 16 l (logical chunk c of a row sits at c ^ row_swz(row))
        uint32_t voff[SG::CPW];
#pragma unroll
        for (int c = 0; c < SG::CPW; c++) {
            const int r = min(w * SG::CPW + c, SG::DMA - 1);
            const int gi = r * 1024 + 16 * l;
            const int row = gi / R, cc = (gi % R) / 16;
            voff[c] = row * R + ((cc ^ row_swz<SG::CPR>(row)) << 4);
        }
        uint32_t roff[NV];
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const int cc = KTile<D, KF>::chunk(i, half);
            roff[i] = frow * R + ((cc ^ row_swz<SG::CPR>(frow)) << 4);
        }
        const uint32_t ring_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((SIA_LDS uint8_t*)ring));
        // page id of tile k's copy (clamped to the last tile, so that every wave
        // issues the same count whatever k is; a clamped copy lands in a free slot)
        auto copy_page = [&](int k) { return pages[min(k, nt - 1) >> 1]; };
        // copies of tile k from physical page pg (its page id, read beforehand)
        auto issue = [&](int k, int pg) {
            const int ti = min(k, nt - 1);
            const int page = max(__builtin_amdgcn_readfirstlane(pg), 0);
            const uint8_t* base = A.rows + ((int64_t)page * kPage + (ti & 1) * 32) * R;
            const uint32_t dst = ring_lds + (k % NS) * SG::SLOT;
#pragma unroll
            for (int c = 0; c < SG::CPW; c++) {
                const int r = min(w * SG::CPW + c, SG::DMA - 1);
                dma16_s(base, voff[c], dst + r * 1024);
            }
            if constexpr (KF != kRowBf16) dma4_s(A.scale + (int64_t)page * kPage, 4 * l, dst + SG::TILE);
        };
        // operands of tile k (k may be past the last tile: then the slot holds a
        // clamped copy and no position is visible). t.ok is the visibility only;
        // the page id `pg` is read without a branch and checked when the tile is
        // scored, so nothing waits for these reads before then. The slot index
        // (k mod NS) is a compile-time constant: the ring sits at LDS address 0,
        // so each read's address is this lane's offset plus an immediate.
        auto fetch = [&](int k, auto slot_c, KTile<D, KF>& t, int& pg) {
            const uint8_t* slot = ring + decltype(slot_c)::value * SG::SLOT;
#pragma unroll
            for (int i = 0; i < NV; i++) t.v[i] = *reinterpret_cast<const u32x4*>(slot + roff[i]);
            if constexpr (KF != kRowBf16) t.sc = *reinterpret_cast<const float*>(slot + SG::TILE + 4 * ((k & 1) * 32 + frow));
            else t.sc = 1.f;
            t.ok = k * 32 + frow < rl;
            pg = pages[min(k, nt - 1) >> 1];
        };
        // appends the key of position ti*32 + l (score sc, lanes 0..31) if it beats
        // tau. Branch-free: a lane that does not take writes to its own spare entry
        // past the buffer (so the MFMAs issued before it stay where they are).
        // Exactly two global stores per step (the ring's copy waits count them).
        auto append = [&](float sc, bool ok, int ti) {
            const int p = ti * 32 + (l & 31);
            const uint32_t k = score_key(sc) & (0u - (uint32_t)(l < 32 && ok));
            const bool take = k > tau;
            const uint64_t mask = __ballot(take);
            const uint32_t at = take ? (uint32_t)cnt + lanes_below(mask) : (uint32_t)(S.cap + l);
            B.key[at] = k;
            B.pos[at] = p;
            cnt += __popcll(mask);
        };
        uint32_t* const spare = B.spare;
        // re-selects inside the buffer (the whole workgroup does so at once, when
        // any of its waves might not take the next two tiles; a wave that holds
        // at most K keys has nothing to drop)
        auto reselect = [&]() {
            if (cnt > S.topk) {
                // keep the Top-K seen so far (or a superset of it); later keys
                // equal to the new threshold lose to the kept ones
                int ties;
                const int n4 = (cnt + 3) & ~3;
                for (int i = cnt + l; i < n4; i += kWave) B.key[i] = 0u;
                buffer_fence();
                // After the first re-selection the buffered keys lie close
                // together, and a superset of the Top-K is usually enough: every
                // key >= L, L found in one histogram pass, with later keys appended
                // only when above L (at least K kept keys >= L precede them). The
                // exact threshold is taken on the first re-selection (keys spread
                // over the whole score range) and when the superset would leave
                // too little room.
                bool done = false;
                uint32_t T = 0u, pm = 0u;
                int above = 0, low = 32;
                if (tau != 0u) {
                    int kept;
                    const uint32_t L = wave_select_floor(B.key, n4, S.topk, B.sel, kept, pm, above, low, spare);
                    if (L != 0u && kept <= S.topk + (S.cap - S.topk) / 2) {
                        ordered_compact<kWave, true>(B.key, n4, L, 0x7fffffff, B.sel, EmitInPlace{B.key, B.pos, {}});
                        cnt = kept;
                        tau = L;
                        done = true;
                    }
                    T = L;
                }
                if (!done) {
                    // exact: the bits under pm are settled (none on the first
                    // re-selection), the rest is refined
                    T = radix_refine<kWave>(B.key, n4, T, pm, S.topk - above, low, B.sel, ties, spare);
                    ordered_compact<kWave, true>(B.key, n4, T, ties, B.sel, EmitInPlace{B.key, B.pos, {}});
                    cnt = S.topk;
                    tau = T;
                }
                buffer_fence();
            }
        };
        constexpr int NMFMA = MB * mfmas_per_block<D, KF>();   // MFMAs per tile
        // Tiles 0 .. NS-1 go out first. Step k: the MFMAs of tile k+1 (its
        // operands read from LDS one step earlier) run interleaved with the
        // epilogue of tile k (ReLU, head weights, head sum, key, append), while the
        // operands of tile k+2 are read. The waves meet every second step: at an
        // even step k, tiles k+2 and k+3 have landed and become visible, and the
        // slots of tiles k and k+1 (read at steps k-2 and k-1) take tiles k+NS and
        // k+NS+1; each copy still goes out two steps before it is read.
#pragma unroll
        for (int k = 0; k < NS; k++) issue(k, copy_page(k));
        int cp_a = copy_page(NS), cp_b = copy_page(NS + 1);   // pages of the next copies
        wait_vmcnt_mem<(NS - 2) * SG::PER_TILE>();   // tiles 0 and 1 have landed
        lds_barrier();
        // tb holds the operands of the next tile to multiply; A0 / A1 alternate as
        // the accumulators of the tile being finished and of the tile being
        // multiplied (two sets, so that the MFMAs never wait for the epilogue)
        KTile<D, KF> tb;
        int pg_b;
        f32x16 A0[MB], A1[MB];
        fetch(0, std::integral_constant<int, 0>{}, tb, pg_b);
        tile_mfma<MB, D, KF>(q, tb, A0);
        float sc_c = tb.sc;
        bool ok_c = tb.ok;
        int pg_c = pg_b;
        fetch(1, std::integral_constant<int, 1>{}, tb, pg_b);
        // step k = k0 + P with k0 a multiple of NS: P (the phase) fixes the ring
        // slots at compile time; the waves meet at even phases
        auto step = [&](int k, f32x16 (&cur)[MB], f32x16 (&nxt)[MB], auto phase) {
            constexpr int P = decltype(phase)::value;
            if constexpr (P % 2 == 0) {
                // At phase 0 each wave votes for a re-selection when its buffer
                // might not take the appends of the next NS steps (at most 32 NS
                // keys); the votes alternate between two sets of flags, so that
                // a set is rewritten only after every wave has read it.
                int* vote = votes + 4 * ((k / NS) & 1);
                if constexpr (P == 0)
                    if (l == 0) vote[w] = cnt > S.cap - 32 * NS;
                // tiles k+2 and k+3 have landed; after the barrier every wave's
                // part of them is visible, and so is every vote. Vector memory
                // accesses complete in issue order, and issued after those
                // copies are the copies of tiles k+4 .. k+NS-1 and, once the loop
                // runs in full, the appends of the last NS-2 steps (two stores
                // each), which may stay in flight; the first steps wait as if
                // no append had been made.
                if (k >= NS - 2) wait_vmcnt_mem<(NS - 4) * SG::PER_TILE + 2 * (NS - 2)>();
                else wait_vmcnt_mem<(NS - 4) * SG::PER_TILE>();
                lds_barrier();
                issue(k + NS, cp_a);
                issue(k + NS + 1, cp_b);
                cp_a = copy_page(k + NS + 2);
                cp_b = copy_page(k + NS + 3);
                if constexpr (P == 0) {
                    const int any = __builtin_amdgcn_readfirstlane(vote[0] | vote[1] | vote[2] | vote[3]);
                    if (any) reselect();
                }
            }
            tile_mfma<MB, D, KF>(q, tb, nxt);   // tile k+1
            const float sc_n = tb.sc;
            const bool ok_n = tb.ok;
            const int pg_n = pg_b;
            fetch(k + 2, std::integral_constant<int, (P + 2) % NS>{}, tb, pg_b);   // (after the MFMAs have read tb)
            const float sc = tile_epilogue<MB, D, KF>(q, cur, sc_c);
            // (vector instructions per MFMA, measured per key format: bf16
            // tiles have twice the MFMAs of fp8 tiles for the same epilogue)
            interleave_mfma_valu<NMFMA, KF == kRowBf16 ? 8 : KF == kRowFp8 ? 12 : 16>();
            append(sc, ok_c && pg_c >= 0, k);
            sc_c = sc_n;
            ok_c = ok_n;
            pg_c = pg_n;
        };
        // the loop unrolled by NS steps (A0 / A1 alternate between even and odd steps)
        for (int k0 = 0; k0 < nt; k0 += NS) {
            auto run = [&](auto phase) {
                constexpr int P = decltype(phase)::value;
                if (k0 + P >= nt) return false;
                if constexpr (P % 2 == 0) step(k0 + P, A0, A1, phase);
                else step(k0 + P, A1, A0, phase);
                return true;
            };
            using std::integral_constant;
            if (!(run(integral_constant<int, 0>{}) && run(integral_constant<int, 1>{}) &&
                  run(integral_constant<int, 2>{}) && run(integral_constant<int, 3>{})))
                break;
            if constexpr (NS == 8) {
                if (!(run(integral_constant<int, 4>{}) && run(integral_constant<int, 5>{}) &&
                      run(integral_constant<int, 6>{}) && run(integral_constant<int, 7>{})))
                    break;
            }
        }
        wait_vmcnt_mem<0>();
    }
    if (live) {
        int32_t* oi = S.out_idx + (int64_t)j * S.topk;
        float* os = S.out_score ? S.out_score + (int64_t)j * S.topk : nullptr;
        const int n4 = (cnt + 3) & ~3;
        for (int i = cnt + l; i < n4; i += kWave) B.key[i] = 0u;
        buffer_fence();
        // (the buffer's first cnt entries are its nonzero keys: only keys above
        // tau >= 0 are appended, and the re-selections keep nonzero keys)
        const int m = select_emit<kWave>(B.key, n4, cnt, S.topk, B.sel, EmitFinalStream{B.pos, oi, os, S.topk, {}}, B.spare);
        for (int r = m + l; r < S.topk; r += kWave) {
            oi[r] = -1;
            if (os) os[r] = -INFINITY;
        }
        wave_sync();
    }
}

// LDS of a stream workgroup: the K ring (at 0), the staged page ids of the
// longest row, then per wave its selection scratch and 64 spare counters.
struct StreamSel {
    SelScratch sel;
    uint32_t spare[kWave];
};
__host__ __device__ inline size_t stream_sel_offset(int max_visible, int dim, bool fp8) {
    const size_t pages_end = stream_ring_bytes(dim, fp8) + (size_t)(max_visible + kPage - 1) / kPage * 4;
    return (pages_end + 15) / 16 * 16;
}
__host__ __device__ inline size_t stream_smem_bytes(int max_visible, int dim, bool fp8) {
    return stream_sel_offset(max_visible, dim, fp8) + 4 * sizeof(StreamSel);
}

// Two workgroups per CU (256 registers per wave): while one selects inside its
// candidate buffers, the other's MFMAs and vector work keep the SIMDs busy.
template <int MB, int D, int KF>
__global__ __launch_bounds__(kStreamThreads, 2) void indexer_stream_kernel(IdxArgs A, StreamArgs S) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ int next_tile;
    __shared__ int tile_seq, tile_rows;
    __shared__ int votes[2][4];   // re-selection votes of the four waves (two alternating sets)
    constexpr int QPT = kStreamThreads / kWave;   // queries per tile, one per wave
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    StreamSel* ss = reinterpret_cast<StreamSel*>(smem + stream_sel_offset(A.max_visible, D, KF != kRowBf16)) + w;
    uint32_t* gb = S.buf + ((int64_t)blockIdx.x * QPT + w) * 2 * (S.cap + kWave);
    WaveBuf B{gb, reinterpret_cast<int32_t*>(gb + S.cap + kWave), &ss->sel, ss->spare};
    int* pages = reinterpret_cast<int*>(smem + stream_ring_bytes(D, KF != kRowBf16));
    uint8_t* ring = smem;
    // optional trace: where (hardware ids of the CU) and when (100 MHz clock)
    // this workgroup ran, and how many query tiles it took
    const uint64_t t_start = S.trace ? __builtin_amdgcn_s_memrealtime() : 0;
    int tiles_run = 0;

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
        const int rows = tile_rows;
        const int npg = (rows + kPage - 1) / kPage;
        for (int i = threadIdx.x; i < npg; i += kStreamThreads) pages[i] = page_of(A, b0, i);
        __syncthreads();
        stream_group<MB, D, KF>(A, S, j, rl, rows, pages, B, ring, &votes[0][0]);
        __syncthreads();
        tiles_run++;
    };
    // Persistent workgroups (their number sized so that all are resident) take
    // work items from a counter: naive = tiles in index order, heavy-first =
    // tiles from the last, zigzag = the pairs (i, T-1-i), heavier tile first.
    const int n_items = S.sched == 2 ? zigzag_workers(S.n_tiles) : S.n_tiles;
    for (;;) {
        if (threadIdx.x == 0) next_tile = (int)atomicAdd(S.counter, 1u);
        __syncthreads();
        const int n = next_tile;
        __syncthreads();
        if (n >= n_items) break;
        const int ta = S.sched == 0 ? n : S.sched == 2 ? zigzag_shard(S.n_tiles, n, 1) : heavy_first_tile(S.n_tiles, n);
        const int tb = S.sched == 2 ? zigzag_shard(S.n_tiles, n, 0) : -1;
#pragma unroll 1
        for (int r = 0; r < 2; r++) {
            const int t = r == 0 ? ta : tb;
            if (t >= 0) run_tile(t);
        }
    }
    if (S.trace && threadIdx.x == 0 && (int)blockIdx.x < S.trace_cap) {
        const uint64_t t_end = __builtin_amdgcn_s_memrealtime();
        // HW_ID (SE, SH, CU, SIMD, wave) and XCC_ID, read whole
        const uint32_t hw = (uint32_t)__builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 4);
        const uint32_t xcc = (uint32_t)__builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 20);
        uint64_t* r = S.trace + (int64_t)blockIdx.x * 4;
        r[0] = ((uint64_t)xcc << 32) | hw;
        r[1] = t_start;
        r[2] = t_end;
        r[3] = (uint64_t)tiles_run;
    }
}

// MXFP8 quantization: four lanes per group of 32 bf16 values (eight each).
// The group's scale is 2^e with e the smallest integer in [-127, 127] such
// that the largest magnitude m satisfies m <= 448 * 2^e: with m = f * 2^E,
// f in [0.5, 1), and 448 = 0.875 * 2^9, that is e = E - 9 when f <= 0.875 and
// E - 8 otherwise. Elements become e4m3 codes of x / 2^e, rounded to nearest
// even by the conversion instruction (never above 448 in magnitude).
__global__ __launch_bounds__(256) void quantize_mxfp8_kernel(const uint16_t* x, int64_t n_groups, uint8_t* codes,
                                                             uint8_t* scales) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t g = t >> 2;
    const int part = (int)(t & 3);
    const bool live = g < n_groups;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (live) v = *reinterpret_cast<const u32x4*>(x + g * 32 + part * 8);
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        f[2 * i] = __uint_as_float(v[i] << 16);
        f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) m = fmaxf(m, fabsf(f[i]));
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    int e = -127;
    if (m > 0.f) {
        int E;
        const float fr = frexpf(m, &E);
        e = min(max(E - 9 + (fr > 0.875f ? 1 : 0), -127), 127);
    }
    const float inv = ldexpf(1.f, -e);
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0] * inv, f[1] * inv, 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2] * inv, f[3] * inv, lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4] * inv, f[5] * inv, 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6] * inv, f[7] * inv, hi, true);
    if (live) {
        *reinterpret_cast<u32x2*>(codes + g * 32 + part * 8) = u32x2{(uint32_t)lo, (uint32_t)hi};
        if (part == 0) scales[g] = (uint8_t)(e + 127);
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

template <int MB, int D, int KF, int G, bool SC>
static hipError_t rows_launch(const IdxArgs& a, const RowsArgs& r, hipStream_t st) {
    const int groups = (a.num_q + G - 1) / G;
    hipLaunchKernelGGL((indexer_rows_kernel<MB, D, KF, G, SC>), dim3(groups * r.n_parts), dim3(kRowsThreads), 0,
                       st, a, r);
    return hipGetLastError();
}

template <int D, int KF, bool SC>
static hipError_t pair_launch(const IdxArgs& a, const RowsArgs& r, hipStream_t st) {
    const int pairs = (a.num_q + 1) / 2;
    hipLaunchKernelGGL((indexer_pair_kernel<D, KF, SC>), dim3(pairs * r.n_parts), dim3(kPairThreads), 0, st, a,
                       r);
    return hipGetLastError();
}

template <int MB, int D, int KF>
static hipError_t rows_launch3(const IdxArgs& a, const RowsArgs& r, int g, bool sc, hipStream_t st) {
    if (g == 2) return sc ? pair_launch<D, KF, true>(a, r, st) : pair_launch<D, KF, false>(a, r, st);
    return sc ? rows_launch<MB, D, KF, 1, true>(a, r, st) : rows_launch<MB, D, KF, 1, false>(a, r, st);
}

hipError_t launch_indexer_rows(const IdxArgs& a, const RowsArgs& r, int mb, int dim, int kf, int group,
                               bool scores_mode, hipStream_t st) {
#define SIA_ROWS(MBv, Dv, KFv)                                                 \
    if (mb == MBv && dim == Dv && kf == KFv)                                  \
        return rows_launch3<MBv, Dv, KFv>(a, r, group, scores_mode, st);
#define SIA_ROWS_KF(MBv, Dv) SIA_ROWS(MBv, Dv, kRowBf16) SIA_ROWS(MBv, Dv, kRowFp8)
    SIA_ROWS_KF(1, 64) SIA_ROWS_KF(1, 128) SIA_ROWS_KF(2, 64) SIA_ROWS_KF(2, 128)
    SIA_ROWS(1, 128, kRowMx) SIA_ROWS(2, 128, kRowMx)   // (MXFP8 rows are 128 wide)
#undef SIA_ROWS_KF
#undef SIA_ROWS
    return hipErrorInvalidValue;
}

hipError_t launch_keys_from_scores(const KeysFromScoresArgs& k, hipStream_t st) {
    hipLaunchKernelGGL(keys_from_scores_kernel, dim3(k.num_q * k.n_parts), dim3(kRowsThreads), 0, st, k);
    return hipGetLastError();
}

hipError_t launch_topk_rows(const SelectArgs& s, hipStream_t st) {
    hipLaunchKernelGGL(topk_rows_kernel, dim3(s.num_q), dim3(kSelThreads), 0, st, s);
    return hipGetLastError();
}

template <int MB, int D, int KF>
static hipError_t stream_launch(const IdxArgs& a, const StreamArgs& s, int grid, hipStream_t st) {
    auto k = indexer_stream_kernel<MB, D, KF>;
    const size_t smem = stream_smem_bytes(a.max_visible, D, KF != kRowBf16);
    hipError_t e = set_smem(k, smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(grid), dim3(kStreamThreads), smem, st, a, s);
    return hipGetLastError();
}

template <int MB, int D, int KF>
static int stream_occupancy(int max_visible) {
    auto k = indexer_stream_kernel<MB, D, KF>;
    const size_t smem = stream_smem_bytes(max_visible, D, KF != kRowBf16);
    if (set_smem(k, smem) != hipSuccess) return 1;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(k),
                                                     kStreamThreads, smem) != hipSuccess || n < 1)
        return 1;
    return n;
}

hipError_t launch_indexer_stream(const IdxArgs& a, const StreamArgs& s, int mb, int dim, int kf,
                                 int grid, hipStream_t st) {
#define SIA_STREAM(MBv, Dv, KFv) \
    if (mb == MBv && dim == Dv && kf == KFv) return stream_launch<MBv, Dv, KFv>(a, s, grid, st);
#define SIA_STREAM_KF(MBv, Dv) SIA_STREAM(MBv, Dv, kRowBf16) SIA_STREAM(MBv, Dv, kRowFp8)
    SIA_STREAM_KF(1, 64) SIA_STREAM_KF(1, 128) SIA_STREAM_KF(2, 64) SIA_STREAM_KF(2, 128)
    SIA_STREAM(1, 128, kRowMx) SIA_STREAM(2, 128, kRowMx)
#undef SIA_STREAM_KF
#undef SIA_STREAM
    return hipErrorInvalidValue;
}

size_t indexer_stream_smem(int max_visible, int dim, bool fp8) {
    return stream_smem_bytes(max_visible, dim, fp8);
}

int indexer_stream_blocks_per_cu(int mb, int dim, int kf, int max_visible) {
#define SIA_OCC(MBv, Dv, KFv) \
    if (mb == MBv && dim == Dv && kf == KFv) return stream_occupancy<MBv, Dv, KFv>(max_visible);
#define SIA_OCC_KF(MBv, Dv) SIA_OCC(MBv, Dv, kRowBf16) SIA_OCC(MBv, Dv, kRowFp8)
    SIA_OCC_KF(1, 64) SIA_OCC_KF(1, 128) SIA_OCC_KF(2, 64) SIA_OCC_KF(2, 128)
    SIA_OCC(1, 128, kRowMx) SIA_OCC(2, 128, kRowMx)
#undef SIA_OCC_KF
#undef SIA_OCC
    return 1;
}

hipError_t launch_quantize_mxfp8(const uint16_t* x, int64_t n_groups, uint8_t* codes, uint8_t* scales,
                                 hipStream_t st) {
    if (n_groups <= 0) return hipSuccess;
    const int64_t blocks = (n_groups * 4 + 255) / 256;
    hipLaunchKernelGGL(quantize_mxfp8_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, n_groups, codes, scales);
    return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, v, n);
    return hipGetLastError();
}

}  // namespace sia
