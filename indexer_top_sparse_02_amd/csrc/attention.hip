// Sparse MLA attention for gfx950: softmax attention of each query over only
// its Top-K rows of the paged latent KV cache ("Rapid Adaptation and Inference
// Optimization", section 4.2 "Sparse Attention Computation": read the selected
// positions straight from the paged main cache, no contiguous copy).
//
// A row c_s is 576 bf16 wide: keys use all 576 columns, values the first 512
// (the latent part shared by K and V in MLA).
//
// Workgroup = (query, block of HB heads, slice of the selected rows), with
// 2*HB/16 waves. At the start the slice's indices are validated, mapped through
// the page table and compacted (skipped entries removed, order kept) into a
// list of physical row ids in LDS. Tiles of 32 rows go from HBM straight into a
// four-slot LDS ring (direct global -> LDS copies), row-major, with the 16-byte
// chunks of a row XOR-swizzled by the row index so that the operand reads below
// are free of bank conflicts. Wave (hb, rb) owns 16 heads and the 16-row half rb
// of every tile:
//   Q K^T    16x16x32 MFMAs over all 576 columns; its Q slice stays in registers
//   softmax  online, per head, against a reference maximum that moves only when
//            a logit exceeds it by more than 2^8; only in such a tile do the two
//            row halves of a head block compute and exchange per-head tile
//            maxima through LDS; P goes to LDS as bf16
//   P V      wave w owns output columns [w*512/NW, (w+1)*512/NW) of all heads;
//            the value operand is read from the same row-major tile with
//            transposing LDS reads (ds_read_b64_tr_b16), so no transposed copy
//            of the values is ever made; the first reads go out before the
//            barrier that publishes P
// The loop is software-pipelined: between two barriers, iteration t runs the
// Q K^T of tile t+1 next to the softmax of tile t, then P V of tile t. The copy of
// tile t+3 goes out as soon as the slot of tile t-1 is free, so two tiles (72 KB)
// are in flight while one is consumed: a gathered row takes microseconds to
// arrive, longer than the arithmetic on one tile.
// Slices of one query are merged afterwards by log-sum-exp.
#include "sia_device.h"
#include "sia_kernels.h"

namespace sia {

constexpr int kDK = 576, kDV = 512;
constexpr int kTR = 32;                     // rows per tile

// Row formats of the latent cache. bf16: 576 values (1152 bytes = 72 chunks
// of 16). FP8: 512 e4m3 latent codes, four fp32 scales (one per 128 latent
// values), 64 bf16 rope values (656 bytes = 41 chunks). Tiles of 32 rows are
// copied 1 KB (64 lanes x 16 bytes) at a time; the fp8 tile's last copy is
// half full (its spare lanes repeat the tile's last chunk).
template <bool KV8>
struct RowFmt {
    static constexpr int RB = KV8 ? 656 : kDK * 2;        // bytes per row
    static constexpr int CH = RB / 16;                    // 16-byte chunks per row
    static constexpr int TB = kTR * RB;                   // bytes per tile
    static constexpr int CHUNKS = kTR * CH;               // chunks per tile
    static constexpr int COPIES = (CHUNKS + 63) / 64;     // 1 KB copies per tile
    static constexpr int SCALES = 512, ROPE = 528;        // (fp8) byte offsets in a row
};
constexpr int kRowB = RowFmt<false>::RB;
constexpr int kPStride = kTR * 2 + 16;      // bytes per head of P (padded: no bank conflicts)
constexpr int kMaxSliceRows = kAttnMaxSliceRows;

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Four bf16 of one column and four consecutive rows of a row-major tile: with
// the 16 lanes of a group addressing rows k0 + j/4 and columns n0 + 4*(j%4)
// (j = lane within the group), lane j receives rows k0..k0+3 of column n0 + j.
// Issued as inline assembly: the result is only valid after lds_wait(). The compiler's own form of this read
// carries no address information, which makes it wait for every global -> LDS
// copy in flight, including those of later tiles.
__device__ __forceinline__ u32x2 ds_read_tr16(const uint8_t* p) {
    const uint32_t a = (uint32_t)(uintptr_t)(const SIA_LDS uint8_t*)p;
    u32x2 v;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(a));
    return v;
}
// Waits for the LDS reads in flight and ties the four pairs of results to the
// wait, so that no copy or use of them is scheduled before it.
__device__ __forceinline__ void lds_wait(u32x2 (&a)[4], u32x2 (&b)[4]) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3])
                 :
                 : "memory");
}

// Eight transposing reads (as ds_read_tr16), then this wave's LDS operations
// complete and the workgroup meets at a barrier, in one asm block: the results
// are defined only when the block ends, after the wait, so no copy of a value
// still in flight can be made. Used to start the value reads of P V before the
// barrier that publishes P.
__device__ __forceinline__ void ds_read_tr16x8_barrier(u32x2 (&a)[4], u32x2 (&b)[4], const uint32_t (&pa)[4],
                                                       const uint32_t (&pb)[4]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %10\n\t"
        "ds_read_b64_tr_b16 %3, %11\n\t"
        "ds_read_b64_tr_b16 %4, %12\n\t"
        "ds_read_b64_tr_b16 %5, %13\n\t"
        "ds_read_b64_tr_b16 %6, %14\n\t"
        "ds_read_b64_tr_b16 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        "s_barrier"
        : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]), "=&v"(b[3])
        : "v"(pa[0]), "v"(pa[1]), "v"(pa[2]), "v"(pa[3]), "v"(pb[0]), "v"(pb[1]), "v"(pb[2]), "v"(pb[3])
        : "memory");
}

// Four 8-bit transposing reads (16 lanes of a group address rows r0 + j/2 and
// columns c0 + 8 (j % 2): lane j receives column c0 + j of rows r0 .. r0 + 7),
// then the wait, in one asm block, so that the results are defined when it ends.
__device__ __forceinline__ void ds_read_tr8x4(const uint8_t* base, const int (&off)[4], u32x2 (&v)[4]) {
    const uint32_t a = (uint32_t)(uintptr_t)(const SIA_LDS uint8_t*)base;
    asm volatile(
        "ds_read_b64_tr_b8 %0, %4\n\t"
        "ds_read_b64_tr_b8 %1, %5\n\t"
        "ds_read_b64_tr_b8 %2, %6\n\t"
        "ds_read_b64_tr_b8 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
        : "v"(a + off[0]), "v"(a + off[1]), "v"(a + off[2]), "v"(a + off[3])
        : "memory");
}

// Eight e4m3 values (bytes in order) as eight bf16 values (exact: e4m3 values
// are bf16 values).
__device__ __forceinline__ bf16x8 e4m3x8_bf16x8(u32x2 v) {
    const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.f, false);
    const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.f, true);
    const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.f, false);
    const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.f, true);
    return as_bf16x8(u32x4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                           __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)});
}

// Eight bf16 values times eight fp32 factors, rounded to nearest even bf16.
__device__ __forceinline__ bf16x8 scale_bf16x8(bf16x8 p, const float (&sc)[8]) {
    const u32x4 u = __builtin_bit_cast(u32x4, p);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const float lo = __uint_as_float(u[i] << 16) * sc[2 * i];
        const float hi = __uint_as_float(u[i] & 0xffff0000u) * sc[2 * i + 1];
        o[i] = f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
    }
    return as_bf16x8(o);
}

// Byte offset of logical 16-byte chunk c of tile row r. bf16 rows: chunks are
// XOR-swizzled by r within aligned groups of eight. fp8 rows are stored as
// they are.
template <bool KV8 = false>
__device__ __forceinline__ int tile_off(int r, int c) {
    if constexpr (KV8) return r * RowFmt<true>::RB + (c << 4);
    else return r * kRowB + ((c ^ (r & 7)) << 4);
}

// Max / sum over the 16 lanes of a DPP row (lanes 16g .. 16g+15), by rotations
// of the row by 8, 4, 2 and 1 lanes.
template <int N>
__device__ __forceinline__ float dpp_ror(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x120 + N, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_max(float v) {
    v = __builtin_fmaxf(v, dpp_ror<8>(v));
    v = __builtin_fmaxf(v, dpp_ror<4>(v));
    v = __builtin_fmaxf(v, dpp_ror<2>(v));
    v = __builtin_fmaxf(v, dpp_ror<1>(v));
    return v;
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_ror<8>(v);
    v += dpp_ror<4>(v);
    v += dpp_ror<2>(v);
    v += dpp_ror<1>(v);
    return v;
}

template <int HB, bool KV8>
struct MlaGeom {
    static constexpr int NHB = HB / 16;          // 16-head blocks
    static constexpr int NW = 2 * NHB;           // waves: (head block, row block)
    static constexpr int NT = NW * kWave;
    static constexpr int CPW = kDV / NW;         // output columns per wave
    static constexpr int NCB = CPW / 16;         // 16-column blocks per wave
    // tile copies per wave: waves below SPLIT issue one more than the rest
    static constexpr int CP_LO = RowFmt<KV8>::COPIES / NW;
    static constexpr int SPLIT = RowFmt<KV8>::COPIES % NW;
};

// The query of one wave's 16 heads in MFMA operand layout. bf16 rows: all 576
// columns as bf16 (32-wide steps of the 16x16x32 bf16 MFMA). fp8 rows: the
// 512 latent columns enter 16x16x128 fp8 MFMAs against the raw e4m3 codes, the
// bf16 query split per head into e4m3 hi = e4m3(X) and lo = e4m3(16 (X - hi))
// with X = q 2^s (one exponent per head, max|q| 2^s in [128, 256)), the two
// products summed with MFMA scales 2^-s and 2^-(s+4); the 64 rope columns stay
// bf16.
template <bool KV8>
struct MlaQuery;
template <>
struct MlaQuery<false> {
    bf16x8 qa[kDK / 32];
};
template <>
struct MlaQuery<true> {
    i32x8 hi[4], lo[4];   // latent blocks of 128: this lane's 32 codes of each
    bf16x8 rope[2];
    int sh, sl;
};

// Wave (hb, rb) owns 16 heads
// and the 16-row half rb of every tile: it computes that block's logits over all
// 576 columns (its Q slice, 72 registers, stays in registers), so the two halves
// of a tile only exchange per-head tile maxima. Iteration t runs, between two
// barriers, the Q K^T MFMAs of tile t+1 next to the softmax of tile t (vector
// work), then P V of tile t. The copy of tile t+3 is issued as soon as tile t-1's
// slot is free (right after the first barrier). The copies are inline assembly
// (dma16): the compiler neither sees nor waits for them, and each wave waits for
// its own copies of a tile with a counted vmcnt wait before the barrier that
// publishes the tile to the other waves.
template <int HB, bool KV8>
__global__ __attribute__((amdgpu_flat_work_group_size(1, 512))) void sparse_mla_kernel(AttnArgs A) {
    using GM = MlaGeom<HB, KV8>;
    using RF = RowFmt<KV8>;
    constexpr int NHB = GM::NHB, NW = GM::NW, NT = GM::NT, CPW = GM::CPW, NCB = GM::NCB;
    constexpr int KS = kDK / 32;   // 18 MFMA steps over a full bf16 row
    // (a slot holds whole 1 KB copies: the fp8 tile's half-full last copy lands
    // in the slot's spare tail)
    constexpr int SLOT = RF::COPIES * 1024;
    __shared__ __attribute__((aligned(16))) uint8_t ring0[SLOT];
    __shared__ __attribute__((aligned(16))) uint8_t ring1[SLOT];
    __shared__ __attribute__((aligned(16))) uint8_t ring2[SLOT];
    __shared__ __attribute__((aligned(16))) uint8_t ring3[SLOT];
    __shared__ __attribute__((aligned(16))) uint32_t rows[kMaxSliceRows];
    // P, alpha and the moved flags of tile t are written after the first barrier
    // of iteration t and read after its second; the next writes come after the
    // first barrier of iteration t+1, which every wave passes only once its reads
    // of tile t are done: one buffer each suffices. The "reference moves" flags
    // of tile t+1 are written in iteration t while those of tile t may still be
    // read, so they alternate by tile parity; the tile maxima, exchanged only in
    // an iteration that moves a reference (with a barrier of its own), need one.
    __shared__ __attribute__((aligned(16))) uint8_t pbuf[HB * kPStride];
    __shared__ __attribute__((aligned(16))) float mx[2][HB];                   // [row half][head]
    __shared__ __attribute__((aligned(16))) int flg[2][NW < 4 ? 4 : NW];        // [parity][wave]
    __shared__ __attribute__((aligned(16))) float alpha_s[HB];
    __shared__ __attribute__((aligned(16))) float lsum[2][HB];
    __shared__ __attribute__((aligned(16))) float mfin[HB];
    __shared__ int scan_s[16];
    __shared__ __attribute__((aligned(16))) int moved_w[NW];   // [wave]: a reference max moved

    const int tid = threadIdx.x, l = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int g = l >> 4, jl = l & 15;
    const int n_hb = A.heads / HB;

    const int bid = blockIdx.x;
    const int xcd = bid & 7, slot = bid >> 3;
    const int num_pairs = A.num_q * A.n_split;
    const int P = (slot / n_hb) * 8 + xcd;
    const int hbk = slot % n_hb;
    if (P >= num_pairs) return;
    const int pair = num_pairs - 1 - P;
    const int j = pair / A.n_split, sp = pair % A.n_split;
    const int head0 = hbk * HB;

    int b = A.q_seq[j];
    const bool seq_ok = b >= 0 && b < A.batch;
    if (!seq_ok) {
        if (tid == 0) atomicOr(A.status, kBadSeq);
        b = 0;
    }
    const int n_b = seq_ok ? A.seq_lens[b] : 0;
    const int r0 = sp * A.rows_per_split;
    const int r1 = seq_ok ? min(A.topk, r0 + A.rows_per_split) : r0;

    // ---- Q of this wave's 16 heads, all 576 columns
    const int hb = w % NHB, rb = w / NHB;
    MlaQuery<KV8> Q;
    if constexpr (!KV8) {
        const uint16_t* qrow = A.q + ((int64_t)j * A.heads + head0 + hb * 16 + jl) * kDK + g * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ks++) Q.qa[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + ks * 32));
    } else {
        // lane (jl, g): head hb*16 + jl; latent block b: elements 128 b + 32 g ..
        // + 31 (the same positions as its key bytes, so the MFMA pairs them
        // whatever k it assigns); rope steps: elements 512 + 32 ks + 8 g .. + 7
        const uint16_t* qrow = A.q + ((int64_t)j * A.heads + head0 + hb * 16 + jl) * kDK;
        u32x4 v[4][4];
        float amax = 0.f;
#pragma unroll
        for (int b = 0; b < 4; b++)
#pragma unroll
            for (int c = 0; c < 4; c++) {
                v[b][c] = *reinterpret_cast<const u32x4*>(qrow + 128 * b + 32 * g + 8 * c);
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    amax = fmaxf(amax, fabsf(__uint_as_float(v[b][c][e] << 16)));
                    amax = fmaxf(amax, fabsf(__uint_as_float(v[b][c][e] & 0xffff0000u)));
                }
            }
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        int sx = 0;
        if (amax > 0.f) {
            int e;
            frexpf(amax, &e);
            sx = min(max(8 - e, -120), 120);
        }
        const float f = ldexpf(1.f, sx);
        Q.sh = 127 - sx;
        Q.sl = 127 - sx - 4;
#pragma unroll
        for (int b = 0; b < 4; b++)
#pragma unroll
            for (int c = 0; c < 4; c++)
#pragma unroll
                for (int e = 0; e < 4; e += 2) {
                    float x[4];
                    x[0] = __uint_as_float(v[b][c][e] << 16) * f;
                    x[1] = __uint_as_float(v[b][c][e] & 0xffff0000u) * f;
                    x[2] = __uint_as_float(v[b][c][e + 1] << 16) * f;
                    x[3] = __uint_as_float(v[b][c][e + 1] & 0xffff0000u) * f;
                    int h = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
                    h = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], h, true);
                    float r[4];
                    r[0] = (x[0] - __builtin_amdgcn_cvt_f32_fp8(h, 0)) * 16.f;
                    r[1] = (x[1] - __builtin_amdgcn_cvt_f32_fp8(h, 1)) * 16.f;
                    r[2] = (x[2] - __builtin_amdgcn_cvt_f32_fp8(h, 2)) * 16.f;
                    r[3] = (x[3] - __builtin_amdgcn_cvt_f32_fp8(h, 3)) * 16.f;
                    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
                    lo = __builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], lo, true);
                    Q.hi[b][c * 2 + e / 2] = h;
                    Q.lo[b][c * 2 + e / 2] = lo;
                }
#pragma unroll
        for (int ks = 0; ks < 2; ks++)
            Q.rope[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 512 + 32 * ks + 8 * g));
    }

    // ---- validated, compacted physical row ids of the slice. Thread t owns the
    // RPT consecutive entries r0 + RPT t ..: all index loads go out together,
    // then all page-table loads, then one prefix sum places the kept rows in
    // order (one round trip of each kind instead of one per NT entries).
    constexpr int RPT = kMaxSliceRows / NT;
    int nr = 0;
    {
        int sidx[RPT];
#pragma unroll
        for (int i = 0; i < RPT; i++) {
            const int r = r0 + tid * RPT + i;
            sidx[i] = r < r1 ? A.idx[(int64_t)j * A.topk + r] : -1;
        }
        int pg[RPT];
#pragma unroll
        for (int i = 0; i < RPT; i++) {
            const int s = sidx[i];
            const bool in = s >= 0 && s < n_b && s < A.max_pages * kPage;
            pg[i] = in ? A.page_table[(int64_t)b * A.max_pages + (s >> 6)] : -1;
            if (s >= 0 && !in) atomicOr(A.status, kBadIndex);
        }
        uint32_t row[RPT];
        int keep = 0;
#pragma unroll
        for (int i = 0; i < RPT; i++) {
            const int s = sidx[i];
            const bool in = s >= 0 && s < n_b && s < A.max_pages * kPage;
            const bool ok = in && pg[i] >= 0 && pg[i] < A.num_pages;
            if (in && !ok) atomicOr(A.status, kBadPage);
            row[i] = ok ? (uint32_t)pg[i] * kPage + (uint32_t)(s & 63) : 0xffffffffu;
            keep += ok;
        }
        int pre, tot;
        scan1<NT>(keep, pre, tot, scan_s);
#pragma unroll
        for (int i = 0; i < RPT; i++) {
            if (row[i] != 0xffffffffu) rows[pre++] = row[i];
        }
        nr = tot;
    }
    __syncthreads();
    const int ntiles = (nr + kTR - 1) / kTR;
    wait_vmcnt<0>();

    auto slot_of = [&](int t) -> uint8_t* {
        const int u = t & 3;
        return u == 0 ? ring0 : u == 1 ? ring1 : u == 2 ? ring2 : ring3;
    };
    // copies of tile t: copy i (= w + NW k) covers tile bytes [1024 i, 1024 i + 1024);
    // all row ids are read from LDS before the first copy is issued
    constexpr int CPMAX = GM::CP_LO + (GM::SPLIT ? 1 : 0);
    const int ncp = GM::CP_LO + (w < GM::SPLIT ? 1 : 0);
    auto issue = [&](int t) {
        uint8_t* dst = slot_of(t);
        // copy k of this wave is tile copy w + NW k; a wave with one copy fewer
        // repeats its last one (same bytes to the same place), so that every wave
        // runs the same branch-free sequence. Row ids are read in groups of up to
        // six before the group's copies go out.
        constexpr int GRP = CPMAX < 6 ? CPMAX : 6;
#pragma unroll
        for (int k0 = 0; k0 < CPMAX; k0 += GRP) {
            uint32_t row[GRP];
#pragma unroll
            for (int k = k0; k < k0 + GRP && k < CPMAX; k++) {
                const int i = w + NW * (k < ncp ? k : ncp - 1);
                const int q = min(i * 64 + l, RF::CHUNKS - 1);
                row[k - k0] = rows[min(t * kTR + q / RF::CH, nr - 1)];
            }
#pragma unroll
            for (int k = k0; k < k0 + GRP && k < CPMAX; k++) {
                const int i = w + NW * (k < ncp ? k : ncp - 1);
                // (lanes past the tile's last chunk copy that chunk again into
                // the slot's spare tail)
                const int q = min(i * 64 + l, RF::CHUNKS - 1);
                const int rr = q / RF::CH, c = q % RF::CH;
                const int cs = KV8 ? c : (c ^ (rr & 7));
                const uint8_t* src = reinterpret_cast<const uint8_t*>(A.kv) + (int64_t)row[k - k0] * RF::RB +
                                     (cs << 4);
                dma16(src, (SIA_LDS void*)(dst + i * 1024));
            }
        }
    };

    // key rows rb*16 + jl, chunks 4 ks + g = 8 (ks / 2) + (4 (ks % 2) + g)
    const int kn = rb * 16 + jl;
    int koffL[2];
#pragma unroll
    for (int e = 0; e < 2; e++) koffL[e] = kn * kRowB + ((((e << 2) | g) ^ (kn & 7)) << 4);
    int voffL[2][4];
    {
        const int h = (jl >> 1) & 1, half8 = (jl & 1) << 3;
        const int base = (w * CPW / 8) << 4;
#pragma unroll
        for (int e = 0; e < 2; e++) {
            const int rr = 8 * g + (jl >> 2) + 4 * e;
#pragma unroll
            for (int v = 0; v < 4; v++) voffL[e][v] = rr * kRowB + base + (((2 * v + h) ^ (rr & 7)) << 4) + half8;
        }
    }

    // fp8 rows: the logits of this wave's 16 heads x 16 rows as the latent
    // blocks' fp8 products times the row's block scales (a0) plus the bf16 rope
    // products (a1)
    auto qk8 = [&](const uint8_t* buf, f32x4& a0, f32x4& a1) {
        if constexpr (KV8) {
        const uint8_t* row = buf + kn * RF::RB;
        f32x4 acc[4];
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const u32x4 k0 = *reinterpret_cast<const u32x4*>(row + 128 * b + 32 * g);
            const u32x4 k1 = *reinterpret_cast<const u32x4*>(row + 128 * b + 32 * g + 16);
            const i32x8 kb = {(int)k0[0], (int)k0[1], (int)k0[2], (int)k0[3],
                              (int)k1[0], (int)k1[1], (int)k1[2], (int)k1[3]};
            acc[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Q.hi[b], kb, f32x4{0.f, 0.f, 0.f, 0.f},
                                                                      0, 0, 0, Q.sh, 0, 127);
            acc[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Q.lo[b], kb, acc[b], 0, 0, 0, Q.sl, 0, 127);
        }
        a1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {
            const u32x4 kr = *reinterpret_cast<const u32x4*>(row + RF::ROPE + 2 * (32 * ks + 8 * g));
            a1 = mfma16(Q.rope[ks], as_bf16x8(kr), a1);
        }
        const f32x4 sc = *reinterpret_cast<const f32x4*>(row + RF::SCALES);
#pragma unroll
        for (int r = 0; r < 4; r++)
            a0[r] = sc[0] * acc[0][r] + sc[1] * acc[1][r] + sc[2] * acc[2][r] + sc[3] * acc[3][r];
        }
    };
    // logits of this wave's 16 heads x 16 rows of the tile in `buf`, as two
    // partial sums (even and odd steps) that the caller adds only where it needs
    // them, so that the vector work in between runs while the MFMAs finish
    auto qk = [&](const uint8_t* buf, f32x4& a0, f32x4& a1) {
        if constexpr (KV8) {
            qk8(buf, a0, a1);
            return;
        } else {
        const bf16x8 (&qa)[KS] = Q.qa;
        const int koff[2] = {koffL[0], koffL[1]};
        // the key operands of the next DEPTH steps are in flight during each MFMA
        constexpr int DEPTH = 6;
        auto kread = [&](int ks) -> u32x4 {
            return *reinterpret_cast<const u32x4*>(buf + koff[ks & 1] + (ks >> 1) * 128);
        };
        u32x4 kb[DEPTH];
#pragma unroll
        for (int i = 0; i < DEPTH; i++) kb[i] = kread(i);
        a0 = f32x4{0.f, 0.f, 0.f, 0.f};
        a1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            const u32x4 kv = kb[ks % DEPTH];
            if (ks + DEPTH < KS) kb[ks % DEPTH] = kread(ks + DEPTH);
            if (ks & 1) a1 = mfma16(qa[ks], as_bf16x8(kv), a1);
            else a0 = mfma16(qa[ks], as_bf16x8(kv), a0);
        }
        // schedule: DEPTH reads, then (MFMA, read) pairs, then the last MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, DEPTH, 0);
#pragma unroll
        for (int i = 0; i < KS - DEPTH; i++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, DEPTH, 0);
        }
    };
    const float scale_log2 = A.sm_scale * 1.4426950408889634f;
    constexpr float kLazyMax = 8.f;
    float m_ref[4], l_run[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {
        m_ref[r] = -INFINITY;
        l_run[r] = 0.f;
    }
    // Scaled, masked logits of this wave's 16 rows of tile t (lane group g holds
    // heads 4g..4g+3), and whether any of them exceeds its head's reference
    // maximum by more than kLazyMax: only then does the softmax of the tile need
    // the exact tile maxima (and a reference may move). The flag goes to LDS for
    // tile parity `par`, where every wave reads all of them after the next barrier.
    auto tile_logits = [&](int t, const f32x4& sv, float (&x)[4], int par) {
        const bool valid = t * kTR + kn < nr;
        bool over = false;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            x[r] = valid ? sv[r] * scale_log2 : -INFINITY;
            over |= x[r] > m_ref[r] + kLazyMax;
        }
        flg[par][w] = __ballot(over) != 0ull;
    };
    // any wave's flag for tile parity par (the same answer in every wave)
    auto any_flag = [&](int par) -> bool {
        int a;
        if constexpr (NW >= 4) {
            const int4 f0 = *reinterpret_cast<const int4*>(&flg[par][0]);
            a = f0.x | f0.y | f0.z | f0.w;
            if constexpr (NW > 4) {
                const int4 f1 = *reinterpret_cast<const int4*>(&flg[par][4]);
                a |= f1.x | f1.y | f1.z | f1.w;
            }
        } else {
            a = flg[par][0] | flg[par][1];
        }
        return __builtin_amdgcn_readfirstlane(a) != 0;
    };

    f32x4 o[NHB][NCB];
#pragma unroll
    for (int h = 0; h < NHB; h++)
#pragma unroll
        for (int cb = 0; cb < NCB; cb++) o[h][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int hh = hb * 16 + 4 * g;   // first of this lane's four heads

    if (ntiles > 0) {
        // every wave issues exactly CPMAX copies per tile, so "tile t landed" is
        // "at most CPMAX copies per later tile still outstanding"
        issue(0);
        if (ntiles > 1) issue(1);
        if (ntiles > 2) issue(2);
        if (ntiles > 2) wait_vmcnt_mem<2 * CPMAX>();
        else if (ntiles > 1) wait_vmcnt_mem<CPMAX>();
        else wait_vmcnt_mem<0>();
        lds_barrier();
        float x[4];
        {
            f32x4 s0, s1;
            qk(ring0, s0, s1);
            tile_logits(0, s0 + s1, x, 0);
        }

        for (int t = 0; t < ntiles; t++) {
            const int par = t & 1;
            // B1: tile t+1 has landed (only tile t+2's copies may still be in
            // flight), the flags of tile t are visible, the slot of tile t-1 is free
            if (t + 2 < ntiles) wait_vmcnt_mem<CPMAX>();
            else wait_vmcnt_mem<0>();
            lds_barrier();
            if (t + 3 < ntiles) issue(t + 3);
            // ---- Q K^T of tile t+1 (matrix cores) ...
            f32x4 sn0 = {0.f, 0.f, 0.f, 0.f}, sn1 = {0.f, 0.f, 0.f, 0.f};
            if (t + 1 < ntiles) qk(slot_of(t + 1), sn0, sn1);
            // ... next to the softmax of tile t (vector units). A reference moves
            // only when a head's tile maximum exceeds it by more than kLazyMax; the
            // maxima are computed and exchanged between the row halves only in a
            // tile where some wave flagged that (the same for all waves).
            const bool rare = any_flag(par);
            float al[4] = {1.f, 1.f, 1.f, 1.f};
            if (rare) {
                float tm[4];
                bool moved = false;
#pragma unroll
                for (int r = 0; r < 4; r++) tm[r] = row16_max(x[r]);
                *reinterpret_cast<f32x4*>(&mx[rb][hh]) = f32x4{tm[0], tm[1], tm[2], tm[3]};
                lds_barrier();
                const f32x4 pm = *reinterpret_cast<const f32x4*>(&mx[rb ^ 1][hh]);
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const float tmax = __builtin_fmaxf(tm[r], pm[r]);
                    const bool mv = tmax > m_ref[r] + kLazyMax;
                    al[r] = mv ? __builtin_amdgcn_exp2f(m_ref[r] - tmax) : 1.f;
                    m_ref[r] = mv ? tmax : m_ref[r];
                    moved |= mv;
                }
                // both row halves compute the same alpha: every lane stores it
                *reinterpret_cast<f32x4*>(&alpha_s[hh]) = f32x4{al[0], al[1], al[2], al[3]};
                moved_w[w] = __ballot(moved) != 0ull;
            }
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float p = __builtin_amdgcn_exp2f(x[r] - m_ref[r]);
                l_run[r] = __builtin_fmaf(l_run[r], al[r], p);
                *reinterpret_cast<__bf16*>(&pbuf[(hh + r) * kPStride + kn * 2]) = static_cast<__bf16>(p);
            }
            if (t + 1 < ntiles) tile_logits(t + 1, sn0 + sn1, x, par ^ 1);
            // B2: P and alpha of tile t are visible. The values of the first four
            // column blocks of tile t (in its slot since the previous iteration)
            // are read on the way into the barrier.
            u32x2 va0[4], vb0[4];
            if constexpr (!KV8) {
                const uint32_t sb = (uint32_t)(uintptr_t)(const SIA_LDS uint8_t*)slot_of(t);
                uint32_t pa_[4], pb_[4];
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    pa_[q] = sb + voffL[0][q];
                    pb_[q] = sb + voffL[1][q];
                }
                ds_read_tr16x8_barrier(va0, vb0, pa_, pb_);
            } else {
                lds_barrier();
            }
            // ---- O = alpha * O + P V of tile t over this wave's columns
            int any = 0;
            if (rare) {
                if constexpr (NW >= 4) {
                    const int4 mv0 = *reinterpret_cast<const int4*>(&moved_w[0]);
                    any = mv0.x | mv0.y | mv0.z | mv0.w;
                    if constexpr (NW > 4) {
                        const int4 mv1 = *reinterpret_cast<const int4*>(&moved_w[4]);
                        any |= mv1.x | mv1.y | mv1.z | mv1.w;
                    }
                } else {
                    any = moved_w[0] | moved_w[1];
                }
            }
            if (__builtin_amdgcn_readfirstlane(any)) {
#pragma unroll
                for (int h = 0; h < NHB; h++) {
                    const f32x4 a4 = *reinterpret_cast<const f32x4*>(&alpha_s[h * 16 + 4 * g]);
#pragma unroll
                    for (int cb = 0; cb < NCB; cb++)
#pragma unroll
                        for (int r = 0; r < 4; r++) o[h][cb][r] *= a4[r];
                }
            }
            bf16x8 pa[NHB];
#pragma unroll
            for (int h = 0; h < NHB; h++)
                pa[h] = as_bf16x8(*reinterpret_cast<const u32x4*>(&pbuf[(h * 16 + jl) * kPStride + g * 16]));
            const uint8_t* buf = slot_of(t);
            if constexpr (KV8) {
                // fp8 values: row r of column block blk is code * scale[r][blk];
                // the scale goes into P (rounded to bf16), the codes are read
                // transposed (one 8-bit read per 16 columns: rows 8g .. 8g+7 of
                // column jl) and widened to bf16 exactly
                bf16x8 ps[NHB];
#pragma unroll
                for (int c0 = 0; c0 < NCB; c0 += 4) {
                    if ((c0 * 16) % 128 == 0) {   // first group of a 128-column block
                        const int blk = (w * CPW + c0 * 16) / 128;
                        float sc8[8];
#pragma unroll
                        for (int e = 0; e < 8; e++)
                            sc8[e] = *reinterpret_cast<const float*>(buf + (8 * g + e) * RF::RB + RF::SCALES + 4 * blk);
#pragma unroll
                        for (int h = 0; h < NHB; h++) ps[h] = scale_bf16x8(pa[h], sc8);
                    }
                    int off[4];
#pragma unroll
                    for (int q = 0; q < 4; q++)
                        off[q] = (8 * g + (jl >> 1)) * RF::RB + w * CPW + (c0 + q) * 16 + 8 * (jl & 1);
                    u32x2 vv[4];
                    ds_read_tr8x4(buf, off, vv);
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        const bf16x8 vb = e4m3x8_bf16x8(vv[q]);
#pragma unroll
                        for (int h = 0; h < NHB; h++) o[h][c0 + q] = mfma16(ps[h], vb, o[h][c0 + q]);
                    }
                }
            } else {
            const int(&voff)[2][4] = voffL;
#pragma unroll
            for (int c0 = 0; c0 < NCB; c0 += 4) {
                u32x2 va[4], vb2[4];
                if (c0 == 0) {
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        va[q] = va0[q];
                        vb2[q] = vb0[q];
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        const int cst = ((c0 + q) >> 2) * 128;
                        va[q] = ds_read_tr16(buf + voff[0][q] + cst);
                        vb2[q] = ds_read_tr16(buf + voff[1][q] + cst);
                    }
                    lds_wait(va, vb2);
                }
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const bf16x8 vb = as_bf16x8(u32x4{va[q][0], va[q][1], vb2[q][0], vb2[q][1]});
#pragma unroll
                    for (int h = 0; h < NHB; h++) o[h][c0 + q] = mfma16(pa[h], vb, o[h][c0 + q]);
                }
            }
            }
        }
    }
    wait_vmcnt<0>();

    // ---- finalize: per-head sums of both row halves, normalize and write
    {
        float ls[4];
#pragma unroll
        for (int r = 0; r < 4; r++) ls[r] = row16_sum(l_run[r]);
        if (jl == 0) {
            *reinterpret_cast<f32x4*>(&lsum[rb][hh]) = f32x4{ls[0], ls[1], ls[2], ls[3]};
            if (rb == 0) *reinterpret_cast<f32x4*>(&mfin[hh]) = f32x4{m_ref[0], m_ref[1], m_ref[2], m_ref[3]};
        }
    }
    __syncthreads();
    const bool split = A.n_split > 1;
#pragma unroll
    for (int h = 0; h < NHB; h++) {
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(&lsum[0][h * 16 + 4 * g]);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(&lsum[1][h * 16 + 4 * g]);
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const float lt = l0[r] + l1[r];
            const float inv = lt > 0.f ? 1.f / lt : 0.f;
            const int64_t head = head0 + h * 16 + 4 * g + r;
#pragma unroll
            for (int cb = 0; cb < NCB; cb++) {
                const int col = w * CPW + cb * 16 + jl;
                const float v = o[h][cb][r] * inv;
                if (split)
                    A.part_o[(((int64_t)j * A.n_split + sp) * A.heads + head) * kDV + col] = v;
                else
                    A.out[((int64_t)j * A.heads + head) * kDV + col] = (uint16_t)f32_to_bf16_rne(v);
            }
        }
    }
    if (tid < HB) {
        const float lt = lsum[0][tid] + lsum[1][tid];
        const float lse = lt > 0.f ? (mfin[tid] + log2f(lt)) * 0.6931471805599453f : -INFINITY;
        if (split)
            A.part_lse[((int64_t)j * A.n_split + sp) * A.heads + head0 + tid] = lse;
        else if (A.lse)
            A.lse[(int64_t)j * A.heads + head0 + tid] = lse;
    }
}

// ---------------------------------------------------------------------------
// Whole-tile variant for bf16 rows: workgroup = (query, block of 16 NWV heads,
// slice of the selected rows), NWV waves, wave w owning heads 16 w .. 16 w + 15
// of the block and ALL 32 rows of every tile. Per tile a wave computes
//   S^T = K Q^T   (rows x heads, 2 row blocks x 18 steps of 16x16x32 MFMAs; the
//                  query slice, 72 registers, stays in registers)
//   softmax       per head against the lazily moved reference maximum; every
//                 statistic of a head lives in the lanes of that head (column jl
//                 of S^T), so nothing is exchanged between waves
//   O^T += V^T P^T (32 column blocks, one MFMA each; P^T is the softmax output
//                 as it sits in registers, the value operand comes from
//                 transposing LDS reads)
// so one barrier per tile (the copy ring) is the only synchronisation. The K
// dimension of P V runs over the tile rows in the order the S^T accumulators
// hold them: slot 8 g + i is row 4 g + i (i < 4) or 16 + 4 g + (i - 4), and the
// value reads fetch the same rows. Output accumulator register r of column
// block cb holds column 16 cb + 4 g + r of head jl, so the rescale and the final
// normalisation are lane-local too.
//
// Tile layout in LDS: 36 blocks of 1 KB, block p holding the 16-byte chunks 2p
// and 2p + 1 of all 32 rows, 32 bytes per row (row r at 32 r). A Q K^T operand
// read then takes 16 rows x 16 bytes spread over 512 contiguous bytes and a
// transposing value read 4 rows x 32 contiguous bytes per 16 lanes, forms the
// LDS serves at close to its full rate (reads of 16-byte pieces of 16 rows 1152
// bytes apart run at about half of it, whatever the chunk swizzle). Every
// operand read is one base address per lane plus an immediate, and so is every
// copy: copy i fills block i with 32 bytes of each of the tile's 32 rows.
// ---------------------------------------------------------------------------

// Global -> LDS copy of 16 bytes per lane from src + OFF (OFF a byte immediate
// within the instruction's signed 13-bit range) to lds + 16 lane; otherwise as
// dma16. The instruction adds its offset to the LDS address as well (M0 + OFF +
// 16 lane), so M0 carries lds - OFF.
template <int OFF>
__device__ __forceinline__ void dma16_imm(const void* src, SIA_LDS void* lds) {
    static_assert(OFF >= 0 && OFF < 4096, "global instruction offset range");
    const uint32_t m = __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)) - (uint32_t)OFF);
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%2" ::"v"(src), "{m0}"(m), "n"(OFF) : "memory");
}

// Two fp32 values rounded to nearest even bf16 (the hardware conversion),
// packed (a in the low half).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, bf16x2v{static_cast<__bf16>(a), static_cast<__bf16>(b)});
}

// S^T block (+)= K Q^T with the query operand held in accumulation registers:
// the query slice is loop-invariant and only ever read by these MFMAs, which
// leaves the vector registers to the output accumulators (whose rescale is
// vector arithmetic). The compiler inserts no hazard waits around inline
// assembly: the key operand comes from LDS reads (the compiler waits for them
// before the asm), the query's accumulation registers are written once, long
// before (see qk_settle), and the result is read by vector code only after
// qk_settle or after a whole P V pass of MFMAs.
__device__ __forceinline__ void mfma16_qk0(f32x4& d, const bf16x8& k, const bf16x8& q) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(k), "a"(q));
}
__device__ __forceinline__ void mfma16_qk(f32x4& d, const bf16x8& k, const bf16x8& q) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(k), "a"(q));
}
// 32 wait states after the last MFMA, then the two logit blocks are defined.
__device__ __forceinline__ void qk_settle(f32x4 (&s)[2]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s[0]), "+v"(s[1]));
}

// Transposing 16-bit read (compiler form): rows k0 .. k0 + 3 of one column, as
// described at ds_read_tr16.
__device__ __forceinline__ u32x2 ds_read_tr16_c(const uint8_t* p) {
    typedef short s16x4v __attribute__((ext_vector_type(4)));
    const s16x4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SIA_LDS s16x4v*)(const SIA_LDS uint8_t*)p);
    return __builtin_bit_cast(u32x2, v);
}

// Copies K .. N-1 of one wave: block hb + NHB k from src + k STEP.
template <int K, int N, int STEP, int NHB>
__device__ __forceinline__ void wave_copies(const uint8_t* src, uint8_t* dst, int hb) {
    if constexpr (K < N) {
        dma16_imm<K * STEP>(src, (SIA_LDS void*)(dst + (hb + NHB * K) * 1024));
        wave_copies<K + 1, N, STEP, NHB>(src, dst, hb);
    }
}

// Copy K alone of the same set (K a std::integral_constant), so that a loop
// can spread a tile's copies between its MFMAs.
template <int STEP, int NHB, typename KC>
__device__ __forceinline__ void wave_copy_k(KC, const uint8_t* src, uint8_t* dst, int hb) {
    constexpr int K = KC::value;
    dma16_imm<K * STEP>(src, (SIA_LDS void*)(dst + (hb + NHB * K) * 1024));
}

// Calls f(std::integral_constant<int, k>{}) for 0 <= k < N (in an unrolled
// loop k is a constant and the tests fold away).
template <int N, int K = 0, typename F>
__device__ __forceinline__ void with_copy_index(int k, F&& f) {
    if constexpr (K < N) {
        if (k == K) f(std::integral_constant<int, K>{});
        else with_copy_index<N, K + 1>(k, f);
    }
}

// The copies of a later tile spread over a tile's 18 Q K^T steps: after step st
// go copies st CP / 18 .. (st + 1) CP / 18 - 1 (CP of them per tile).
template <int CP, int KS, typename F>
__device__ __forceinline__ void copies_after_step(int st, F&& f) {
#pragma unroll
    for (int k = st * CP / KS; k < (st + 1) * CP / KS; k++) with_copy_index<CP>(k, f);
}

// A copy issuer that issues nothing.
struct NoCopies {
    template <typename KC>
    __device__ void operator()(KC) const {}
};

// A value-operand reader that reads nothing.
struct NoReads {
    __device__ void operator()(int) const {}
};

// NHB blocks of 16 heads per workgroup; RH = 1: one wave per head block over
// 32-row tiles; RH = 2: 64-row tiles, two waves per head block, wave rh taking
// rows 32 rh .. 32 rh + 31 of every tile with a softmax of its own, the two
// merged by log-sum-exp at the end (twice the waves per SIMD for the same LDS
// traffic and MFMA work, where one workgroup per query and head block leaves a
// single wave per SIMD exposed to every latency).
template <int NHB, int RH>
struct WaveGeom {
    static constexpr int NW = NHB * RH;                   // waves
    static constexpr int HB = 16 * NHB;                   // heads per workgroup
    static constexpr int NT = NW * kWave;
    static constexpr int TR = 32 * RH;                    // rows per tile
    static constexpr int AHEAD = 4 / RH - 1;              // tiles issued ahead of the one computed
    // copies of a 32-row sub-tile: blocks hb + NHB k, by the waves of row half rh
    static constexpr int CP_LO = RowFmt<false>::COPIES / NHB;
    static constexpr int SPLIT = RowFmt<false>::COPIES % NHB;   // head blocks below issue one more
    static constexpr int CPMAX = CP_LO + (SPLIT ? 1 : 0);
    // Q K^T of tile t+1 runs before the softmax of tile t only where a wave has
    // the registers for two tiles' logits (one wave per SIMD)
    static constexpr bool PIPE = NW <= 4 && RH == 1;
    // the query slice in accumulation registers (Q K^T as inline assembly): only
    // with one wave per SIMD; at two the compiler would split the 256 registers
    // evenly between the two kinds
    static constexpr bool QA = NW <= 4;
};

template <int NHB, int RH>
__global__ __launch_bounds__(NHB * RH * kWave) void sparse_mla_wave_kernel(AttnArgs A) {
    using GM = WaveGeom<NHB, RH>;
    // (the pipelined loop spreads a tile's copies over the Q K^T steps: every
    // wave must issue the same count, CP_LO)
    static_assert(!GM::PIPE || GM::SPLIT == 0, "spread copies: the same count in every wave");
    constexpr int HB = GM::HB, NT = GM::NT, NW = GM::NW, CPMAX = GM::CPMAX, TR = GM::TR, AHEAD = GM::AHEAD;
    constexpr int TB = RowFmt<false>::TB;
    constexpr int KS = kDK / 32;    // 18 Q K^T steps
    constexpr int NCB = kDV / 16;   // 32 output column blocks
    static_assert(RowFmt<false>::CHUNKS == RowFmt<false>::COPIES * 64, "a tile is whole 1 KB copies");
    static_assert(RH == 1 || RH == 2, "row halves");
    __shared__ __attribute__((aligned(16))) uint8_t ring[4][TB];
    __shared__ __attribute__((aligned(16))) uint32_t rows[kMaxSliceRows];
    __shared__ int scan_s[16];
    __shared__ __attribute__((aligned(16))) float xm[RH == 2 ? NW : 1][16], xl[RH == 2 ? NW : 1][16];

    const int tid = threadIdx.x, l = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int hb = w % NHB, rh = w / NHB;   // head block, row half
    const int g = l >> 4, jl = l & 15;
    const int n_hb = A.heads / HB;

    // head blocks of one (query, slice) run on the same XCD one after another
    const int bid = blockIdx.x;
    const int xcd = bid & 7, slot = bid >> 3;
    const int num_pairs = A.num_q * A.n_split;
    const int P = (slot / n_hb) * 8 + xcd;
    const int hbk = slot % n_hb;
    if (P >= num_pairs) return;
    const int pair = num_pairs - 1 - P;
    const int j = pair / A.n_split, sp = pair % A.n_split;
    const int head0 = hbk * HB + 16 * hb;   // this wave's first head

    // The prologue's global reads in two rounds: the query slice, the sequence
    // id and the slice's indices (none depends on another), then the sequence
    // length and the page table entries of the indices (the query moves into
    // the accumulation registers only after the row list is built, so that its
    // loads do not hold up the rest).
    // ---- the wave's query as the B operand of Q K^T: step s, head head0 + jl,
    // dims 32 s + 8 g .. + 7
    bf16x8 qb[KS];
    {
        const uint16_t* qrow = A.q + ((int64_t)j * A.heads + head0 + jl) * kDK + g * 8;
#pragma unroll
        for (int s = 0; s < KS; s++) qb[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + s * 32));
    }
    const int r0 = sp * A.rows_per_split;
    const int r1_all = min(A.topk, r0 + A.rows_per_split);
    constexpr int RPT = kMaxSliceRows / NT;
    int sidx[RPT];
#pragma unroll
    for (int i = 0; i < RPT; i++) {
        const int r = r0 + tid * RPT + i;
        sidx[i] = r < r1_all ? A.idx[(int64_t)j * A.topk + r] : -1;
    }
    int b = A.q_seq[j];
    const bool seq_ok = b >= 0 && b < A.batch;
    if (!seq_ok) {
        if (tid == 0) atomicOr(A.status, kBadSeq);
        b = 0;
    }
    if (!seq_ok) {
#pragma unroll
        for (int i = 0; i < RPT; i++) sidx[i] = -1;
    }

    // ---- validated, compacted physical row ids of the slice (as in
    // sparse_mla_kernel)
    int nr = 0;
    {
        // (the page table entry of every index inside the table's span, read
        // beside the sequence length; the length check follows)
        int pg[RPT];
#pragma unroll
        for (int i = 0; i < RPT; i++) {
            const int s = sidx[i];
            pg[i] = s >= 0 && s < A.max_pages * kPage ? A.page_table[(int64_t)b * A.max_pages + (s >> 6)] : -1;
        }
        const int n_b = seq_ok ? A.seq_lens[b] : 0;
#pragma unroll
        for (int i = 0; i < RPT; i++) {
            const int s = sidx[i];
            const bool in = s >= 0 && s < n_b && s < A.max_pages * kPage;
            if (!in) pg[i] = -1;
            if (s >= 0 && !in) atomicOr(A.status, kBadIndex);
        }
        uint32_t row[RPT];
        int keep = 0;
#pragma unroll
        for (int i = 0; i < RPT; i++) {
            const int s = sidx[i];
            const bool in = s >= 0 && s < n_b && s < A.max_pages * kPage;
            const bool ok = in && pg[i] >= 0 && pg[i] < A.num_pages;
            if (in && !ok) atomicOr(A.status, kBadPage);
            row[i] = ok ? (uint32_t)pg[i] * kPage + (uint32_t)(s & 63) : 0xffffffffu;
            keep += ok;
        }
        int pre, tot;
        scan1<NT>(keep, pre, tot, scan_s);
#pragma unroll
        for (int i = 0; i < RPT; i++) {
            if (row[i] != 0xffffffffu) rows[pre++] = row[i];
        }
        nr = tot;
    }
    // the query into the accumulation registers, then the wait states a vector
    // write needs before an MFMA reads what it wrote
    if constexpr (GM::QA) {
#pragma unroll
        for (int s = 0; s < KS; s++) asm volatile("" : "+a"(qb[s]));
        asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
    }
    __syncthreads();
    const int ntiles = (nr + TR - 1) / TR;
    wait_vmcnt<0>();

    // 32-row sub-tile rh of tile t lives in ring slot (RH t + rh) % 4
    auto sub_of = [&](int t) -> uint8_t* { return ring[(RH * t + rh) & 3]; };
    // copies of tile t by wave (hb, rh): copy k fills block i = hb + NHB k of
    // sub-tile rh: lane l takes chunk 2 i + l % 2 of row 32 rh + l / 2 (rows past
    // the slice repeat its last row). A wave with one copy fewer repeats its
    // last one, so that every wave issues CPMAX copies per tile.
    // (the row id of a tile is read from LDS one tile ahead of its copies, so
    // that the copies do not wait for that read)
    auto row_of = [&](int t) -> uint32_t { return rows[min(t * TR + 32 * rh + (l >> 1), nr - 1)]; };
    auto issue = [&](int t, uint32_t row) {
        uint8_t* dst = sub_of(t);
        const uint8_t* src = reinterpret_cast<const uint8_t*>(A.kv) + (int64_t)row * kRowB + 32 * hb + 16 * (l & 1);
        constexpr int STEP = 32 * NHB;   // source bytes between a wave's copies
        wave_copies<0, GM::CP_LO, STEP, NHB>(src, dst, hb);
        if constexpr (GM::SPLIT) {
            // one more copy: block hb + NHB CP_LO where it exists, else a repeat
            const int k = hb < GM::SPLIT ? GM::CP_LO : GM::CP_LO - 1;
            dma16_imm<0>(src + STEP * k, (SIA_LDS void*)(dst + (hb + NHB * k) * 1024));
        }
    };

    // key operand of row block rb, step s: sub-tile row 16 rb + jl, chunk 4 s + g
    // (block 2 s + g / 2, half g % 2): kbase + 2048 s + 512 rb
    const int kbase = (g >> 1) * 1024 + jl * 32 + (g & 1) * 16;
    // value operand of column block cb, read e: lane addresses sub-tile row
    // 16 e + 4 g + jl / 4, chunk 2 cb + (jl / 2) % 2 (block cb), byte 8 (jl % 2):
    // vbase + 1024 cb + 512 e
    const int vbase = (4 * g + (jl >> 2)) * 32 + ((jl >> 1) & 1) * 16 + 8 * (jl & 1);

    const float scale_log2 = A.sm_scale * 1.4426950408889634f;
    constexpr float kLazyMax = 8.f;
    // reference maximum of head jl and the running sum over this lane's rows;
    // the finite start keeps exp2 of a masked logit at 0 in a wave that has not
    // met a valid row yet (a row half can start with an empty sub-tile)
    float m_ref = -1e30f, l_run = 0.f;

    // S^T of sub-tile `buf` for the wave's heads: s[rb] register r = logit of
    // sub-tile row 16 rb + 4 g + r and head jl. With xe/pk given, step st < 8
    // also computes exponential st of the previous tile's prepared logits (row
    // block st / 4, register st % 4), so that they run beside the MFMAs, and the
    // loop's end packs them into P^T. After the MFMAs of step st, cp issues that
    // step's share of a later tile's CPMAX copies (cp: NoCopies, or an issuer of
    // one copy); in the last VD steps (no key reads left) vr(i) reads value
    // operand i of the P V that follows (vr: NoReads, or its reader).
    constexpr int VD = GM::QA ? 4 : 2;
    auto qk = [&](const uint8_t* buf, f32x4 (&s)[2], const float (*xe)[4], bf16x8* pk, auto cp, auto vr) {
        float pe[2][4];
        constexpr int DEPTH = GM::QA ? 3 : 2;   // steps whose key operands are in flight
        auto kread = [&](int st, int rb) -> bf16x8 {
            return as_bf16x8(*reinterpret_cast<const u32x4*>(buf + kbase + st * 2048 + rb * 512));
        };
        bf16x8 kb[DEPTH][2];
#pragma unroll
        for (int i = 0; i < DEPTH; i++) {
            kb[i][0] = kread(i, 0);
            kb[i][1] = kread(i, 1);
        }
#pragma unroll
        for (int st = 0; st < KS; st++) {
            const bf16x8 k0 = kb[st % DEPTH][0], k1 = kb[st % DEPTH][1];
            if (st + DEPTH < KS) {
                kb[st % DEPTH][0] = kread(st + DEPTH, 0);
                kb[st % DEPTH][1] = kread(st + DEPTH, 1);
            }
            if constexpr (GM::QA) {
                if (st == 0) {
                    mfma16_qk0(s[0], k0, qb[st]);
                    mfma16_qk0(s[1], k1, qb[st]);
                } else {
                    mfma16_qk(s[0], k0, qb[st]);
                    mfma16_qk(s[1], k1, qb[st]);
                }
            } else {
                const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                s[0] = mfma16(k0, qb[st], st == 0 ? z : s[0]);
                s[1] = mfma16(k1, qb[st], st == 0 ? z : s[1]);
            }
            if (xe != nullptr && st < 8) {
                const int rb = st >> 2, r = st & 3;
                pe[rb][r] = __builtin_amdgcn_exp2f(xe[rb][r] - m_ref);
                l_run += pe[rb][r];
            }
            copies_after_step<CPMAX, KS>(st, cp);
            if (st >= KS - VD) vr(st - (KS - VD));
        }
        if (xe != nullptr)
            *pk = as_bf16x8(u32x4{pack_bf16x2(pe[0][0], pe[0][1]), pack_bf16x2(pe[0][2], pe[0][3]),
                                  pack_bf16x2(pe[1][0], pe[1][1]), pack_bf16x2(pe[1][2], pe[1][3])});
    };

    f32x4 o[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; cb++) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // softmax of the wave's sub-tile of tile t from its logits: P^T (bf16,
    // B-operand layout) for P V; moves the reference (rescaling O and the sum)
    // where a logit exceeds it by more than kLazyMax
    auto softmax = [&](int t, const f32x4 (&s)[2]) -> bf16x8 {
        float x[2][4];
        bool over = false;
#pragma unroll
        for (int rb = 0; rb < 2; rb++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const bool valid = t * TR + 32 * rh + rb * 16 + 4 * g + r < nr;
                x[rb][r] = valid ? s[rb][r] * scale_log2 : -INFINITY;
                over |= x[rb][r] > m_ref + kLazyMax;
            }
        if (__builtin_amdgcn_readfirstlane(__ballot(over) != 0ull ? 1 : 0)) {
            float tm = x[0][0];
#pragma unroll
            for (int rb = 0; rb < 2; rb++)
#pragma unroll
                for (int r = 0; r < 4; r++) tm = __builtin_fmaxf(tm, x[rb][r]);
            tm = __builtin_fmaxf(tm, __shfl_xor(tm, 16));
            tm = __builtin_fmaxf(tm, __shfl_xor(tm, 32));
            const bool mv = tm > m_ref + kLazyMax;
            const float al = mv ? __builtin_amdgcn_exp2f(m_ref - tm) : 1.f;
            m_ref = mv ? tm : m_ref;
            l_run *= al;
            if (__builtin_amdgcn_readfirstlane(__ballot(mv) != 0ull ? 1 : 0)) {
#pragma unroll
                for (int cb = 0; cb < NCB; cb++)
#pragma unroll
                    for (int r = 0; r < 4; r++) o[cb][r] *= al;
            }
        }
        float p[2][4];
#pragma unroll
        for (int rb = 0; rb < 2; rb++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                p[rb][r] = __builtin_amdgcn_exp2f(x[rb][r] - m_ref);
                l_run += p[rb][r];
            }
        return as_bf16x8(u32x4{pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                               pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3])});
    };

    // Logits of the wave's sub-tile of tile t, scaled to log2 units and masked
    // past the slice (x[rb][r]); moves the reference where a logit exceeds it by
    // more than kLazyMax, rescaling O and the sum.
    auto prep = [&](int t, const f32x4 (&s)[2], float (&x)[2][4]) {
        bool over = false;
#pragma unroll
        for (int rb = 0; rb < 2; rb++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const bool valid = t * TR + 32 * rh + rb * 16 + 4 * g + r < nr;
                x[rb][r] = valid ? s[rb][r] * scale_log2 : -INFINITY;
                over |= x[rb][r] > m_ref + kLazyMax;
            }
        if (__builtin_amdgcn_readfirstlane(__ballot(over) != 0ull ? 1 : 0)) {
            float tm = x[0][0];
#pragma unroll
            for (int rb = 0; rb < 2; rb++)
#pragma unroll
                for (int r = 0; r < 4; r++) tm = __builtin_fmaxf(tm, x[rb][r]);
            tm = __builtin_fmaxf(tm, __shfl_xor(tm, 16));
            tm = __builtin_fmaxf(tm, __shfl_xor(tm, 32));
            const bool mv = tm > m_ref + kLazyMax;
            const float al = mv ? __builtin_amdgcn_exp2f(m_ref - tm) : 1.f;
            m_ref = mv ? tm : m_ref;
            l_run *= al;
            if (__builtin_amdgcn_readfirstlane(__ballot(mv) != 0ull ? 1 : 0)) {
#pragma unroll
                for (int cb = 0; cb < NCB; cb++)
#pragma unroll
                    for (int r = 0; r < 4; r++) o[cb][r] *= al;
            }
        }
    };

    // O^T += V^T P^T over sub-tile `buf`: column block cb takes two transposing
    // reads (rows 4 g .., 16 + 4 g ..: its eight k slots, in P's order); the
    // reads of the next VD blocks are in flight during each MFMA
    auto vread = [&](const uint8_t* buf, int cb) -> bf16x8 {
        const u32x2 a = ds_read_tr16_c(buf + vbase + 1024 * cb);
        const u32x2 bb = ds_read_tr16_c(buf + vbase + 1024 * cb + 512);
        return as_bf16x8(u32x4{a[0], a[1], bb[0], bb[1]});
    };
    // (vb: the first VD value operands, read beforehand when `pre` is true)
    auto pv = [&](const uint8_t* buf, const bf16x8 pk, bf16x8 (&vb)[VD], bool pre) {
        if (!pre) {
#pragma unroll
            for (int i = 0; i < VD; i++) vb[i] = vread(buf, i);
        }
#pragma unroll
        for (int cb = 0; cb < NCB; cb++) {
            const bf16x8 v = vb[cb % VD];
            if (cb + VD < NCB) vb[cb % VD] = vread(buf, cb + VD);
            o[cb] = mfma16(v, pk, o[cb]);
        }
    };

    if (ntiles > 0) {
        // every wave issues exactly CPMAX copies per tile, so "tile t landed" is
        // "at most CPMAX copies per later tile still outstanding"
#pragma unroll
        for (int t = 0; t < AHEAD; t++)
            if (t < ntiles) issue(t, row_of(t));
        uint32_t row_next = row_of(AHEAD);
        if constexpr (GM::PIPE) {
            if (ntiles > 2) wait_vmcnt_mem<2 * CPMAX>();
            else if (ntiles > 1) wait_vmcnt_mem<CPMAX>();
            else wait_vmcnt_mem<0>();
            lds_barrier();
            float x[2][4];
            {
                f32x4 s[2];
                qk(sub_of(0), s, nullptr, nullptr, NoCopies{}, NoReads{});
                qk_settle(s);
                prep(0, s, x);
            }
            for (int t = 0; t < ntiles; t++) {
                // tile t+1 has landed (tile t+2's copies may still be in
                // flight), the slot of tile t-1 is free
                if (t + 2 < ntiles) wait_vmcnt_mem<CPMAX>();
                else wait_vmcnt_mem<0>();
                lds_barrier();
                // One branch-free block: Q K^T of tile t+1 with the exponentials
                // of tile t and the copies of tile t+3 between its MFMAs, then
                // P V of tile t (in the last iteration that Q K^T reads a slot of
                // stale rows and its result is not used; copies of a tile past
                // the last bring the slice's last row into the free slot of tile
                // t-1, unread). The logits of tile t+1 are prepared after P V.
                const uint8_t* cp_src = reinterpret_cast<const uint8_t*>(A.kv) + (int64_t)row_next * kRowB + 32 * hb + 16 * (l & 1);
                uint8_t* cp_dst = sub_of(t + 3);
                row_next = row_of(t + 4);
                auto copier = [&](auto kc) { wave_copy_k<32 * NHB, NHB>(kc, cp_src, cp_dst, hb); };
                f32x4 sn[2];
                bf16x8 pk;
                bf16x8 vb[VD];
                auto vreader = [&](int i) { vb[i] = vread(sub_of(t), i); };
                qk(sub_of(t + 1), sn, x, &pk, copier, vreader);
                pv(sub_of(t), pk, vb, true);
                if (t + 1 < ntiles) {
                    qk_settle(sn);
                    prep(t + 1, sn, x);
                }
            }
        } else {
            for (int t = 0; t < ntiles; t++) {
                // tile t has landed (the AHEAD - 1 tiles after it may still be
                // in flight), the slots of tile t-1 are free
                if (AHEAD > 2 && t + 2 < ntiles) wait_vmcnt_mem<(AHEAD > 2 ? 2 : 0) * CPMAX>();
                else if (AHEAD > 1 && t + 1 < ntiles) wait_vmcnt_mem<(AHEAD > 1 ? 1 : 0) * CPMAX>();
                else wait_vmcnt_mem<0>();
                lds_barrier();
                if (t + AHEAD < ntiles) {
                    issue(t + AHEAD, row_next);
                    row_next = row_of(t + AHEAD + 1);
                }
                f32x4 s[2];
                qk(sub_of(t), s, nullptr, nullptr, NoCopies{}, NoReads{});
                qk_settle(s);
                const bf16x8 pk = softmax(t, s);
                bf16x8 vb[VD];
                pv(sub_of(t), pk, vb, false);
            }
        }
    }
    wait_vmcnt<0>();

    // ---- finalize: the sums of the four lane groups; with two row halves the
    // halves merge first (log-sum-exp), wave rh finishing output columns
    // 256 rh .. 256 rh + 255 from its own and its partner's accumulators
    float lt = l_run;
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    float m_fin = m_ref, a_own = 1.f, a_oth = 0.f;
    constexpr int NCBF = NCB / RH;   // column blocks this wave finishes: rh NCBF ..
    const f32x4* xo = nullptr;
    if constexpr (RH == 2) {
        // the ring is free once every wave has left the loop
        __syncthreads();
        f32x4* mine = reinterpret_cast<f32x4*>(&ring[0][0]) + w * (NCBF * kWave);
        // (selects between static indices: an index that depends on rh would put
        // the accumulator array in scratch memory)
#pragma unroll
        for (int c = 0; c < NCBF; c++) mine[c * kWave + l] = rh == 0 ? o[NCBF + c] : o[c];
        if (g == 0) {
            xm[w][jl] = m_ref;
            xl[w][jl] = lt;
        }
        __syncthreads();
        const int pw = hb + NHB * (1 - rh);
        const float mp = xm[pw][jl], lp = xl[pw][jl];
        m_fin = __builtin_fmaxf(m_ref, mp);
        a_own = __builtin_amdgcn_exp2f(m_ref - m_fin);
        a_oth = __builtin_amdgcn_exp2f(mp - m_fin);
        lt = lt * a_own + lp * a_oth;
        xo = reinterpret_cast<const f32x4*>(&ring[0][0]) + pw * (NCBF * kWave);
    }
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int64_t head = head0 + jl;
    const int cb_first = rh * NCBF;
    auto final_block = [&](int c) -> f32x4 {
        f32x4 v = rh == 0 ? o[c] : o[(RH - 1) * NCBF + c];
        if constexpr (RH == 2) {
            const f32x4 u = xo[c * kWave + l];
#pragma unroll
            for (int r = 0; r < 4; r++) v[r] = v[r] * a_own + u[r] * a_oth;
        }
        return v * inv;
    };
    if (A.n_split > 1) {
        float* dst = A.part_o + (((int64_t)j * A.n_split + sp) * A.heads + head) * kDV + 4 * g + 16 * cb_first;
#pragma unroll
        for (int c = 0; c < NCBF; c++) *reinterpret_cast<f32x4*>(dst + c * 16) = final_block(c);
    } else {
        uint16_t* dst = A.out + ((int64_t)j * A.heads + head) * kDV + 4 * g + 16 * cb_first;
#pragma unroll
        for (int c = 0; c < NCBF; c++) {
            const f32x4 v = final_block(c);
            *reinterpret_cast<u32x2*>(dst + c * 16) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
    }
    if (g == 0 && rh == 0) {
        const float lse = lt > 0.f ? (m_fin + log2f(lt)) * 0.6931471805599453f : -INFINITY;
        if (A.n_split > 1)
            A.part_lse[((int64_t)j * A.n_split + sp) * A.heads + head] = lse;
        else if (A.lse)
            A.lse[(int64_t)j * A.heads + head] = lse;
    }
}

// ---------------------------------------------------------------------------
// Wide whole-tile variant for bf16 rows: 128 heads per workgroup in 4 waves of
// 32 (one wave per SIMD). As in sparse_mla_wave_kernel every wave takes all 32
// rows of a tile, but with two 16-head blocks per wave each key and value
// operand read from LDS feeds two MFMAs, which halves the LDS traffic per
// flop. Registers: the query slice (2 x 72) in vector registers and the output
// accumulators (2 x 32 blocks of 4 = 256) in the accumulation registers; the
// P V MFMAs are inline assembly on those, and no vector instruction touches
// the accumulators inside the loop (the compiler would otherwise keep copies of
// them in vector registers): the rare rescale when a reference maximum moves
// goes through a per-wave LDS buffer, as does the final normalisation.
// ---------------------------------------------------------------------------
constexpr int kWideNW = 4;                       // waves
constexpr int kWideHB = 32 * kWideNW;            // heads per workgroup
constexpr int kWideCP = RowFmt<false>::COPIES / kWideNW;   // copies per wave and tile
static_assert(RowFmt<false>::COPIES % kWideNW == 0, "copies split evenly");

// O^T block += V^T P^T with the accumulator in accumulation registers. The
// compiler inserts no hazard waits around inline assembly: P (written by
// vector instructions) goes through p_settle first; the value operand comes
// from LDS reads the compiler waits for.
__device__ __forceinline__ void mfma16_pv_acc(f32x4& d, const bf16x8& v, const bf16x8& p) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(v), "v"(p));
}
// 16 wait states after the vector instructions that wrote P^T of both head
// blocks (a read of an operand fewer than 6 wait states after its write has
// returned the old contents), then P^T is defined.
__device__ __forceinline__ void p_settle(bf16x8 (&pk)[2]) {
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(pk[0]), "+v"(pk[1]));
}
// An accumulation-register block set to zero by an MFMA of zero operands.
__device__ __forceinline__ void acc_zero(f32x4& d, const bf16x8& z) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %1, 0" : "=a"(d) : "v"(z));
}
// Accumulation-register block -> LDS (16 bytes per lane at lds), and back.
__device__ __forceinline__ void acc_to_lds(uint32_t lds, const f32x4& d) {
    asm volatile("ds_write_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(lds), "a"(d) : "memory");
}
__device__ __forceinline__ void acc_from_lds(uint32_t lds, f32x4& d) {
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=a"(d) : "v"(lds) : "memory");
}

__global__ __launch_bounds__(kWideNW * kWave) void sparse_mla_wide_kernel(AttnArgs A) {
    constexpr int NT = kWideNW * kWave, HB = kWideHB;
    constexpr int TB = RowFmt<false>::TB;
    constexpr int KS = kDK / 32;    // 18 Q K^T steps
    constexpr int NCB = kDV / 16;   // 32 output column blocks
    __shared__ __attribute__((aligned(16))) uint8_t ring[4][TB];
    __shared__ __attribute__((aligned(16))) uint32_t rows[kMaxSliceRows];
    __shared__ int scan_s[16];
    __shared__ __attribute__((aligned(16))) f32x4 resc[kWideNW][kWave];   // per-wave rescale buffer

    const int tid = threadIdx.x, l = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int g = l >> 4, jl = l & 15;
    const int n_hb = A.heads / HB;

    const int bid = blockIdx.x;
    const int xcd = bid & 7, slot = bid >> 3;
    const int num_pairs = A.num_q * A.n_split;
    const int P = (slot / n_hb) * 8 + xcd;
    const int hbk = slot % n_hb;
    if (P >= num_pairs) return;
    const int pair = num_pairs - 1 - P;
    const int j = pair / A.n_split, sp = pair % A.n_split;
    const int head0 = hbk * HB + 32 * w;   // this wave's first head; block h: head0 + 16 h

    // The prologue's global reads in two rounds: the query slices, the
    // sequence id and the slice's indices (none depends on another), then the
    // sequence length and the page table entries of the indices.
    // ---- the wave's query as the B operand of Q K^T: block h, step s: head
    // head0 + 16 h + jl, dims 32 s + 8 g .. + 7
    bf16x8 qb[2][KS];
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const uint16_t* qrow = A.q + ((int64_t)j * A.heads + head0 + 16 * h + jl) * kDK + g * 8;
#pragma unroll
        for (int s = 0; s < KS; s++) qb[h][s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + s * 32));
    }
    const int r0 = sp * A.rows_per_split;
    const int r1_all = min(A.topk, r0 + A.rows_per_split);
    constexpr int RPT = kMaxSliceRows / NT;
    int sidx[RPT];
#pragma unroll
    for (int i = 0; i < RPT; i++) {
        const int r = r0 + tid * RPT + i;
        sidx[i] = r < r1_all ? A.idx[(int64_t)j * A.topk + r] : -1;
    }
    int b = A.q_seq[j];
    const bool seq_ok = b >= 0 && b < A.batch;
    if (!seq_ok) {
        if (tid == 0) atomicOr(A.status, kBadSeq);
        b = 0;
    }
    if (!seq_ok) {
#pragma unroll
        for (int i = 0; i < RPT; i++) sidx[i] = -1;
    }

    // ---- validated, compacted physical row ids of the slice (as in
    // sparse_mla_kernel)
    int nr = 0;
    {
        // (the page table entry of every index inside the table's span, read
        // beside the sequence length; the length check follows)
        int pg[RPT];
#pragma unroll
        for (int i = 0; i < RPT; i++) {
            const int s = sidx[i];
            pg[i] = s >= 0 && s < A.max_pages * kPage ? A.page_table[(int64_t)b * A.max_pages + (s >> 6)] : -1;
        }
        const int n_b = seq_ok ? A.seq_lens[b] : 0;
#pragma unroll
        for (int i = 0; i < RPT; i++) {
            const int s = sidx[i];
            const bool in = s >= 0 && s < n_b && s < A.max_pages * kPage;
            if (!in) pg[i] = -1;
            if (s >= 0 && !in) atomicOr(A.status, kBadIndex);
        }
        uint32_t row[RPT];
        int keep = 0;
#pragma unroll
        for (int i = 0; i < RPT; i++) {
            const int s = sidx[i];
            const bool in = s >= 0 && s < n_b && s < A.max_pages * kPage;
            const bool ok = in && pg[i] >= 0 && pg[i] < A.num_pages;
            if (in && !ok) atomicOr(A.status, kBadPage);
            row[i] = ok ? (uint32_t)pg[i] * kPage + (uint32_t)(s & 63) : 0xffffffffu;
            keep += ok;
        }
        int pre, tot;
        scan1<NT>(keep, pre, tot, scan_s);
#pragma unroll
        for (int i = 0; i < RPT; i++) {
            if (row[i] != 0xffffffffu) rows[pre++] = row[i];
        }
        nr = tot;
    }
    __syncthreads();
    const int ntiles = (nr + kTR - 1) / kTR;
    wait_vmcnt<0>();

    // copies of tile t (layout as in sparse_mla_wave_kernel): copy k of wave w
    // fills block w + 4 k with chunk 2 (w + 4 k) + l % 2 of tile row l / 2
    // (the row id of a tile is read from LDS one tile ahead of its copies, so
    // that the copies do not wait for that read)
    auto row_of = [&](int t) -> uint32_t { return rows[min(t * kTR + (l >> 1), nr - 1)]; };
    auto issue = [&](int t, uint32_t row) {
        uint8_t* dst = ring[t & 3];
        const uint8_t* src = reinterpret_cast<const uint8_t*>(A.kv) + (int64_t)row * kRowB + 32 * w + 16 * (l & 1);
        wave_copies<0, kWideCP, 32 * kWideNW, kWideNW>(src, dst, w);
    };
    const int kbase = (g >> 1) * 1024 + jl * 32 + (g & 1) * 16;
    const int vbase = (4 * g + (jl >> 2)) * 32 + ((jl >> 1) & 1) * 16 + 8 * (jl & 1);

    const float scale_log2 = A.sm_scale * 1.4426950408889634f;
    constexpr float kLazyMax = 8.f;
    // reference maximum and running sum (over this lane's rows) of the lane's
    // head in each block
    float m_ref[2] = {-1e30f, -1e30f}, l_run[2] = {0.f, 0.f};
    // S^T of tile `buf`: s[rb][h] register r = logit of row 16 rb + 4 g + r and
    // head head0 + 16 h + jl; each key operand read serves both head blocks.
    // With xe/pk given, step st < 16 also computes exponential st of the
    // previous tile's prepared logits (the 16 of this lane: block st / 8, row
    // block (st / 4) % 2, register st % 4), so that they run beside the MFMAs,
    // and the last step packs them into P^T. After the MFMAs of step st, cp
    // issues that step's share of a later tile's kWideCP copies (cp: NoCopies,
    // or an issuer of one copy), so that the copies' address work runs beside
    // the MFMAs too; in the last VD steps (no key reads left) vr(i) reads value
    // operand i of the P V that follows (vr: NoReads, or its reader).
    constexpr int VD = 4;
    auto qk = [&](const uint8_t* buf, f32x4 (&s)[2][2], const float (*xe)[2][4], bf16x8* pk, auto cp, auto vr) {
        float pe[2][2][4];
        constexpr int DEPTH = 3;
        auto kread = [&](int st, int rb) -> bf16x8 {
            return as_bf16x8(*reinterpret_cast<const u32x4*>(buf + kbase + st * 2048 + rb * 512));
        };
        bf16x8 kb[DEPTH][2];
#pragma unroll
        for (int i = 0; i < DEPTH; i++) {
            kb[i][0] = kread(i, 0);
            kb[i][1] = kread(i, 1);
        }
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < KS; st++) {
            const bf16x8 k0 = kb[st % DEPTH][0], k1 = kb[st % DEPTH][1];
            if (st + DEPTH < KS) {
                kb[st % DEPTH][0] = kread(st + DEPTH, 0);
                kb[st % DEPTH][1] = kread(st + DEPTH, 1);
            }
#pragma unroll
            for (int h = 0; h < 2; h++) {
                s[0][h] = mfma16(k0, qb[h][st], st == 0 ? z : s[0][h]);
                s[1][h] = mfma16(k1, qb[h][st], st == 0 ? z : s[1][h]);
            }
            if (xe != nullptr && st < 16) {
                const int h = st >> 3, rb = (st >> 2) & 1, r = st & 3;
                pe[h][rb][r] = __builtin_amdgcn_exp2f(xe[h][rb][r] - m_ref[h]);
                l_run[h] += pe[h][rb][r];
            }
            copies_after_step<kWideCP, KS>(st, cp);
            if (st >= KS - VD) vr(st - (KS - VD));
        }
        if (xe != nullptr) {
#pragma unroll
            for (int h = 0; h < 2; h++)
                pk[h] = as_bf16x8(u32x4{pack_bf16x2(pe[h][0][0], pe[h][0][1]), pack_bf16x2(pe[h][0][2], pe[h][0][3]),
                                        pack_bf16x2(pe[h][1][0], pe[h][1][1]), pack_bf16x2(pe[h][1][2], pe[h][1][3])});
        }
    };

    f32x4 o[2][NCB];
    {
        bf16x8 zb = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
        asm volatile("s_nop 7\n\ts_nop 7" : "+v"(zb));   // (wait states after its vector write)
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
            for (int cb = 0; cb < NCB; cb++) acc_zero(o[h][cb], zb);
    }
    const uint32_t resc_lds = (uint32_t)(uintptr_t)(SIA_LDS f32x4*)&resc[w][l];

    // Logits of tile t for both head blocks, scaled to log2 units and masked
    // past the slice (x[h][rb][r]); moves a block's reference where a logit
    // exceeds it by more than kLazyMax, rescaling that block's accumulators
    // through LDS and its sum (in tile 0 the accumulators are still zero).
    auto prep = [&](int t, const f32x4 (&s)[2][2], float (&x)[2][2][4]) {
#pragma unroll
        for (int h = 0; h < 2; h++) {
            bool over = false;
#pragma unroll
            for (int rb = 0; rb < 2; rb++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const bool valid = t * kTR + rb * 16 + 4 * g + r < nr;
                    x[h][rb][r] = valid ? s[rb][h][r] * scale_log2 : -INFINITY;
                    over |= x[h][rb][r] > m_ref[h] + kLazyMax;
                }
            if (__builtin_amdgcn_readfirstlane(__ballot(over) != 0ull ? 1 : 0)) {
                float tm = x[h][0][0];
#pragma unroll
                for (int rb = 0; rb < 2; rb++)
#pragma unroll
                    for (int r = 0; r < 4; r++) tm = __builtin_fmaxf(tm, x[h][rb][r]);
                tm = __builtin_fmaxf(tm, __shfl_xor(tm, 16));
                tm = __builtin_fmaxf(tm, __shfl_xor(tm, 32));
                const bool mv = tm > m_ref[h] + kLazyMax;
                const float al = mv ? __builtin_amdgcn_exp2f(m_ref[h] - tm) : 1.f;
                m_ref[h] = mv ? tm : m_ref[h];
                l_run[h] *= al;
                if (t > 0 && __builtin_amdgcn_readfirstlane(__ballot(mv) != 0ull ? 1 : 0)) {
                    // (the previous tile's P V MFMAs wrote these accumulators:
                    // 32 wait states before the LDS writes read them)
                    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
                    for (int cb = 0; cb < NCB; cb++) {
                        acc_to_lds(resc_lds, o[h][cb]);
                        f32x4 v = resc[w][l];
                        v *= al;
                        resc[w][l] = v;
                        lds_wait_all();
                        acc_from_lds(resc_lds, o[h][cb]);
                    }
                }
            }
        }
    };
    // O^T += V^T P^T over tile `buf`: each value operand (two transposing reads)
    // serves both head blocks
    // (the first VD value operands are read during the preceding Q K^T)
    auto vread = [&](const uint8_t* buf, int cb) -> bf16x8 {
        const u32x2 a = ds_read_tr16_c(buf + vbase + 1024 * cb);
        const u32x2 bb = ds_read_tr16_c(buf + vbase + 1024 * cb + 512);
        return as_bf16x8(u32x4{a[0], a[1], bb[0], bb[1]});
    };
    auto pv = [&](const uint8_t* buf, const bf16x8 (&pk)[2], bf16x8 (&vb)[VD]) {
#pragma unroll
        for (int cb = 0; cb < NCB; cb++) {
            const bf16x8 v = vb[cb % VD];
            if (cb + VD < NCB) vb[cb % VD] = vread(buf, cb + VD);
            mfma16_pv_acc(o[0][cb], v, pk[0]);
            mfma16_pv_acc(o[1][cb], v, pk[1]);
        }
    };

    if (ntiles > 0) {
        // Q K^T of tile t+1 goes out before the softmax of tile t, so that the
        // matrix cores work through it while the softmax runs
        issue(0, row_of(0));
        if (ntiles > 1) issue(1, row_of(1));
        if (ntiles > 2) issue(2, row_of(2));
        uint32_t row_next = row_of(3);
        if (ntiles > 2) wait_vmcnt_mem<2 * kWideCP>();
        else if (ntiles > 1) wait_vmcnt_mem<kWideCP>();
        else wait_vmcnt_mem<0>();
        lds_barrier();
        float x[2][2][4];
        {
            f32x4 s[2][2];
            qk(ring[0], s, nullptr, nullptr, NoCopies{}, NoReads{});
            prep(0, s, x);
        }
        for (int t = 0; t < ntiles; t++) {
            // tile t+1 has landed (tile t+2's copies may still be in flight),
            // the slot of tile t-1 is free
            if (t + 2 < ntiles) wait_vmcnt_mem<kWideCP>();
            else wait_vmcnt_mem<0>();
            lds_barrier();
            // No branch from here to the end of P V: one scheduling region in
            // which the exponentials of tile t and the copies of tile t+3 sit
            // between the MFMAs of the next tile's Q K^T. (In the last iteration
            // that Q K^T reads a slot of stale rows and its result is not used;
            // the copies of a tile past the last, of the slice's last row, land
            // in the free slot of tile t-1 and are not read.)
            const uint8_t* cp_src = reinterpret_cast<const uint8_t*>(A.kv) + (int64_t)row_next * kRowB + 32 * w + 16 * (l & 1);
            uint8_t* cp_dst = ring[(t + 3) & 3];
            row_next = row_of(t + 4);
            auto copier = [&](auto kc) { wave_copy_k<32 * kWideNW, kWideNW>(kc, cp_src, cp_dst, w); };
            f32x4 sn[2][2];
            bf16x8 pk[2];
            bf16x8 vb[VD];
            auto vreader = [&](int i) { vb[i] = vread(ring[t & 3], i); };
            qk(ring[(t + 1) & 3], sn, x, pk, copier, vreader);
            p_settle(pk);
            pv(ring[t & 3], pk, vb);
            if (t + 1 < ntiles) prep(t + 1, sn, x);
        }
    }
    wait_vmcnt<0>();

    // ---- finalize: each head block's accumulators through this wave's part of
    // the (now free) ring: 32 blocks x 1 KB, normalized on the way out
    __syncthreads();
    // the last P V MFMAs are read by the LDS writes below: 32 wait states first
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    f32x4* stage = reinterpret_cast<f32x4*>(&ring[0][0]) + w * (NCB * kWave);
    const uint32_t stage_lds = (uint32_t)(uintptr_t)(SIA_LDS f32x4*)stage;
#pragma unroll
    for (int h = 0; h < 2; h++) {
        float lt = l_run[h];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
        for (int cb = 0; cb < NCB; cb++) acc_to_lds(stage_lds + (cb * kWave + l) * 16, o[h][cb]);
        lds_wait_all();
        const int64_t head = head0 + 16 * h + jl;
        if (A.n_split > 1) {
            float* dst = A.part_o + (((int64_t)j * A.n_split + sp) * A.heads + head) * kDV + 4 * g;
#pragma unroll
            for (int cb = 0; cb < NCB; cb++) *reinterpret_cast<f32x4*>(dst + cb * 16) = stage[cb * kWave + l] * inv;
        } else {
            uint16_t* dst = A.out + ((int64_t)j * A.heads + head) * kDV + 4 * g;
#pragma unroll
            for (int cb = 0; cb < NCB; cb++) {
                const f32x4 v = stage[cb * kWave + l] * inv;
                *reinterpret_cast<u32x2*>(dst + cb * 16) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            }
        }
        // (the next block's writes reuse the stage only after these reads)
        lds_wait_all();
        if (g == 0) {
            const float lse = lt > 0.f ? (m_ref[h] + log2f(lt)) * 0.6931471805599453f : -INFINITY;
            if (A.n_split > 1)
                A.part_lse[((int64_t)j * A.n_split + sp) * A.heads + head] = lse;
            else if (A.lse)
                A.lse[(int64_t)j * A.heads + head] = lse;
        }
    }
}

// Merge of the row slices of one (query, head) by log-sum-exp.
__global__ __launch_bounds__(128) void mla_combine_kernel(AttnArgs A) {
    const int64_t jh = blockIdx.x;            // query * heads + head
    const int64_t j = jh / A.heads, h = jh % A.heads;
    float mx = -INFINITY;
    for (int s = 0; s < A.n_split; s++) mx = fmaxf(mx, A.part_lse[(j * A.n_split + s) * A.heads + h]);
    float wsum = 0.f;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    const int c0 = threadIdx.x * 4;
    if (mx != -INFINITY) {
        for (int s = 0; s < A.n_split; s++) {
            const float ls = A.part_lse[(j * A.n_split + s) * A.heads + h];
            const float wgt = __expf(ls - mx);
            wsum += wgt;
            const f32x4 v = *reinterpret_cast<const f32x4*>(A.part_o + ((j * A.n_split + s) * A.heads + h) * kDV + c0);
#pragma unroll
            for (int e = 0; e < 4; e++) acc[e] += wgt * v[e];
        }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    uint16_t* dst = A.out + (j * A.heads + h) * kDV + c0;
    const uint32_t lo = f32_to_bf16_rne(acc[0] * inv) | (f32_to_bf16_rne(acc[1] * inv) << 16);
    const uint32_t hi = f32_to_bf16_rne(acc[2] * inv) | (f32_to_bf16_rne(acc[3] * inv) << 16);
    *reinterpret_cast<u32x2*>(dst) = u32x2{lo, hi};
    if (threadIdx.x == 0 && A.lse) A.lse[j * A.heads + h] = wsum > 0.f ? mx + logf(wsum) : -INFINITY;
}

template <int HB, bool KV8>
static hipError_t mla_launch(const AttnArgs& a, hipStream_t st) {
    const int n_hb = a.heads / HB;
    const int64_t pairs = (int64_t)a.num_q * a.n_split;
    const int64_t blocks = (pairs + 7) / 8 * 8 * n_hb;
    hipLaunchKernelGGL((sparse_mla_kernel<HB, KV8>), dim3((unsigned)blocks), dim3(MlaGeom<HB, KV8>::NT), 0, st, a);
    return hipGetLastError();
}

template <int NHB, int RH>
static hipError_t mla_wave_launch(const AttnArgs& a, hipStream_t st) {
    using GM = WaveGeom<NHB, RH>;
    const int n_hb = a.heads / GM::HB;
    const int64_t pairs = (int64_t)a.num_q * a.n_split;
    const int64_t blocks = (pairs + 7) / 8 * 8 * n_hb;
    hipLaunchKernelGGL((sparse_mla_wave_kernel<NHB, RH>), dim3((unsigned)blocks), dim3(GM::NT), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_sparse_mla(const AttnArgs& a, hipStream_t st) {
    if (a.wave_heads == 3 && !a.kv8 && a.heads_per_block == kWideHB) {
        const int64_t pairs = (int64_t)a.num_q * a.n_split;
        const int64_t blocks = (pairs + 7) / 8 * 8 * (a.heads / kWideHB);
        hipLaunchKernelGGL(sparse_mla_wide_kernel, dim3((unsigned)blocks), dim3(kWideNW * kWave), 0, st, a);
        return hipGetLastError();
    }
    if (a.wave_heads && !a.kv8) {
        switch (a.heads_per_block * 4 + a.wave_heads) {
            case 128 * 4 + 1: return mla_wave_launch<8, 1>(a, st);
            case 64 * 4 + 1: return mla_wave_launch<4, 1>(a, st);
            case 32 * 4 + 1: return mla_wave_launch<2, 1>(a, st);
            case 64 * 4 + 2: return mla_wave_launch<4, 2>(a, st);
            case 32 * 4 + 2: return mla_wave_launch<2, 2>(a, st);
            default: return hipErrorInvalidValue;
        }
    }
    switch (a.heads_per_block * 2 + (a.kv8 ? 1 : 0)) {
        case 128: return mla_launch<64, false>(a, st);
        case 64: return mla_launch<32, false>(a, st);
        case 32: return mla_launch<16, false>(a, st);
        case 129: return mla_launch<64, true>(a, st);
        case 65: return mla_launch<32, true>(a, st);
        case 33: return mla_launch<16, true>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_mla_combine(const AttnArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)((int64_t)a.num_q * a.heads)), dim3(128), 0,
                       st, a);
    return hipGetLastError();
}

}  // namespace sia
