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
// list of physical row ids in LDS. Then, per tile of 32 rows:
//   copy     the tile's rows go from HBM straight into an LDS ring slot (36 KB,
//            three slots, direct global -> LDS copies issued two tiles ahead),
//            row-major, with the 16-byte chunks of a row XOR-swizzled by the row
//            index so that both operand reads below are free of bank conflicts
//   Q K^T    wave (hb, rb) computes logits of its 16 heads x 16 rows with
//            16x16x32 MFMAs over all 576 columns; its Q slice stays in registers
//   softmax  online, per head: the two row-block waves of a head block exchange
//            their tile maxima through LDS; P goes to LDS as bf16
//   P V      wave w owns output columns [w*512/NW, (w+1)*512/NW) of all heads;
//            the value operand is read from the same row-major tile with
//            transposing LDS reads (ds_read_b64_tr_b16), so no transposed copy
//            of the values is ever made
// Slices of one query are merged afterwards by log-sum-exp.
#include "sia_device.h"
#include "sia_kernels.h"

namespace sia {

constexpr int kDK = 576, kDV = 512;
constexpr int kRowB = kDK * 2;              // bytes per latent row (1152 = 72 chunks of 16)
constexpr int kRowChunks = kRowB / 16;
constexpr int kTR = 32;                     // rows per tile
constexpr int kTileB = kTR * kRowB;         // 36864
constexpr int kTileCopies = kTileB / 1024;  // 36 copies of 64 lanes x 16 bytes
constexpr int kPStride = kTR * 2 + 16;      // bytes per head of P (padded: no bank conflicts)
constexpr int kMaxSliceRows = kAttnMaxSliceRows;
constexpr int kQKHalf = kDK / 64;           // 32-column MFMA steps over half a row (9)

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

// Byte offset of logical 16-byte chunk c of tile row r (chunks are XOR-swizzled
// by r within aligned groups of eight).
__device__ __forceinline__ int tile_off(int r, int c) { return r * kRowB + ((c ^ (r & 7)) << 4); }

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

template <int HB>
struct MlaGeom {
    static constexpr int NHB = HB / 16;          // 16-head blocks
    static constexpr int NW = 2 * NHB;           // waves: (head block, row block)
    static constexpr int NT = NW * kWave;
    static constexpr int CPW = kDV / NW;         // output columns per wave
    static constexpr int NCB = CPW / 16;         // 16-column blocks per wave
    // tile copies per wave: waves below SPLIT issue one more than the rest
    static constexpr int CP_LO = kTileCopies / NW;
    static constexpr int SPLIT = kTileCopies % NW;
};

template <int HB>
__global__ __attribute__((amdgpu_flat_work_group_size(1, 512))) void sparse_mla_kernel(AttnArgs A) {
    using GM = MlaGeom<HB>;
    constexpr int NHB = GM::NHB, NW = GM::NW, NT = GM::NT, CPW = GM::CPW, NCB = GM::NCB;
    __shared__ __attribute__((aligned(16))) uint8_t ring0[kTileB];
    __shared__ __attribute__((aligned(16))) uint8_t ring1[kTileB];
    __shared__ __attribute__((aligned(16))) uint8_t ring2[kTileB];
    __shared__ __attribute__((aligned(16))) uint32_t rows[kMaxSliceRows];
    __shared__ __attribute__((aligned(16))) uint8_t pbuf[HB * kPStride];
    __shared__ __attribute__((aligned(16))) f32x4 sx[NW][2][kWave];   // partial logits, lane layout
    __shared__ __attribute__((aligned(16))) float alpha_s[HB];
    __shared__ __attribute__((aligned(16))) float lsum[HB];
    __shared__ __attribute__((aligned(16))) float mfin[HB];
    __shared__ int scan_s[16];
    __shared__ int rescale[2];   // by tile parity: some head's reference max moved

    const int tid = threadIdx.x, l = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform
    const int g = l >> 4, jl = l & 15;
    const int n_hb = A.heads / HB;

    // XCD-aware block order: the head blocks of one (query, slice) pair get block
    // ids 8 apart, which the dispatcher places on the same XCD (shared L2), so the
    // second copy of the pair's rows is served from L2.
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

    // ---- Q slice of this wave in registers (issued first, waited for below):
    // its 16 heads, columns [288 rb, 288 rb + 288)
    const int hb = w % NHB, rb = w / NHB;
    bf16x8 qa[kQKHalf];
    {
        const uint16_t* qrow = A.q + ((int64_t)j * A.heads + head0 + hb * 16 + jl) * kDK + rb * (kDK / 2) + g * 8;
#pragma unroll
        for (int ks = 0; ks < kQKHalf; ks++)
            qa[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + ks * 32));
    }

    // ---- validated, compacted physical row ids of the slice
    int nr = 0;
    for (int base = r0; base < r1; base += NT) {
        const int r = base + tid;
        uint32_t row = 0u;
        int keep = 0;
        if (r < r1) {
            const int s = A.idx[(int64_t)j * A.topk + r];
            if (s >= 0) {
                if (s >= n_b || s >= A.max_pages * kPage) {
                    atomicOr(A.status, kBadIndex);
                } else {
                    const int page = A.page_table[(int64_t)b * A.max_pages + (s >> 6)];
                    if (page >= 0 && page < A.num_pages) {
                        row = (uint32_t)page * kPage + (uint32_t)(s & 63);
                        keep = 1;
                    } else {
                        atomicOr(A.status, kBadPage);
                    }
                }
            }
        }
        int pre, tot;
        scan1<NT>(keep, pre, tot, scan_s);
        if (keep) rows[nr + pre] = row;
        nr += tot;
    }
    __syncthreads();
    const int ntiles = (nr + kTR - 1) / kTR;
    wait_vmcnt<0>();   // Q is in; from here on only tile copies are in flight

    // copies of tile t into `dst`: copy i covers tile bytes [1024 i, 1024 i + 1024);
    // rows past the end repeat the last kept row (finite data, masked out below)
    auto issue = [&](int t, uint8_t* dst) {
#pragma unroll
        for (int i = w; i < kTileCopies; i += NW) {
            const int q = i * 64 + l;
            const int rr = q / kRowChunks, c = q % kRowChunks;
            const uint32_t row = rows[min(t * kTR + rr, nr - 1)];
            const uint8_t* src = reinterpret_cast<const uint8_t*>(A.kv) + (int64_t)row * kRowB +
                                 ((c ^ (rr & 7)) << 4);
            __builtin_amdgcn_global_load_lds(src, (SIA_LDS void*)(dst + i * 1024), 16, 0, 0);
        }
    };
    // this wave's own copies of the tile after t have landed or not been issued
    auto wait_tile = [&](int t) {
        if (t + 1 < ntiles) {
            if (w < GM::SPLIT) wait_vmcnt<GM::CP_LO + 1>();
            else wait_vmcnt<GM::CP_LO>();
        } else {
            wait_vmcnt<0>();
        }
    };

    const float scale_log2 = A.sm_scale * 1.4426950408889634f;
    // Online softmax with a lazily moved reference max: p = 2^(x - m_ref) where
    // m_ref only moves when a head's running max exceeds it by more than
    // kLazyMax (log2 units), so p <= 2^kLazyMax and O, l are rescaled only then.
    // O / l and the log-sum-exp are unchanged in exact arithmetic.
    constexpr float kLazyMax = 8.f;
    float m_ref[4], l_run[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {
        m_ref[r] = -INFINITY;
        l_run[r] = 0.f;
    }
    f32x4 o[NHB][NCB];
#pragma unroll
    for (int h = 0; h < NHB; h++)
#pragma unroll
        for (int cb = 0; cb < NCB; cb++) o[h][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (tid < 2) rescale[tid] = 0;

    // Per-lane byte offsets inside a tile (chunk 8a + b of row r sits at
    // r*1152 + 128a + ((b ^ (r & 7)) << 4)):
    //  keys: rows jl and 16 + jl, chunks 36 rb + 4 ks + g of this wave's half row
    //  values: rows 8g + jl/4 (and +4), columns w*CPW + 16 cb + 4*(jl%4) .. +3
    int koffL[2][2], voffL[2][4];
#pragma unroll
    for (int c = 0; c < 2; c++) {
        const int kn = c * 16 + jl;
#pragma unroll
        for (int e = 0; e < 2; e++)
            koffL[c][e] = kn * kRowB + (((((rb + e) & 1) << 2 | g) ^ (kn & 7)) << 4) + ((rb * 36) & ~7) * 16;
    }
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

    auto tile = [&](int t, const uint8_t* buf) {
        // The slot's addresses are formed here from opaque copies of the lane
        // offsets, so that they are not kept live per slot across the loop.
        int koff[2][2], voff[2][4];
#pragma unroll
        for (int c = 0; c < 2; c++)
#pragma unroll
            for (int e = 0; e < 2; e++) {
                koff[c][e] = koffL[c][e];
                asm volatile("" : "+v"(koff[c][e]));
            }
#pragma unroll
        for (int e = 0; e < 2; e++)
#pragma unroll
            for (int v = 0; v < 4; v++) {
                voff[e][v] = voffL[e][v];
                asm volatile("" : "+v"(voff[e][v]));
            }

        // ---- partial logits of 16 heads x 32 rows over this wave's half row;
        // the key reads of the next three steps are in flight during the MFMAs
        auto kload = [&](u32x4 (&kb)[2][3], int k0) {
#pragma unroll
            for (int i = 0; i < 3; i++) {
                const int ks = k0 + i;
#pragma unroll
                for (int c = 0; c < 2; c++)
                    kb[c][i] = *reinterpret_cast<const u32x4*>(buf + koff[c][ks & 1] + ((4 * rb + 4 * ks) >> 3) * 128);
            }
        };
        f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        u32x4 kb[2][3];
        kload(kb, 0);
#pragma unroll
        for (int k0 = 0; k0 < kQKHalf; k0 += 3) {
            u32x4 kn[2][3];
            if (k0 + 3 < kQKHalf) kload(kn, k0 + 3);
#pragma unroll
            for (int i = 0; i < 3; i++)
#pragma unroll
                for (int c = 0; c < 2; c++) acc[c] = mfma16(qa[k0 + i], as_bf16x8(kb[c][i]), acc[c]);
            if (k0 + 3 < kQKHalf) {
#pragma unroll
                for (int c = 0; c < 2; c++)
#pragma unroll
                    for (int i = 0; i < 3; i++) kb[c][i] = kn[c][i];
            }
        }
        // the flag of tile t+1 is cleared now: every read of it (tile t-1) is done
        if (tid == 0) rescale[(t + 1) & 1] = 0;
        // the two half-row partials of the head block meet in LDS; both waves then
        // hold the full logits (a + b = b + a bit for bit) and run the same softmax
        sx[w][0][l] = acc[0];
        sx[w][1][l] = acc[1];
        lds_barrier();
        const int pw = w ^ NHB;   // partner wave: same head block, other half
        const f32x4 s0 = acc[0] + sx[pw][0][l];
        const f32x4 s1 = acc[1] + sx[pw][1][l];
        const bool v0 = t * kTR + jl < nr, v1 = t * kTR + 16 + jl < nr;
        const int hh = hb * 16 + 4 * g;   // first of this lane's four heads
        float al[4];
        bool moved = false;
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const float x0 = v0 ? s0[r] * scale_log2 : -INFINITY;
            const float x1 = v1 ? s1[r] * scale_log2 : -INFINITY;
            const float tm = row16_max(__builtin_fmaxf(x0, x1));
            const bool mv = tm > m_ref[r] + kLazyMax;   // also when m_ref is still -inf
            al[r] = mv ? __builtin_amdgcn_exp2f(m_ref[r] - tm) : 1.f;
            m_ref[r] = mv ? tm : m_ref[r];
            moved |= mv;
            const float p0 = __builtin_amdgcn_exp2f(x0 - m_ref[r]), p1 = __builtin_amdgcn_exp2f(x1 - m_ref[r]);
            l_run[r] = l_run[r] * al[r] + (p0 + p1);
            const __bf16 pm = static_cast<__bf16>(rb ? p1 : p0);   // this wave writes P of its row block
            *reinterpret_cast<__bf16*>(pbuf + (hh + r) * kPStride + (rb * 16 + jl) * 2) = pm;
        }
        if (rb == 0 && jl == 0) *reinterpret_cast<f32x4*>(&alpha_s[hh]) = f32x4{al[0], al[1], al[2], al[3]};
        if (moved) rescale[t & 1] = 1;
        lds_barrier();

        // ---- O = alpha * O + P V over this wave's columns
        if (__builtin_amdgcn_readfirstlane(rescale[t & 1])) {
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
            pa[h] = as_bf16x8(*reinterpret_cast<const u32x4*>(pbuf + (h * 16 + jl) * kPStride + g * 16));
#pragma unroll
        for (int c0 = 0; c0 < NCB; c0 += 4) {
            u32x2 va[4], vb2[4];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int cst = ((c0 + q) >> 2) * 128;
                va[q] = ds_read_tr16(buf + voff[0][q] + cst);
                vb2[q] = ds_read_tr16(buf + voff[1][q] + cst);
            }
            lds_wait(va, vb2);
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const bf16x8 vb = as_bf16x8(u32x4{va[q][0], va[q][1], vb2[q][0], vb2[q][1]});
#pragma unroll
                for (int h = 0; h < NHB; h++) o[h][c0 + q] = mfma16(pa[h], vb, o[h][c0 + q]);
            }
        }
    };

    if (ntiles > 0) {
        issue(0, ring0);
        if (ntiles > 1) issue(1, ring1);
        for (int t = 0; t < ntiles; t++) {
            const int u = t % 3;
            wait_tile(t);
            lds_barrier();
            if (t + 2 < ntiles) issue(t + 2, u == 0 ? ring2 : u == 1 ? ring0 : ring1);
            tile(t, u == 0 ? ring0 : u == 1 ? ring1 : ring2);
        }
    }
    wait_vmcnt<0>();

    // ---- finalize: per-head sums, normalize and write
    if (rb == 0) {
        const int hh = hb * 16 + 4 * g;
        float ls[4];
#pragma unroll
        for (int r = 0; r < 4; r++) ls[r] = row16_sum(l_run[r]);
        if (jl == 0) {
            *reinterpret_cast<f32x4*>(&lsum[hh]) = f32x4{ls[0], ls[1], ls[2], ls[3]};
            *reinterpret_cast<f32x4*>(&mfin[hh]) = f32x4{m_ref[0], m_ref[1], m_ref[2], m_ref[3]};
        }
    }
    __syncthreads();
    const bool split = A.n_split > 1;
#pragma unroll
    for (int h = 0; h < NHB; h++) {
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(&lsum[h * 16 + 4 * g]);
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const float lt = l0[r];
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
        const float lt = lsum[tid];
        const float lse = lt > 0.f ? (mfin[tid] + log2f(lt)) * 0.6931471805599453f : -INFINITY;
        if (split)
            A.part_lse[((int64_t)j * A.n_split + sp) * A.heads + head0 + tid] = lse;
        else if (A.lse)
            A.lse[(int64_t)j * A.heads + head0 + tid] = lse;
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

template <int HB>
static hipError_t mla_launch(const AttnArgs& a, hipStream_t st) {
    const int n_hb = a.heads / HB;
    const int64_t pairs = (int64_t)a.num_q * a.n_split;
    const int64_t blocks = (pairs + 7) / 8 * 8 * n_hb;
    hipLaunchKernelGGL(sparse_mla_kernel<HB>, dim3((unsigned)blocks), dim3(MlaGeom<HB>::NT), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_sparse_mla(const AttnArgs& a, hipStream_t st) {
    switch (a.heads_per_block) {
        case 64: return mla_launch<64>(a, st);
        case 32: return mla_launch<32>(a, st);
        case 16: return mla_launch<16>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_mla_combine(const AttnArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)((int64_t)a.num_q * a.heads)), dim3(128), 0,
                       st, a);
    return hipGetLastError();
}

}  // namespace sia
