// Sparse MLA attention for gfx950: softmax attention of each query over only
// its Top-K rows of the paged latent KV cache ("Rapid Adaptation and Inference
// Optimization", section 4.2 "Sparse Attention Computation": read the selected
// positions straight from the paged main cache, no contiguous copy).
//
// A row c_s is 576 bf16 wide: keys use all 576 columns, values the first 512
// (the latent part shared by K and V in MLA).
//
// Workgroup = (query, block of heads, slice of the selected rows); 4 waves.
// Per tile of 32 selected rows:
//   gather   each thread owns one row (page table lookup once) and 9 of its
//            16-byte column chunks; chunks land in LDS row-major (keys) and the
//            first 512 columns also transposed (values, row index contiguous).
//   Q K^T    the 576 columns are split over the 4 waves (144 each); a wave keeps
//            its slice of Q in registers and runs 32x32x16 MFMAs against the
//            row-major tile; the four partial logits go through LDS.
//   softmax  online: running max and sum per head, rescale factor alpha.
//   P V      wave w owns output columns [128w, 128w+128) for all heads of the
//            block: P (bf16) and the transposed values come from LDS.
// Slices of one query are merged afterwards by log-sum-exp.
#include "sia_device.h"
#include "sia_kernels.h"

namespace sia {

constexpr int kDK = 576, kDV = 512;
constexpr int kTR = 32;                       // rows per tile
constexpr int kKRowStride = kDK * 2 + 16;     // bytes per row in LDS (padded)
constexpr int kVTStride = kTR * 2 + 16;       // bytes per value column in LDS (padded)
constexpr int kPStride = kTR * 2 + 16;        // bytes per head of P in LDS
constexpr int kKSplit = kDK / 4;              // columns per wave for Q K^T (144)
constexpr int kQKSteps = kKSplit / 16;        // 9
constexpr int kChunks = kDK * 2 / 16;         // 72 chunks of 16 bytes per row
constexpr int kChunksPerThread = kTR * kChunks / 256;   // 9

template <int HB>
struct AttnSmem {
    uint8_t krow[kTR * kKRowStride];
    uint8_t vt[kDV * kVTStride];
    float spart[4][HB][kTR];
    uint8_t p[HB * kPStride];
    float alpha[HB];
    float mrun[HB];
    float lrun[HB];
    int valid[kTR];
};

template <int HB>
__global__ __launch_bounds__(256) void sparse_mla_kernel(AttnArgs A) {
    constexpr int MB = (HB + 31) / 32;          // 32-row MFMA blocks of heads
    extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
    AttnSmem<HB>& S = *reinterpret_cast<AttnSmem<HB>*>(smem_raw);

    const int tid = threadIdx.x, w = tid / kWave, l = lane_id(), half = l >> 5, m32 = l & 31;
    const int n_hb = A.heads / HB;

    // XCD-aware block order: the head blocks of one (query, slice) pair get block
    // ids 8 apart, which the dispatcher places on the same XCD (shared L2).
    const int bid = blockIdx.x;
    const int xcd = bid & 7, slot = bid >> 3;
    const int num_pairs = A.num_q * A.n_split;
    const int P = (slot / n_hb) * 8 + xcd;
    const int hb = slot % n_hb;
    if (P >= num_pairs) return;
    const int pair = num_pairs - 1 - P;        // later (longer) queries first
    const int j = pair / A.n_split, sp = pair % A.n_split;
    const int head0 = hb * HB;

    int b = A.q_seq[j];
    bool seq_ok = b >= 0 && b < A.batch;
    if (!seq_ok) {
        if (tid == 0) atomicOr(A.status, kBadSeq);
        b = 0;
    }
    const int n_b = seq_ok ? A.seq_lens[b] : 0;
    const int r0 = sp * A.rows_per_split;
    const int r1 = seq_ok ? min(A.topk, r0 + A.rows_per_split) : r0;
    const int ntiles = r1 > r0 ? (r1 - r0 + kTR - 1) / kTR : 0;

    // ---- Q slice in registers: heads head0 + mb*32 + m32, columns of wave w
    bf16x8 qa[MB][kQKSteps];
#pragma unroll
    for (int mb = 0; mb < MB; mb++) {
        const int hl = mb * 32 + m32;
#pragma unroll
        for (int ks = 0; ks < kQKSteps; ks++) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (hl < HB)
                v = *reinterpret_cast<const u32x4*>(
                    A.q + ((int64_t)j * A.heads + head0 + hl) * kDK + w * kKSplit + ks * 16 + half * 8);
            qa[mb][ks] = as_bf16x8(v);
        }
    }

    const float scale_log2 = A.sm_scale * 1.4426950408889634f;
    // softmax ownership: lanes of wave w handle heads w*HPW .. w*HPW+HPW-1
    constexpr int HPW = HB / 4, LPH = kWave / HPW, RPL = kTR / LPH;
    const int sh = w * HPW + l / LPH;          // head (within block) of this lane
    const int sr0 = (l % LPH) * RPL;           // first row of this lane
    float m_run = -INFINITY, l_run = 0.f;

    f32x16 o[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; mb++)
#pragma unroll
        for (int nb = 0; nb < 4; nb++) o[mb][nb] = f32x16{};

    // ---- gather prefetch: thread owns row (tid % 32), chunks tid/32 + 8i
    const int grow = tid & 31, gc0 = tid >> 5;
    u32x4 pre[kChunksPerThread];
    int pre_valid = 0;
    auto fetch = [&](int t) {
        const int ri = r0 + t * kTR + grow;
        int64_t off = -1;
        if (ri < r1) {
            const int s = A.idx[(int64_t)j * A.topk + ri];
            if (s >= 0) {
                if (s >= n_b || s >= A.max_pages * kPage) {
                    if (gc0 == 0) atomicOr(A.status, kBadIndex);
                } else {
                    const int page = A.page_table[(int64_t)b * A.max_pages + (s >> 6)];
                    if (page >= 0 && page < A.num_pages)
                        off = ((int64_t)page * kPage + (s & 63)) * (kDK * 2);
                    else if (gc0 == 0)
                        atomicOr(A.status, kBadPage);
                }
            }
        }
        pre_valid = off >= 0;
#pragma unroll
        for (int i = 0; i < kChunksPerThread; i++) {
            pre[i] = u32x4{0u, 0u, 0u, 0u};
            if (off >= 0)
                pre[i] = *reinterpret_cast<const u32x4*>(
                    reinterpret_cast<const uint8_t*>(A.kv) + off + (gc0 + 8 * i) * 16);
        }
    };

    if (ntiles > 0) fetch(0);
    for (int t = 0; t < ntiles; t++) {
        // ---- stage the prefetched tile into LDS
#pragma unroll
        for (int i = 0; i < kChunksPerThread; i++) {
            const int c = gc0 + 8 * i;
            *reinterpret_cast<u32x4*>(S.krow + grow * kKRowStride + c * 16) = pre[i];
            if (c < kDV / 8) {
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const uint32_t d = pre[i][e];
                    *reinterpret_cast<uint16_t*>(S.vt + (c * 8 + 2 * e) * kVTStride + grow * 2) =
                        (uint16_t)(d & 0xffffu);
                    *reinterpret_cast<uint16_t*>(S.vt + (c * 8 + 2 * e + 1) * kVTStride + grow * 2) =
                        (uint16_t)(d >> 16);
                }
            }
        }
        if (gc0 == 0) S.valid[grow] = pre_valid;
        __syncthreads();
        if (t + 1 < ntiles) fetch(t + 1);

        // ---- partial logits over this wave's 144 columns
        f32x16 acc[MB];
#pragma unroll
        for (int mb = 0; mb < MB; mb++) acc[mb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < kQKSteps; ks++) {
            const u32x4 kb = *reinterpret_cast<const u32x4*>(
                S.krow + m32 * kKRowStride + (w * kKSplit + ks * 16 + half * 8) * 2);
#pragma unroll
            for (int mb = 0; mb < MB; mb++) acc[mb] = mfma32(qa[mb][ks], as_bf16x8(kb), acc[mb]);
        }
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int hl = mb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                if (hl < HB) S.spart[w][hl][m32] = acc[mb][r];
            }
        __syncthreads();

        // ---- online softmax for this lane's head and rows
        {
            float x[RPL];
            float tmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < RPL; i++) {
                const int rr = sr0 + i;
                float s = S.spart[0][sh][rr] + S.spart[1][sh][rr] + S.spart[2][sh][rr] + S.spart[3][sh][rr];
                x[i] = S.valid[rr] ? s * scale_log2 : -INFINITY;
                tmax = fmaxf(tmax, x[i]);
            }
#pragma unroll
            for (int d = 1; d < LPH; d <<= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, d, kWave));
            const float m_new = fmaxf(m_run, tmax);
            float alpha = 1.f, psum = 0.f;
            uint32_t pb[4] = {0u, 0u, 0u, 0u};
            if (m_new != -INFINITY) {
                alpha = exp2f(m_run - m_new);
#pragma unroll
                for (int i = 0; i < RPL; i++) {
                    const float pv = exp2f(x[i] - m_new);
                    psum += pv;
                    const uint32_t bits = f32_to_bf16_rne(pv);
                    pb[i >> 1] |= (i & 1) ? (bits << 16) : bits;
                }
            }
#pragma unroll
            for (int d = 1; d < LPH; d <<= 1) psum += __shfl_xor(psum, d, kWave);
            l_run = l_run * alpha + psum;
            m_run = m_new;
            uint8_t* pdst = S.p + sh * kPStride + sr0 * 2;
            if constexpr (RPL == 8) *reinterpret_cast<u32x4*>(pdst) = u32x4{pb[0], pb[1], pb[2], pb[3]};
            else if constexpr (RPL == 4) *reinterpret_cast<u32x2*>(pdst) = u32x2{pb[0], pb[1]};
            else *reinterpret_cast<uint32_t*>(pdst) = pb[0];
            if (l % LPH == 0) S.alpha[sh] = alpha;
        }
        __syncthreads();

        // ---- O = alpha * O + P V over this wave's 128 output columns
#pragma unroll
        for (int mb = 0; mb < MB; mb++) {
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int hl = mb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                const float a = hl < HB ? S.alpha[hl] : 1.f;
#pragma unroll
                for (int nb = 0; nb < 4; nb++) o[mb][nb][r] *= a;
            }
        }
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {
            bf16x8 pa[MB];
#pragma unroll
            for (int mb = 0; mb < MB; mb++) {
                const int hl = mb * 32 + m32;
                u32x4 v = {0u, 0u, 0u, 0u};
                if (hl < HB) v = *reinterpret_cast<const u32x4*>(S.p + hl * kPStride + (ks * 16 + half * 8) * 2);
                pa[mb] = as_bf16x8(v);
            }
#pragma unroll
            for (int nb = 0; nb < 4; nb++) {
                const int col = w * 128 + nb * 32 + m32;
                const u32x4 vb = *reinterpret_cast<const u32x4*>(S.vt + col * kVTStride + (ks * 16 + half * 8) * 2);
#pragma unroll
                for (int mb = 0; mb < MB; mb++) o[mb][nb] = mfma32(pa[mb], as_bf16x8(vb), o[mb][nb]);
            }
        }
        __syncthreads();
    }

    // ---- finalize: normalize and write
    if (l % LPH == 0) {
        S.mrun[sh] = m_run;
        S.lrun[sh] = l_run;
    }
    __syncthreads();
    const bool split = A.n_split > 1;
#pragma unroll
    for (int mb = 0; mb < MB; mb++) {
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int hl = mb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            if (hl >= HB) continue;
            const float lsum = S.lrun[hl];
            const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
            const int64_t head = head0 + hl;
#pragma unroll
            for (int nb = 0; nb < 4; nb++) {
                const int col = w * 128 + nb * 32 + m32;
                const float v = o[mb][nb][r] * inv;
                if (split)
                    A.part_o[(((int64_t)j * A.n_split + sp) * A.heads + head) * kDV + col] = v;
                else
                    A.out[((int64_t)j * A.heads + head) * kDV + col] = (uint16_t)f32_to_bf16_rne(v);
            }
        }
    }
    if (tid < HB) {
        const float lsum = S.lrun[tid];
        const float lse = lsum > 0.f ? (S.mrun[tid] + log2f(lsum)) * 0.6931471805599453f : -INFINITY;
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
    auto k = sparse_mla_kernel<HB>;
    const size_t smem = sizeof(AttnSmem<HB>);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    const int n_hb = a.heads / a.heads_per_block;
    const int64_t pairs = (int64_t)a.num_q * a.n_split;
    const int64_t blocks = (pairs + 7) / 8 * 8 * n_hb;
    hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(256), smem, st, a);
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
