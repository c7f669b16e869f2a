// Indexer input preparation for gfx950: the projections that produce the
// indexer's query, its head weights and the new tokens' index keys, run as
// three independent chains ("Rapid Adaptation and Inference Optimization",
// section 4.3 "Multi-Stream Parallel Preparation"; "Day0 Inference Adaptation
// and Performance Optimization for New-Architecture LLMs", section 3.2
// "Three-Stream Coordination for Indexer Input Preparation"):
//   chain 1: q = xq Wq^T, then q -> MXFP8 (codes + E8M0 block scales)
//   chain 2: k = LayerNorm(xh Wk^T) * gamma + beta, rounded to bf16, quantized
//            to MXFP8 and written into the paged index cache at each token's
//            position
//   chain 3: w = xh Ww^T (fp32 head weights)
//
// The projections are one GEMM kernel: out[M, N] = x[M, K] W[N, K]^T with bf16
// operands and fp32 accumulation on 32x32x16 bf16 MFMAs. Both operands have K
// contiguous, which is the MFMA operand layout (a lane holds 8 consecutive k
// of one row of x or of W). A workgroup of four waves computes a 64 x 64 tile
// over one slice of K; slices write fp32 partial tiles that a second kernel
// adds in slice order, so the result does not depend on scheduling.
#include "sia_device.h"
#include "sia_kernels.h"

namespace sia {

constexpr int kGemmThreads = 256;

// Partial products of one 64 x 64 output tile over K slice `z`:
// part[z][m][n] = sum over k in the slice of x[m][k] W[n][k].
__global__ __launch_bounds__(kGemmThreads) void proj_gemm_kernel(GemmArgs G) {
    const int w = threadIdx.x / kWave, l = lane_id();
    const int tn = blockIdx.x, tm = blockIdx.y, z = blockIdx.z;
    const int m0 = tm * 64 + (w & 1) * 32, n0 = tn * 64 + (w >> 1) * 32;
    const int k_per = G.k_slice;
    const int k0 = z * k_per, k1 = min(G.K, k0 + k_per);
    // lane l: row m0 + l%32 of x and row n0 + l%32 of W, k = 8 (l/32) .. + 7 of
    // each 16-wide step (rows past M or N read row 0 and are not stored)
    const int r = l & 31, kk = (l >> 5) * 8;
    const bool mok = m0 + r < G.M, nok = n0 + r < G.N;
    const uint16_t* xa = G.x + (int64_t)(mok ? m0 + r : 0) * G.K + kk;
    const uint16_t* wb = G.w + (int64_t)(nok ? n0 + r : 0) * G.K + kk;
    f32x16 acc = {};
    constexpr int U = 4;   // steps loaded ahead
    u32x4 a[U], b[U];
    int k = k0;
#pragma unroll
    for (int u = 0; u < U; u++) {
        const int kc = min(k + 16 * u, k1 - 16);
        a[u] = *reinterpret_cast<const u32x4*>(xa + kc);
        b[u] = *reinterpret_cast<const u32x4*>(wb + kc);
    }
    for (; k < k1; k += 16 * U) {
#pragma unroll
        for (int u = 0; u < U; u++) {
            if (k + 16 * u < k1) acc = mfma32(as_bf16x8(a[u]), as_bf16x8(b[u]), acc);
            const int kn = min(k + 16 * (u + U), k1 - 16);
            a[u] = *reinterpret_cast<const u32x4*>(xa + kn);
            b[u] = *reinterpret_cast<const u32x4*>(wb + kn);
        }
    }
    // 32x32 accumulator layout: lane l holds column n0 + l%32, rows
    // 8 (i/4) + 4 (l/32) + i%4 of the wave's 32 rows for register i
    float* out = G.part + (int64_t)z * G.M * G.N;
    const int n = n0 + r;
    if (n < G.N) {
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const int m = m0 + 8 * (i >> 2) + 4 * (l >> 5) + (i & 3);
            if (m < G.M) out[(int64_t)m * G.N + n] = acc[i];
        }
    }
}

// out = the sum of the slices' partials, in slice order, as bf16 (RNE) or fp32.
__global__ __launch_bounds__(256) void proj_reduce_kernel(const float* part, int splits, int64_t mn,
                                                          uint16_t* out_bf16, float* out_f32) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < mn; i += (int64_t)gridDim.x * 256) {
        float s = part[i];
        for (int z = 1; z < splits; z++) s += part[(int64_t)z * mn + i];
        if (out_bf16) out_bf16[i] = (uint16_t)f32_to_bf16_rne(s);
        if (out_f32) out_f32[i] = s;
    }
}

// One wave per token: the key's slices added in order, LayerNorm over its 128
// values (mean and variance in fp32, a butterfly sum in lane order), times
// gamma plus beta, rounded to bf16 (the stored key value), then quantized to
// MXFP8 like quantize_mxfp8_kernel (four groups of 32) and written into the
// paged index cache at the token's position. Lane l holds elements 2l, 2l+1.
__global__ __launch_bounds__(256) void key_norm_quant_kernel(KeyPrepArgs K) {
    const int w = threadIdx.x / kWave, l = lane_id();
    const int t = blockIdx.x * 4 + w;
    if (t >= K.M) return;   // (whole waves: no barrier below)
    const int64_t mn = (int64_t)K.M * 128;
    float x0 = 0.f, x1 = 0.f;
    for (int z = 0; z < K.splits; z++) {
        x0 += K.part[z * mn + (int64_t)t * 128 + 2 * l];
        x1 += K.part[z * mn + (int64_t)t * 128 + 2 * l + 1];
    }
    float s = x0 + x1;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d);
    const float mean = s * (1.f / 128.f);
    const float d0 = x0 - mean, d1 = x1 - mean;
    float v = d0 * d0 + d1 * d1;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
    const float rstd = 1.f / sqrtf(v * (1.f / 128.f) + K.eps);
    const float y0 = d0 * rstd * K.gamma[2 * l] + K.beta[2 * l];
    const float y1 = d1 * rstd * K.gamma[2 * l + 1] + K.beta[2 * l + 1];
    const uint32_t b0 = f32_to_bf16_rne(y0), b1 = f32_to_bf16_rne(y1);
    if (K.k_out) reinterpret_cast<uint32_t*>(K.k_out)[(int64_t)t * 64 + l] = b0 | (b1 << 16);
    // MXFP8 of the bf16 values: groups of 32 = lanes 16g .. 16g+15
    const float f0 = __uint_as_float(b0 << 16), f1 = __uint_as_float(b1 << 16);
    float m = fmaxf(fabsf(f0), fabsf(f1));
#pragma unroll
    for (int d = 8; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d));
    int e = -127;
    if (m > 0.f) {
        int E;
        const float fr = frexpf(m, &E);
        e = min(max(E - 9 + (fr > 0.875f ? 1 : 0), -127), 127);
    }
    const float inv = ldexpf(1.f, -e);
    const int code = __builtin_amdgcn_cvt_pk_fp8_f32(f0 * inv, f1 * inv, 0, false) & 0xffff;
    // the token's cache row
    const int b = K.q_seq[t], pos = K.q_pos[t];
    bool ok = b >= 0 && b < K.batch && pos >= 0 && pos < K.max_pages * kPage;
    int page = ok ? K.page_table[(int64_t)b * K.max_pages + pos / kPage] : -1;
    ok = ok && page >= 0 && page < K.num_pages;
    if (!ok) {
        if (l == 0) atomicOr(K.status, kBadPage);
        return;
    }
    const int64_t row = (int64_t)page * kPage + pos % kPage;
    reinterpret_cast<uint16_t*>(K.codes + row * 128)[l] = (uint16_t)code;
    if ((l & 15) == 0) K.scales[row * 4 + (l >> 4)] = (uint8_t)(e + 127);
}

hipError_t launch_proj_gemm(const GemmArgs& g, hipStream_t st) {
    const dim3 grid((unsigned)((g.N + 63) / 64), (unsigned)((g.M + 63) / 64),
                    (unsigned)((g.K + g.k_slice - 1) / g.k_slice));
    hipLaunchKernelGGL(proj_gemm_kernel, grid, dim3(kGemmThreads), 0, st, g);
    return hipGetLastError();
}

hipError_t launch_proj_reduce(const float* part, int splits, int64_t mn, uint16_t* out_bf16, float* out_f32,
                              hipStream_t st) {
    if (mn <= 0) return hipSuccess;
    int64_t blocks = (mn + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(proj_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, st, part, splits, mn, out_bf16,
                       out_f32);
    return hipGetLastError();
}

hipError_t launch_key_norm_quant(const KeyPrepArgs& k, hipStream_t st) {
    if (k.M <= 0) return hipSuccess;
    hipLaunchKernelGGL(key_norm_quant_kernel, dim3((unsigned)((k.M + 3) / 4)), dim3(256), 0, st, k);
    return hipGetLastError();
}

}  // namespace sia
