// Device-side helpers shared by the gfx950 kernels: vector types, MFMA
// wrappers, fp8 -> bf16 conversion, the order-preserving score key and
// wave/block scans.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sia {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kPage = 64;
constexpr int kWave = 64;

// Device status bits (mirror of the SIA_DEVSTATUS_* values of the C header).
constexpr uint32_t kBadSeq = 1u, kBadPage = 2u, kRowTooLong = 4u, kBadIndex = 8u;

// D[32x32] += A[32x16] * B[16x32], bf16 in, fp32 accumulate.
// Lane l holds A row l%32, k = 8*(l/32)+i; B column l%32, k = 8*(l/32)+i;
// accumulator register r holds D[8*(r/4) + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Upper 16 bits of two fp32 packed into one dword (x0 in the low half). Exact
// for values that are representable in bf16.
__device__ __forceinline__ uint32_t pack_hi16(float x0, float x1) {
    return (__float_as_uint(x0) >> 16) | (__float_as_uint(x1) & 0xffff0000u);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Eight OCP e4m3fn codes (bytes of lo, then hi) -> eight bf16, two per
// instruction (scale 1.0). Exact: every e4m3fn value, subnormals included, is a
// bf16 value.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    u32x4 r;
    r[0] = __builtin_bit_cast(uint32_t, a);
    r[1] = __builtin_bit_cast(uint32_t, b);
    r[2] = __builtin_bit_cast(uint32_t, c);
    r[3] = __builtin_bit_cast(uint32_t, d);
    return as_bf16x8(r);
}

// Round-to-nearest-even fp32 -> bf16 bits (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Order-preserving key of a score: larger score <=> larger key. -0 and +0 map
// to one key; NaN maps to 1, below every number; 0 marks "no candidate".
__device__ __forceinline__ uint32_t score_key(float f) {
    // (selects only: callers inside software-pipelined loops need it branch-free)
    uint32_t u = __float_as_uint(f);
    u = u == 0x80000000u ? 0u : u;
    const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (u & 0x7fffffffu) > 0x7f800000u ? 1u : k;
}

__device__ __forceinline__ float key_score(uint32_t k) {
    if (k <= 1u) return __uint_as_float(0x7fc00000u);  // never emitted for real keys
    uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

#define SIA_LDS __attribute__((address_space(3)))

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding: vmcnt in bits 3:0
// and 15:14, expcnt in 6:4, lgkmcnt in 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt vmcnt(N) that is also a compiler memory barrier: no memory access
// moves across it. Pairs with dma16, whose copies the compiler does not see.
template <int N>
__device__ __forceinline__ void wait_vmcnt_mem() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Global -> LDS copy of 16 bytes per active lane: lane i's bytes land at
// lds + 16 i (lds must be wave-uniform). Written as inline assembly so that the
// compiler neither counts nor waits for it (its own tracking of such copies
// falls back to draining every copy in flight before unrelated LDS accesses).
// The copy completes in order with the wave's other vector-memory loads: a
// reader of the destination waits with wait_vmcnt_mem<number of loads issued
// after it>.
__device__ __forceinline__ void dma16(const void* src, SIA_LDS void* lds) {
    const uint32_t m = __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)));
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m) : "memory");
}

// The same copy addressed as a wave-uniform base (SGPRs) plus a per-lane byte
// offset, to the LDS byte address `lds` (wave-uniform): no per-copy vector
// address arithmetic.
__device__ __forceinline__ void dma16_s(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
}

// The same copy with the non-temporal hint, for rows that are read once per
// launch (decode scoring streams every index row exactly once): they do not
// displace reused data in the caches, and streaming reads come in faster.
__device__ __forceinline__ void dma16_s_nt(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
}

// 4 bytes per lane from base + voff to lds + 4 * lane (same conventions).
__device__ __forceinline__ void dma4_s(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
}

// Workgroup barrier for LDS traffic only: this wave's LDS operations are
// complete, then all waves meet. Unlike __syncthreads() it does not wait for
// outstanding global -> LDS copies (whose completion is waited for explicitly
// with counted vmcnt waits); the clobber keeps the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Workgroup barrier that waits for nothing: this wave's LDS reads still in
// flight complete behind it (the compiler waits for their results where they
// are used). The caller makes its own writes that others read after the
// barrier complete first (lds_wait_all).
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// This wave's LDS (and scalar memory) operations complete.
__device__ __forceinline__ void lds_wait_all() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// D[16x16] += A[16x32] * B[32x16], bf16 in, fp32 accumulate.
// Lane l holds A row l%16, k = 8*(l/16)+i; B column l%16, k = 8*(l/16)+i;
// accumulator register r holds D[4*(l/16) + r][l%16].
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Orders this wave's LDS accesses (wave-synchronous code paths).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
}

// Inclusive prefix sum over the 64 lanes of a wave, with DPP lane moves (no LDS
// round trips): shifts by 1, 2, 4, 8 within each row of 16 lanes, then the last
// lane of row 0 is added to rows 1 and 3 and the last lane of row 1 to rows 2, 3.
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
    return v;
}

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, kWave));
    return v;
}

// Exclusive prefix sums of two counters over NT threads (NT = 64: one wave, no
// barrier; NT > 64: the whole block, with barriers). `scratch` holds >= 2*NT/64
// ints of LDS private to the caller.
template <int NT>
__device__ __forceinline__ void scan2(int a, int b, int& a_pre, int& b_pre, int& a_tot,
                                      int& b_tot, int* scratch) {
    // pack both counters into one 32-bit word: each is < 65536 here
    int v = a | (b << 16);
    int inc = wave_incl_scan(v);
    if constexpr (NT == kWave) {
        int tot = __shfl(inc, kWave - 1, kWave);
        int exc = inc - v;
        a_pre = exc & 0xffff; b_pre = exc >> 16;
        a_tot = tot & 0xffff; b_tot = tot >> 16;
    } else {
        constexpr int NW = NT / kWave;
        const int w = threadIdx.x / kWave;
        if (lane_id() == kWave - 1) scratch[w] = inc;
        __syncthreads();
        int before = 0, tot = 0;
#pragma unroll
        for (int i = 0; i < NW; i++) {
            int s = scratch[i];
            before += (i < w) ? s : 0;
            tot += s;
        }
        __syncthreads();
        int exc = before + inc - v;
        a_pre = exc & 0xffff; b_pre = exc >> 16;
        a_tot = tot & 0xffff; b_tot = tot >> 16;
    }
}

// Exclusive prefix sum of one counter over NT threads (same conventions as scan2).
template <int NT>
__device__ __forceinline__ void scan1(int v, int& pre, int& tot, int* scratch) {
    const int inc = wave_incl_scan(v);
    if constexpr (NT == kWave) {
        tot = __shfl(inc, kWave - 1, kWave);
        pre = inc - v;
    } else {
        constexpr int NW = NT / kWave;
        const int w = threadIdx.x / kWave;
        if (lane_id() == kWave - 1) scratch[w] = inc;
        __syncthreads();
        int before = 0, t = 0;
#pragma unroll
        for (int i = 0; i < NW; i++) {
            const int x = scratch[i];
            before += (i < w) ? x : 0;
            t += x;
        }
        __syncthreads();
        pre = before + inc - v;
        tot = t;
    }
}

}  // namespace sia
