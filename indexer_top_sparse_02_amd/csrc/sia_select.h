// Exact Top-m selection over score keys held in LDS.
//
// The order is (score descending, position ascending); keys come from
// score_key(), so "larger key" is "larger score" and equal keys are equal
// scores. Selection runs in two steps:
//   1. radix threshold: four 8-bit passes, most significant digit first, find the
//      key T of the m-th element and how many elements with key == T to keep;
//   2. ordered compaction: walk the keys in index order and emit every key > T
//      plus the first `ties` keys == T, so the output is ascending in index and
//      ties go to the lowest indices.
// Keys equal to 0 mark non-candidates; callers pass m <= number of nonzero keys,
// which keeps T >= 1 so that 0 keys are never emitted.
//
// NT = 64: one wave works alone (no block barriers); NT = 256 or 512: the whole
// block cooperates and every thread must call.
#pragma once
#include "sia_device.h"

namespace sia {

template <int NT>
__device__ __forceinline__ void sel_sync() {
    if constexpr (NT == kWave) wave_sync();
    else __syncthreads();
}

// LDS the selection needs besides the keys (per wave for NT = 64).
struct SelScratch {
    uint32_t hist[256];
    int bcast[4];
    int scan[16];
};

template <int NT>
__device__ __forceinline__ int sel_tid() {
    if constexpr (NT == kWave) return lane_id();
    else return threadIdx.x;
}

// Step 1. keys: LDS, readable in groups of four (16-byte aligned; entries past n
// may hold anything). Returns T; `ties` = number of key == T elements to keep.
template <int NT>
__device__ uint32_t radix_threshold(const uint32_t* keys, int n, int m, SelScratch* s,
                                    int& ties) {
    const int tid = sel_tid<NT>();
    uint32_t prefix = 0, pmask = 0;
    int rem = m;
    for (int pass = 0; pass < 4; pass++) {
        const int shift = 24 - 8 * pass;
        for (int i = tid; i < 256; i += NT) s->hist[i] = 0;
        sel_sync<NT>();
        for (int i = tid * 4; i < n; i += NT * 4) {
            u32x4 k4 = *reinterpret_cast<const u32x4*>(keys + i);
#pragma unroll
            for (int e = 0; e < 4; e++) {
                uint32_t k = k4[e];
                if (i + e < n && (k & pmask) == prefix)
                    atomicAdd(&s->hist[(k >> shift) & 255u], 1u);
            }
        }
        sel_sync<NT>();
        if (tid < kWave) {
            // lane l owns bins 255-4l .. 252-4l (descending)
            int c[4];
            int tot = 0;
#pragma unroll
            for (int e = 0; e < 4; e++) { c[e] = (int)s->hist[255 - (4 * tid + e)]; tot += c[e]; }
            int inc = wave_incl_scan(tot);
            int above = inc - tot;   // elements in bins higher than this lane's
#pragma unroll
            for (int e = 0; e < 4; e++) {
                if (above < rem && above + c[e] >= rem) {
                    s->bcast[0] = 255 - (4 * tid + e);
                    s->bcast[1] = above;
                }
                above += c[e];
            }
        }
        sel_sync<NT>();
        const int digit = s->bcast[0];
        const int above = s->bcast[1];
        prefix |= (uint32_t)digit << shift;
        pmask |= 255u << shift;
        rem -= above;
        sel_sync<NT>();
    }
    ties = rem;
    return prefix;
}

// Step 2. Calls emit(rank, index, key) for each kept element, ranks 0..m-1 in
// ascending index. `keys` may be compacted in place by emit (emit may only write
// at index rank <= index, and reads of a round happen before its writes).
template <int NT, typename Emit>
__device__ void ordered_compact(const uint32_t* keys, int n, uint32_t T, int ties,
                                SelScratch* s, Emit&& emit) {
    const int tid = sel_tid<NT>();
    int run_gt = 0, run_eq = 0;
    for (int base = 0; base < n; base += NT * 4) {
        const int i = base + tid * 4;
        u32x4 k4 = {0u, 0u, 0u, 0u};
        if (i < n) k4 = *reinterpret_cast<const u32x4*>(keys + i);
        int gt = 0, eq = 0;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            if (i + e >= n) k4[e] = 0u;
            gt += k4[e] > T;
            eq += k4[e] == T;
        }
        int gpre, epre, gtot, etot;
        scan2<NT>(gt, eq, gpre, epre, gtot, etot, s->scan);
        int eq_before = run_eq + epre;
        int rank = run_gt + gpre + min(eq_before, ties);
        // positions of this round are read (by emit through its own state) before
        // any write of this round: emit is given the key, and index-based reads
        // are done by the caller's prefetch hook below.
        emit.prefetch(i, k4);
        sel_sync<NT>();
#pragma unroll
        for (int e = 0; e < 4; e++) {
            uint32_t k = k4[e];
            bool take = false;
            if (k > T) take = true;
            else if (k == T) { take = eq_before < ties; eq_before++; }
            if (take) emit(rank++, i + e, e, k);
        }
        sel_sync<NT>();
        run_gt += gtot;
        run_eq += etot;
    }
}

// Count of nonzero keys among keys[0..n).
template <int NT>
__device__ int count_nonzero(const uint32_t* keys, int n, SelScratch* s) {
    const int tid = sel_tid<NT>();
    int c = 0;
    for (int i = tid * 4; i < n; i += NT * 4) {
        u32x4 k4 = *reinterpret_cast<const u32x4*>(keys + i);
#pragma unroll
        for (int e = 0; e < 4; e++) c += (i + e < n && k4[e] != 0u);
    }
    c = wave_sum(c);
    if constexpr (NT == kWave) {
        return c;
    } else {
        const int w = threadIdx.x / kWave;
        if (lane_id() == 0) s->scan[w] = c;
        __syncthreads();
        int tot = 0;
        for (int i = 0; i < NT / kWave; i++) tot += s->scan[i];
        __syncthreads();
        return tot;
    }
}

}  // namespace sia
