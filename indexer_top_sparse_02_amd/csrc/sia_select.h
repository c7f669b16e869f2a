// Exact Top-m selection over score keys held in LDS.
//
// The order is (score descending, position ascending); keys come from
// score_key(), so "larger key" is "larger score" and equal keys are equal
// scores. Selection runs in two steps:
//   1. radix threshold: passes of up to 8 bits (four from scratch; callers that
//      know the leading bits refine only the rest), most significant first, find the
//      key T of the m-th element and how many elements with key == T to keep;
//   2. ordered compaction: walk the keys in index order and emit every key > T
//      plus the first `ties` keys == T, so the output is ascending in index and
//      ties go to the lowest indices.
// Keys equal to 0 mark non-candidates; callers pass m <= number of nonzero keys,
// which keeps T >= 1 so that 0 keys are never emitted.
//
// NT = 64: one wave works alone (no block barriers); NT = a larger block size: the whole
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

// hist[digit] += 1 for every active lane (LDS atomics; digits of the coarse
// and refinement passes are spread enough that conflicts stay low). One wave
// (NT = 64): branch-free, an inactive lane adds to its own counter spare[lane]
// instead (64 LDS counters the caller lends, never read), so that the adds of a
// group of keys go out back to back with no exec-mask changes between them.
template <int NT>
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t* spare, uint32_t digit, bool active) {
    if constexpr (NT == kWave) atomicAdd(active ? hist + digit : spare + lane_id(), 1u);
    else if (active) atomicAdd(&hist[digit], 1u);
}

// Keys per thread and round of the histogram passes: four 16-byte groups, read
// before any of the round's adds.
constexpr int kHistGroups = 4;

// Step 1, refinement: the bits above `lowbit` are settled (`prefix` under
// `pmask`) and `rem` elements matching the prefix are still to be taken. Finds
// the remaining low bits in passes of up to 8 bits. keys: LDS, readable in
// groups of four (16-byte aligned; entries past n may hold anything). Returns
// T; `ties` = number of key == T elements to keep. spare: 64 LDS counters for
// the branch-free adds of one wave (NT = 64 only).
template <int NT>
__device__ uint32_t radix_refine(const uint32_t* keys, int n, uint32_t prefix, uint32_t pmask,
                                 int rem, int lowbit, SelScratch* s, int& ties, uint32_t* spare = nullptr) {
    const int tid = sel_tid<NT>();
    while (lowbit > 0) {
        const int width = lowbit < 8 ? lowbit : 8;
        const int shift = lowbit - width;
        const uint32_t dmask = (1u << width) - 1u;
        for (int i = tid; i < 256; i += NT) s->hist[i] = 0;
        sel_sync<NT>();
        for (int i0 = tid * 4; i0 < n; i0 += NT * 4 * kHistGroups) {
            u32x4 kk[kHistGroups];
#pragma unroll
            for (int u = 0; u < kHistGroups; u++) {
                const int i = i0 + u * NT * 4;
                kk[u] = i < n ? *reinterpret_cast<const u32x4*>(keys + i) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < kHistGroups; u++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const uint32_t k = kk[u][e];
                    hist_add<NT>(s->hist, spare, (k >> shift) & dmask,
                                 i0 + u * NT * 4 + e < n && k != 0u && (k & pmask) == prefix);
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
        pmask |= dmask << shift;
        rem -= above;
        lowbit = shift;
        sel_sync<NT>();
    }
    ties = rem;
    return prefix;
}

// Step 1 from scratch: all 32 bits.
template <int NT>
__device__ uint32_t radix_threshold(const uint32_t* keys, int n, int m, SelScratch* s, int& ties,
                                    uint32_t* spare = nullptr) {
    return radix_refine<NT>(keys, n, 0u, 0u, m, 32, s, ties, spare);
}

// One wave, a superset of the Top-m in one histogram pass. The leading bits on
// which the AND and the OR of all nonzero keys agree are shared by every key; one
// histogram of the (up to) 8 bits below them finds the digit b of the m-th largest
// key. Every key whose digit is at least b, i.e. every key >= L = shared bits | b,
// is at least as large as the m-th largest, so keeping them keeps the Top-m (and
// at least m keys). Returns L (0 when all nonzero keys are to be kept) and sets
// `kept` to the number of nonzero keys >= L. keys: LDS, readable in groups of four
// (16-byte aligned, entries past n may hold anything); callers pass 1 <= m <= the
// number of nonzero keys. For an exact threshold from there, `pmask_out` and
// `above` give the settled bits and the number of keys above digit b, and `low`
// the number of bits still open (the arguments radix_refine continues from).
// spare: 64 LDS counters for the branch-free histogram adds.
__device__ uint32_t wave_select_floor(const uint32_t* keys, int n, int m, SelScratch* s, int& kept,
                                     uint32_t& pmask_out, int& above_out, int& low, uint32_t* spare) {
    const int l = lane_id();
    uint32_t a = ~0u, o = 0u;
    for (int i0 = l * 4; i0 < n; i0 += kWave * 4 * kHistGroups) {
        u32x4 kk[kHistGroups];
#pragma unroll
        for (int u = 0; u < kHistGroups; u++) {
            const int i = i0 + u * kWave * 4;
            kk[u] = i < n ? *reinterpret_cast<const u32x4*>(keys + i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kHistGroups; u++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const uint32_t k = kk[u][e];
                if (i0 + u * kWave * 4 + e < n && k != 0u) {
                    a &= k;
                    o |= k;
                }
            }
    }
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1) {
        a &= (uint32_t)__shfl_xor((int)a, d, kWave);
        o |= (uint32_t)__shfl_xor((int)o, d, kWave);
    }
    const uint32_t diff = a ^ o;
    const int lead = diff == 0u ? 32 : __builtin_clz(diff);   // shared leading bits
    const int width = 32 - lead < 8 ? 32 - lead : 8;
    const int shift = 32 - lead - width;
    const uint32_t dmask = (1u << width) - 1u;   // (width 0: every key in digit 0)
    const uint32_t pmask = lead == 0 ? 0u : ~0u << (32 - lead);
    for (int i = l; i < 256; i += kWave) s->hist[i] = 0;
    wave_sync();
    for (int i0 = l * 4; i0 < n; i0 += kWave * 4 * kHistGroups) {
        u32x4 kk[kHistGroups];
#pragma unroll
        for (int u = 0; u < kHistGroups; u++) {
            const int i = i0 + u * kWave * 4;
            kk[u] = i < n ? *reinterpret_cast<const u32x4*>(keys + i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kHistGroups; u++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const uint32_t k = kk[u][e];
                hist_add<kWave>(s->hist, spare, (k >> shift) & dmask, i0 + u * kWave * 4 + e < n && k != 0u);
            }
    }
    wave_sync();
    {
        // lane l owns bins 255-4l .. 252-4l (descending)
        int c[4];
        int tot = 0;
#pragma unroll
        for (int e = 0; e < 4; e++) { c[e] = (int)s->hist[255 - (4 * l + e)]; tot += c[e]; }
        const int inc = wave_incl_scan(tot);
        int above = inc - tot;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            if (above < m && above + c[e] >= m) {
                s->bcast[0] = 255 - (4 * l + e);
                s->bcast[1] = above + c[e];
                s->bcast[2] = above;
            }
            above += c[e];
        }
    }
    wave_sync();
    const uint32_t b = (uint32_t)s->bcast[0];
    kept = s->bcast[1];
    above_out = s->bcast[2];
    wave_sync();
    pmask_out = pmask | (dmask << shift);
    low = shift;
    return (a & pmask) | (b << shift);
}

// Top bits of a key used for the coarse histogram (11 bits: sign, exponent and
// two mantissa bits of the score, i.e. quarter-octave bins).
constexpr int kCoarseBits = 11;
constexpr int kCoarseBins = 1 << kCoarseBits;
__device__ __forceinline__ uint32_t coarse_bin(uint32_t key) { return key >> (32 - kCoarseBits); }

// Floor of the Top-K from a coarse histogram of the keys seen so far: the
// largest bin b with at least K counted keys in bins >= b, or 0 when fewer than
// K keys are counted. A key in a lower bin has K larger keys and can never be
// selected, so it need not be kept; a histogram read while other waves still
// add to it only undercounts, which lowers b and stays valid. One wave.
// hist: kCoarseBins counters in LDS. PACKED: two queries per counter (low and
// high 16 bits; each query's total must stay below 65536, so that sums of the
// packed words never carry across the halves); results in b0 and b1.
template <bool PACKED>
__device__ void coarse_floor(const uint32_t* hist, int K, int& b0, int& b1) {
    static_assert(kCoarseBins == 32 * kWave, "32 bins per lane");
    const int l = lane_id();
    // level 1: lane l sums bins 32 l .. 32 l + 31
    const u32x4* h4 = reinterpret_cast<const u32x4*>(hist + 32 * l);
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const u32x4 v = h4[i];
        s += (v[0] + v[1]) + (v[2] + v[3]);
    }
    const uint32_t pre = (uint32_t)wave_incl_scan((int)s);
    const uint32_t tot = (uint32_t)__shfl((int)pre, kWave - 1, kWave);
    const uint32_t above = tot - pre;   // keys in the bins of higher lanes
    constexpr uint32_t M = PACKED ? 0xffffu : 0xffffffffu;
    int lane_of[2];
#pragma unroll
    for (int h = 0; h < (PACKED ? 2 : 1); h++) {
        const uint32_t a = (above >> (16 * h)) & M, c = (s >> (16 * h)) & M;
        const uint64_t m = __ballot(a < (uint32_t)K && a + c >= (uint32_t)K);
        lane_of[h] = m ? __builtin_ctzll(m) : -1;
    }
    // level 2: lanes 0..31 (query 0) and 32..63 (query 1) take one bin each of
    // the 32 bins of that query's lane
    const int h = PACKED ? (l >> 5) : 0;
    const int L = h ? lane_of[1] : lane_of[0];
    const int i5 = l & 31;
    uint32_t c = 0;
    if (L >= 0) c = (hist[32 * L + i5] >> (16 * h)) & M;
    // keys in the bins above lane L's (read from lane L, this lane's query)
    const uint32_t a_l = ((uint32_t)__shfl((int)above, L >= 0 ? L : 0, kWave) >> (16 * h)) & M;
    if (!PACKED && l >= 32) c = 0;
    const int p2 = wave_incl_scan((int)c);
    const int p31 = __shfl(p2, 31, kWave);
    const int incl = h ? p2 - p31 : p2;
    const int tot2 = h ? __shfl(p2, kWave - 1, kWave) - p31 : p31;
    const uint32_t a2 = a_l + (uint32_t)(tot2 - incl);   // keys above bin 32 L + i5
    const bool hit = L >= 0 && a2 < (uint32_t)K && a2 + c >= (uint32_t)K;
    const uint64_t hm = __ballot(hit);
    const uint32_t m0 = (uint32_t)hm, m1 = (uint32_t)(hm >> 32);
    b0 = m0 ? 32 * lane_of[0] + __builtin_ctz(m0) : 0;
    b1 = PACKED && m1 ? 32 * lane_of[1] + __builtin_ctz(m1) : 0;
}

// From a coarse histogram of the candidate keys (kCoarseBins counters in LDS),
// find the bin that holds the m-th largest key. Returns the bin; `above` = keys
// in higher bins, `total` = all counted keys. Block-wide (NT threads).
template <int NT>
__device__ int coarse_select(const uint32_t* hist, int m, SelScratch* s, int& above, int& total) {
    constexpr int PER = kCoarseBins / NT;   // bins per thread, descending
    const int tid = sel_tid<NT>();
    int c[PER];
    int sum = 0;
#pragma unroll
    for (int e = 0; e < PER; e++) { c[e] = (int)hist[kCoarseBins - 1 - (PER * tid + e)]; sum += c[e]; }
    int pre, tot;
    scan1<NT>(sum, pre, tot, s->scan);
    if (tid == 0) s->bcast[2] = -1;
    sel_sync<NT>();
    int run = pre;
#pragma unroll
    for (int e = 0; e < PER; e++) {
        if (run < m && run + c[e] >= m) {
            s->bcast[2] = kCoarseBins - 1 - (PER * tid + e);
            s->bcast[3] = run;
        }
        run += c[e];
    }
    sel_sync<NT>();
    const int bin = s->bcast[2];
    above = s->bcast[3];
    total = tot;
    sel_sync<NT>();
    return bin;
}

// Step 2. Calls emit(rank, index, e, key) for each kept element, ranks 0..m-1 in
// ascending index. Each thread takes 8 consecutive keys per round. With
// InPlace, emit may overwrite keys/positions at index rank <= index: every read
// of a round (keys here, emit.prefetch) happens before the round's writes.
template <int NT, bool InPlace = false, typename Emit>
__device__ void ordered_compact(const uint32_t* keys, int n, uint32_t T, int ties,
                                SelScratch* s, Emit&& emit) {
    constexpr int EPT = 8;
    const int tid = sel_tid<NT>();
    int run_gt = 0, run_eq = 0;
    for (int base = 0; base < n; base += NT * EPT) {
        const int i = base + tid * EPT;
        u32x4 ka = {0u, 0u, 0u, 0u}, kb = {0u, 0u, 0u, 0u};
        if (i < n) ka = *reinterpret_cast<const u32x4*>(keys + i);
        if (i + 4 < n) kb = *reinterpret_cast<const u32x4*>(keys + i + 4);
#pragma unroll
        for (int e = 0; e < 4; e++) {
            if (i + e >= n) ka[e] = 0u;
            if (i + 4 + e >= n) kb[e] = 0u;
        }
        // index-based reads of the elements that may be kept start before the
        // counts and the scan, so their latency overlaps them
        emit.prefetch(i, ka, T);
        emit.prefetch2(i + 4, kb, T);
        int gt = 0, eq = 0;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            gt += (ka[e] > T) + (kb[e] > T);
            eq += (ka[e] == T) + (kb[e] == T);
        }
        int gpre, epre, gtot, etot;
        scan2<NT>(gt, eq, gpre, epre, gtot, etot, s->scan);
        int eq_before = run_eq + epre;
        int rank = run_gt + gpre + min(eq_before, ties);
        if constexpr (InPlace) sel_sync<NT>();
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const uint32_t k = e < 4 ? ka[e] : kb[e - 4];
            bool take = false;
            if (k > T) take = true;
            else if (k == T) { take = eq_before < ties; eq_before++; }
            if (take) emit(rank++, i + e, e, k);
        }
        if constexpr (InPlace) sel_sync<NT>();
        run_gt += gtot;
        run_eq += etot;
    }
}

// Select the top min(m_cap, nonzero) of keys[0..n) given `hist`, the coarse
// histogram of exactly the nonzero keys, and emit them in index order.
template <int NT, typename Emit>
__device__ int select_emit_coarse(const uint32_t* keys, int n, const uint32_t* hist, int m_cap,
                                  SelScratch* s, Emit&& emit) {
    int above, total;
    const int bin = coarse_select<NT>(hist, m_cap, s, above, total);
    const int m = min(m_cap, total);
    if (m <= 0) return 0;
    if (m == total) {
        ordered_compact<NT>(keys, n, 0u, 0, s, emit);   // every nonzero key
        return m;
    }
    int ties;
    const uint32_t T = radix_refine<NT>(keys, n, (uint32_t)bin << (32 - kCoarseBits),
                                        ~0u << (32 - kCoarseBits), m - above, 32 - kCoarseBits, s, ties);
    ordered_compact<NT>(keys, n, T, ties, s, emit);
    return m;
}

}  // namespace sia
