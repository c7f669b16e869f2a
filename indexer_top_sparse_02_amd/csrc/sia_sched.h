// Work order of causal prefill tiles. Tile i holds queries of increasing
// position, so its cost grows with i ("light at the beginning, heavy at the
// end" on the page "Day 0 Inference Adaptation and Performance Optimization for
// Hybrid Sparse Attention LLMs", section "Understanding the New Architecture").
// Compiled for host and device so that the host-side query (sia_zigzag_assign)
// and the kernels share one definition.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sia {

// Zigzag pairing ("Day0 ... for a New Hybrid-Attention LLM Architecture",
// section 4.3): of S shards, worker i takes shard i and shard S-1-i. Returns the
// k-th (k = 0 or 1) shard of worker i, or -1 if that worker has no such shard
// (odd S: the middle shard sits alone on the last worker).
__host__ __device__ inline int32_t zigzag_shard(int32_t num_shards, int32_t worker, int32_t k) {
    const int32_t workers = (num_shards + 1) / 2;
    if (worker < 0 || worker >= workers || k < 0 || k > 1) return -1;
    const int32_t a = worker, b = num_shards - 1 - worker;
    if (k == 0) return a;
    return b > a ? b : -1;
}

__host__ __device__ inline int32_t zigzag_workers(int32_t num_shards) {
    return (num_shards + 1) / 2;
}

// Heaviest-first order for a work queue: the n-th tile handed out.
__host__ __device__ inline int32_t heavy_first_tile(int32_t num_tiles, int32_t n) {
    return num_tiles - 1 - n;
}

}  // namespace sia
