// Drives the C ABI's host side (argument validation, launch planning,
// workspace layout) under AddressSanitizer and UndefinedBehaviorSanitizer on a
// machine without a GPU: sia_api.hip is built for the host only and the kernel
// launchers are replaced by stubs that count their calls and report a launch
// error, so a call that passes validation returns SIA_ERR_HIP. Built and run
// by tests/test_sanitizers.py.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "sia.h"
#include "sia_kernels.h"

static int launches = 0;
namespace sia {
#define STUB(sig) \
    sig {         \
        launches++; \
        return hipErrorInvalidValue; \
    }
STUB(hipError_t launch_indexer_rows(const IdxArgs&, const RowsArgs&, int, int, int, int, bool, hipStream_t))
STUB(hipError_t launch_keys_from_scores(const KeysFromScoresArgs&, hipStream_t))
STUB(hipError_t launch_topk_rows(const SelectArgs&, hipStream_t))
STUB(hipError_t launch_indexer_stream(const IdxArgs&, const StreamArgs&, int, int, int, int, hipStream_t))
STUB(hipError_t launch_fill_u32(uint32_t*, uint32_t, int64_t, hipStream_t))
STUB(hipError_t launch_quantize_mxfp8(const uint16_t*, int64_t, uint8_t*, uint8_t*, hipStream_t))
STUB(hipError_t launch_proj_gemm(const GemmArgs&, hipStream_t))
STUB(hipError_t launch_proj_reduce(const float*, int, int64_t, uint16_t*, float*, hipStream_t))
STUB(hipError_t launch_key_norm_quant(const KeyPrepArgs&, hipStream_t))
STUB(hipError_t launch_sparse_mla(const AttnArgs&, hipStream_t))
STUB(hipError_t launch_mla_combine(const AttnArgs&, hipStream_t))
int indexer_stream_blocks_per_cu(int, int, int, int) { return 2; }
size_t indexer_stream_smem(int max_visible, int dim, bool fp8) {
    return (size_t)(max_visible + 63) / 64 * 4 + (size_t)dim * (fp8 ? 1 : 2) * 32 * 8 + 4 * 1360;
}
}  // namespace sia

static int fails = 0;
#define EXPECT(x, want)                                                                              \
    do {                                                                                             \
        const long got_ = (long)(x);                                                                 \
        if (got_ != (long)(want)) {                                                                  \
            std::fprintf(stderr, "%s:%d: %s = %ld, expected %ld (%s)\n", __FILE__, __LINE__, #x, got_, \
                         (long)(want), sia_last_error());                                            \
            fails++;                                                                                 \
        }                                                                                            \
    } while (0)

int main() {
    // host memory stands in for device buffers: nothing here is dereferenced
    // unless a launch happens, and the launchers are stubs
    std::vector<uint8_t> buf(1 << 20);
    void* p = buf.data();
    const int32_t* ip = static_cast<const int32_t*>(p);
    alignas(256) static uint8_t ws[1 << 16];
    sia_page_table pt{ip, ip, 2, 4, 64};
    sia_paged_cache kf{p, reinterpret_cast<const float*>(p), 8, 128, SIA_FP8_E4M3FN};
    sia_paged_cache kb{p, nullptr, 8, 64, SIA_BF16};
    sia_paged_cache kmx{p, p, 8, 128, SIA_MXFP8_E4M3};
    sia_queries qs{4, ip, ip, 2, 200};
    const float* w = reinterpret_cast<const float*>(p);
    int32_t* out = static_cast<int32_t*>(p);
    // workspace sizes, including extreme shapes (no overflow, no crash)
    EXPECT(sia_indexer_workspace_size(&pt, &kf, &qs, 64, 2048) > 256, 1);
    sia_queries big{1 << 20, ip, ip, 2, 256};
    sia_page_table pt_big{ip, ip, 1 << 19, 1 << 20, 64};
    EXPECT(sia_indexer_workspace_size(&pt_big, &kf, &big, 64, 8192) > 0, 1);
    EXPECT(sia_indexer_workspace_size(&pt, &kf, &qs, 0, 16), 0);
    EXPECT(sia_mla_workspace_size(&qs, 128, 512, 2048) >= 256, 1);
    EXPECT(sia_mla_workspace_size(&qs, 24, 512, 2048), 0);
    EXPECT(sia_topk_workspace_size(-1, 10, 10), 0);
    // validation failures: nothing is launched
    int before = launches;
    sia_page_table bad_pt{ip, ip, 2, 4, 32};
    EXPECT(sparse_indexer_topk(&bad_pt, &kf, &qs, p, w, 64, 16, out, nullptr, -1, ws, sizeof ws, nullptr),
           SIA_ERR_UNSUPPORTED);
    EXPECT(sparse_indexer_topk(nullptr, &kf, &qs, p, w, 64, 16, out, nullptr, -1, ws, sizeof ws, nullptr),
           SIA_ERR_INVALID_ARG);
    EXPECT(sparse_indexer_topk(&pt, &kf, &qs, p, w, 65, 16, out, nullptr, -1, ws, sizeof ws, nullptr),
           SIA_ERR_UNSUPPORTED);
    EXPECT(sparse_indexer_topk(&pt, &kf, &qs, p, w, 64, 9000, out, nullptr, -1, ws, sizeof ws, nullptr),
           SIA_ERR_UNSUPPORTED);
    EXPECT(sparse_indexer_topk(&pt, &kf, &qs, p, w, 64, 16, out, nullptr, 7, ws, sizeof ws, nullptr),
           SIA_ERR_INVALID_ARG);
    EXPECT(sparse_indexer_topk(&pt, &kf, &qs, p, w, 64, 16, out, nullptr, -1, ws, 8, nullptr), SIA_ERR_WORKSPACE);
    EXPECT(sparse_indexer_topk(&pt, &kmx, &qs, p, w, 64, 16, out, nullptr, -1, ws, sizeof ws, nullptr),
           SIA_ERR_INVALID_ARG);   // an MXFP8 cache with a bf16 query
    EXPECT(sparse_indexer_topk_mxfp8(&pt, &kf, &qs, static_cast<uint8_t*>(p), static_cast<uint8_t*>(p), w, 64, 16,
                                     out, nullptr, -1, ws, sizeof ws, nullptr),
           SIA_ERR_INVALID_ARG);
    sia_paged_cache kmx64{p, p, 8, 64, SIA_MXFP8_E4M3};
    EXPECT(sparse_indexer_scores_mxfp8(&pt, &kmx64, &qs, static_cast<uint8_t*>(p), static_cast<uint8_t*>(p), w, 64,
                                       reinterpret_cast<float*>(p), 256, ws, sizeof ws, nullptr),
           SIA_ERR_UNSUPPORTED);
    sia_paged_cache kv{p, nullptr, 8, 576, SIA_BF16};
    EXPECT(sparse_mla_attention(&pt, &kv, &qs, p, 24, 512, ip, 64, 0.04f, p, nullptr, ws, sizeof ws, nullptr),
           SIA_ERR_UNSUPPORTED);
    EXPECT(sparse_mla_attention(&pt, &kv, &qs, p, 128, 512, ip, 64, NAN, p, nullptr, ws, sizeof ws, nullptr),
           SIA_ERR_INVALID_ARG);
    EXPECT(sparse_mla_attention_noalloc(&pt, &kv, &big, p, 128, 512, ip, 8192, 0.04f, p, nullptr, nullptr),
           SIA_ERR_WORKSPACE);
    EXPECT(sia_quantize_mxfp8(p, 4, 48, static_cast<uint8_t*>(p), static_cast<uint8_t*>(p), nullptr),
           SIA_ERR_UNSUPPORTED);
    sia_indexer_weights W{p, p, w, w, p, 1536, 7168, 64, 128, 1e-6f};
    void* streams[3] = {nullptr, nullptr, nullptr};
    void* events[3] = {nullptr, nullptr, nullptr};
    EXPECT(sia_indexer_prepare(&W, p, p, &pt, &kmx, &qs, static_cast<uint8_t*>(p), static_cast<uint8_t*>(p),
                               const_cast<float*>(w), nullptr, nullptr, ws, sizeof ws, streams, events),
           SIA_ERR_INVALID_ARG);   // events are required
    sia_indexer_weights W_bad = W;
    W_bad.dq = 1000;
    EXPECT(sia_indexer_prepare_workspace_size(&W_bad, 4), 0);
    EXPECT(sia_indexer_prepare_workspace_size(&W, 4) > 256, 1);
    EXPECT(launches, before);
    // valid calls reach the (stubbed) launchers and report the launch error
    std::vector<uint8_t> big_ws(sia_indexer_workspace_size(&pt, &kf, &qs, 64, 16) + 256);
    void* wsa = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(big_ws.data()) + 255) / 256 * 256);
    EXPECT(sparse_indexer_topk(&pt, &kf, &qs, p, w, 64, 16, out, nullptr, -1, wsa, big_ws.size() - 256, nullptr),
           SIA_ERR_HIP);
    EXPECT(sparse_indexer_topk_mxfp8(&pt, &kmx, &qs, static_cast<uint8_t*>(p), static_cast<uint8_t*>(p), w, 64, 16,
                                     out, nullptr, -1, wsa, big_ws.size() - 256, nullptr),
           SIA_ERR_HIP);
    EXPECT(sparse_mla_attention(&pt, &kv, &qs, p, 128, 512, ip, 64, 0.04f, p, nullptr, ws, sizeof ws, nullptr),
           SIA_ERR_HIP);
    EXPECT(launches > before, 1);
    int32_t z[5];
    EXPECT(sia_zigzag_assign(5, z), SIA_OK);
    EXPECT(z[0] * 10 + z[1], 4);
    EXPECT(sia_version() > 0, 1);
    if (fails) return 1;
    std::printf("api driver: all checks passed (%d stub launches)\n", launches);
    return 0;
}
