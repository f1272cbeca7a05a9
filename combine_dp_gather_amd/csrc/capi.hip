// Host-only parts of the C ABI: status text, version, and the gather layout.
#include <atomic>

#include "moe_dev.h"

extern "C" const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported combination";
        case MOE_ERR_CAPACITY: return "caller buffer too small";
        case MOE_ERR_HIP: return "HIP launch failed";
        case MOE_ERR_SCRATCH_LIMIT: return "problem larger than the fixed scratch of a no-allocation entry point";
    }
    return "unknown status";
}

extern "C" const char* moe_version(void) { return "0.1.0 gfx950"; }

// Offsets of the replica slices in the global buffer (SGLang walkthrough "SGLang 源码完全拆解
// (十七)", sections "本 rank 的切片位置怎么算" and "DpPaddingMode"; static bound of the DP note,
// section "跳过同步：用约定代替通信").  Sizes are known on the host before any launch, as the
// DP note requires of every collective's shape.
extern "C" moe_status moe_gather_layout(const int32_t* num_tokens, int32_t W, moe_pad_mode mode,
                                        int32_t is_extend, int32_t max_len_with_idle,
                                        int32_t static_bound, moe_gather_layout_t* out) {
    MOE_CHECK_ARG(num_tokens && out);
    MOE_CHECK_ARG(W >= 1 && W <= MOE_MAX_REPLICAS);
    MOE_CHECK_ARG(mode == MOE_PAD_AUTO || mode == MOE_PAD_MAX_LEN || mode == MOE_PAD_SUM_LEN);
    MOE_CHECK_ARG(static_bound >= 0);
    int64_t n[MOE_MAX_REPLICAS];
    int64_t mx = 0, sm = 0, mn = INT64_MAX;
    for (int i = 0; i < W; ++i) {
        MOE_CHECK_ARG(num_tokens[i] >= 0);
        if (static_bound > 0) MOE_CHECK_ARG(num_tokens[i] <= static_bound);
        n[i] = static_bound > 0 ? static_bound : num_tokens[i];
        mx = n[i] > mx ? n[i] : mx;
        mn = n[i] < mn ? n[i] : mn;
        sm += n[i];
    }
    int32_t m = mode;
    if (m == MOE_PAD_AUTO) {
        if (is_extend && W > 1) {
            m = (max_len_with_idle && mn == 0) ? MOE_PAD_MAX_LEN : MOE_PAD_SUM_LEN;
        } else {
            m = (2 * sm >= mx * W) ? MOE_PAD_MAX_LEN : MOE_PAD_SUM_LEN;
        }
    }
    moe_gather_layout_t L{};
    L.mode = m;
    L.num_replicas = W;
    for (int i = 0; i < W; ++i) L.sizes[i] = static_cast<int32_t>(n[i]);
    if (sm == 0) {
        L.rows = 0;  // all replicas idle: nothing to gather
        for (int i = 0; i <= W; ++i) L.offsets[i] = 0;
    } else if (m == MOE_PAD_SUM_LEN) {
        L.offsets[0] = 0;
        for (int i = 0; i < W; ++i) L.offsets[i + 1] = L.offsets[i] + n[i];
        L.rows = sm;
    } else {
        for (int i = 0; i <= W; ++i) L.offsets[i] = static_cast<int64_t>(i) * mx;
        L.rows = static_cast<int64_t>(W) * mx;
    }
    *out = L;
    return MOE_OK;
}

namespace moe {
int device_cus() {
    static std::atomic<int> cus[64];  // zero-initialised: not yet queried
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 256;
    }
    int v = cus[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) {
            (void)hipGetLastError();
            v = 256;
        }
        cus[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

int stream_cus(hipStream_t stream) {
    const int all = device_cus();
    const uint32_t words = static_cast<uint32_t>((all + 31) / 32);
    uint32_t mask[32] = {};
    if (words > 32 || hipExtStreamGetCUMask(stream, words, mask) != hipSuccess) {
        (void)hipGetLastError();
        return all;
    }
    int n = 0;
    for (uint32_t i = 0; i < words; ++i) n += __builtin_popcount(mask[i]);
    return n > 0 && n < all ? n : all;
}
}  // namespace moe

extern "C" moe_status moe_stream_create_cu_masked(const uint32_t* cu_mask, uint32_t words, hipStream_t* out) {
    MOE_CHECK_ARG(cu_mask && out && words >= 1 && words <= 32);
    int n = 0;
    for (uint32_t i = 0; i < words; ++i) n += __builtin_popcount(cu_mask[i]);
    MOE_CHECK_ARG(n > 0);
    if (hipExtStreamCreateWithCUMask(out, words, cu_mask) != hipSuccess) {
        (void)hipGetLastError();
        return MOE_ERR_HIP;
    }
    return MOE_OK;
}

extern "C" moe_status moe_stream_destroy(hipStream_t stream) {
    MOE_CHECK_ARG(stream != nullptr);
    if (hipStreamDestroy(stream) != hipSuccess) {
        (void)hipGetLastError();
        return MOE_ERR_HIP;
    }
    return MOE_OK;
}
