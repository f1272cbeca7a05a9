// Shared device/host helpers of the HIP library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

#define MOE_CHECK_ARG(cond)                      \
    do {                                         \
        if (!(cond)) return MOE_ERR_INVALID_ARG; \
    } while (0)

#define MOE_LAUNCH_CHECK()                                       \
    do {                                                         \
        if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP; \
    } while (0)

namespace moe {

constexpr int kWave = 64;

// Compute units of the current device, and how many of them a stream may use (its CU mask,
// all of them for an ordinary stream).  Persistent grids are sized by the latter, so a
// kernel on a stream confined to part of the GPU keeps one block per usable CU.
int device_cus();
int stream_cus(hipStream_t stream);

inline int dtype_size(moe_dtype dt) {
    switch (dt) {
        case MOE_F32: return 4;
        case MOE_BF16: return 2;
        case MOE_FP8_E4M3: return 1;
    }
    return 0;
}

// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// pack two fp32 into two bf16 (lo in the low half)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Streaming accesses: data touched once per kernel (gather, scatter, permute, combine, the
// entry step) is loaded and stored with the non-temporal hint, so the caches do not keep it
// for reuse.  On gfx950 this moves large buffers markedly faster than plain accesses when
// each block also works on a contiguous span (a device copy: about 6.3 against 4.9 TB/s).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
template <typename V>
__device__ __forceinline__ V ld_stream(const V* p) {
    if constexpr (sizeof(V) == 16) {
        const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
        V r;
        __builtin_memcpy(&r, &v, 16);
        return r;
    } else if constexpr (sizeof(V) == 8) {
        const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
        V r;
        __builtin_memcpy(&r, &v, 8);
        return r;
    } else {
        return __builtin_nontemporal_load(p);
    }
}
template <typename V>
__device__ __forceinline__ void st_stream(V* p, const V& v) {
    if constexpr (sizeof(V) == 16) {
        u32x4_t t;
        __builtin_memcpy(&t, &v, 16);
        __builtin_nontemporal_store(t, reinterpret_cast<u32x4_t*>(p));
    } else if constexpr (sizeof(V) == 8) {
        u32x2_t t;
        __builtin_memcpy(&t, &v, 8);
        __builtin_nontemporal_store(t, reinterpret_cast<u32x2_t*>(p));
    } else {
        __builtin_nontemporal_store(v, p);
    }
}

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// a launch's x dimension counts its work-items in 32 bits: blocks * threads < 2^32
inline bool grid_fits(int64_t blocks, int64_t threads) {
    return blocks >= 0 && blocks <= static_cast<int64_t>(0xffffffffu) / threads;
}

inline bool aligned(const void* p, uintptr_t a) {
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

}  // namespace moe
