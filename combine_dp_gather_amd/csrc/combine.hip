// Combine: weighted un-permute of the expert outputs back to global-row order.
//
// vLLM walkthrough "vLLM 源码完全拆解(二十七): Dual Batch Overlap": in the modular-kernel
// block figure the top-k weights are applied by finalize after the un-permute, and the
// combine call of section "第 3 段：combine 前再交一次棒" passes no weights of its own.
// Here both happen in one pass, in gather form:
//     out[g] = scale * sum_{j ascending, pair_row[g*k+j] >= 0} w[g,j] * y_perm[pair_row[g*k+j]]
// One wave owns one output row (no atomics, deterministic).  Lane j < k fetches the pair's
// row index and weight once; the column loop then reads up to 8 source rows per batch with
// all loads issued before the fp32 FMAs, so each lane keeps 8 16-byte loads in flight.
#include "moe_dev.h"

namespace moe {
namespace {

constexpr int C_THREADS = 256;
constexpr int C_WAVES = C_THREADS / kWave;
constexpr int kBatchJ = 8;

template <typename T>
struct Vec;
template <>
struct Vec<uint16_t> {  // 8 bf16 in 16 bytes
    using V = uint4;
    static constexpr int N = 8;
    __device__ static void unpack(const V& v, float (&f)[N]) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f[2 * q] = __uint_as_float(w[q] << 16);
            f[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
        }
    }
    __device__ static V pack(const float (&f)[N]) {
        V v;
        v.x = pack_bf16x2(f[0], f[1]);
        v.y = pack_bf16x2(f[2], f[3]);
        v.z = pack_bf16x2(f[4], f[5]);
        v.w = pack_bf16x2(f[6], f[7]);
        return v;
    }
};
template <>
struct Vec<float> {  // 4 fp32 in 16 bytes
    using V = float4;
    static constexpr int N = 4;
    __device__ static void unpack(const V& v, float (&f)[N]) {
        f[0] = v.x;
        f[1] = v.y;
        f[2] = v.z;
        f[3] = v.w;
    }
    __device__ static V pack(const float (&f)[N]) { return V{f[0], f[1], f[2], f[3]}; }
};

template <typename T>
__global__ __launch_bounds__(C_THREADS) void combine_kernel(
    const T* __restrict__ y, const int32_t* __restrict__ pair_row, const float* __restrict__ w,
    int64_t G, int k, int64_t H, float scale, T* __restrict__ out) {
    using VT = Vec<T>;
    using V = typename VT::V;
    const int lane = lane_id();
    const int64_t g = static_cast<int64_t>(blockIdx.x) * C_WAVES + threadIdx.x / kWave;
    if (g >= G) return;
    int32_t my_row = -1;
    float my_w = 0.f;
    if (lane < k) {
        my_row = pair_row[g * k + lane];
        my_w = w[g * k + lane];
    }
    const int64_t vec_per_row = H / VT::N;
    const V* __restrict__ yv = reinterpret_cast<const V*>(y);
    V* __restrict__ ov = reinterpret_cast<V*>(out) + g * vec_per_row;
    for (int64_t c = lane; c < vec_per_row; c += kWave) {
        float acc[VT::N];
#pragma unroll
        for (int q = 0; q < VT::N; ++q) acc[q] = 0.f;
        for (int j0 = 0; j0 < k; j0 += kBatchJ) {
            V v[kBatchJ];
            float wj[kBatchJ];
            bool use[kBatchJ];
#pragma unroll
            for (int t = 0; t < kBatchJ; ++t) {
                const int j = j0 + t;
                const int32_t r = __shfl(my_row, j < k ? j : 0);
                wj[t] = __shfl(my_w, j < k ? j : 0);
                use[t] = (j < k) && (r >= 0);
                v[t] = use[t] ? yv[static_cast<int64_t>(r) * vec_per_row + c] : V{};
            }
#pragma unroll
            for (int t = 0; t < kBatchJ; ++t) {
                if (!use[t]) continue;
                float f[VT::N];
                VT::unpack(v[t], f);
#pragma unroll
                for (int q = 0; q < VT::N; ++q) acc[q] = __builtin_fmaf(wj[t], f[q], acc[q]);
            }
        }
#pragma unroll
        for (int q = 0; q < VT::N; ++q) acc[q] *= scale;
        ov[c] = VT::pack(acc);
    }
}

// element-wise fallback for H not a multiple of the vector width or unaligned buffers
template <typename T>
__global__ __launch_bounds__(C_THREADS) void combine_scalar_kernel(
    const T* __restrict__ y, const int32_t* __restrict__ pair_row, const float* __restrict__ w,
    int64_t G, int k, int64_t H, float scale, T* __restrict__ out) {
    const int64_t g = static_cast<int64_t>(blockIdx.x) * C_WAVES + threadIdx.x / kWave;
    if (g >= G) return;
    for (int64_t c = lane_id(); c < H; c += kWave) {
        float acc = 0.f;
        for (int j = 0; j < k; ++j) {
            const int32_t r = pair_row[g * k + j];
            if (r < 0) continue;
            float v;
            if constexpr (sizeof(T) == 2) v = bf16_to_f32(y[static_cast<int64_t>(r) * H + c]);
            else v = y[static_cast<int64_t>(r) * H + c];
            acc = __builtin_fmaf(w[g * k + j], v, acc);
        }
        acc *= scale;
        if constexpr (sizeof(T) == 2) out[g * H + c] = f32_to_bf16(acc);
        else out[g * H + c] = acc;
    }
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_combine(const void* y_perm, moe_dtype dt, const moe_plan* plan,
                                  const float* topk_w, float routed_scale, int64_t H, void* out,
                                  hipStream_t stream) {
    using namespace moe;
    MOE_CHECK_ARG(plan && H > 0);
    MOE_CHECK_ARG(dt == MOE_F32 || dt == MOE_BF16);
    MOE_CHECK_ARG(plan->G >= 0 && plan->top_k >= 1 && plan->top_k <= 64);
    const int64_t G = plan->G;
    const int k = plan->top_k;
    if (G == 0) return MOE_OK;
    MOE_CHECK_ARG(plan->pair_row && topk_w && out);
    MOE_CHECK_ARG(plan->cap == 0 || y_perm != nullptr);
    const dim3 grid(static_cast<unsigned>(ceil_div(G, C_WAVES)));
    const int vec = dt == MOE_BF16 ? 8 : 4;
    const bool vec_ok = (H % vec == 0) && aligned(out, 16) && (y_perm == nullptr || aligned(y_perm, 16));
    if (dt == MOE_BF16) {
        if (vec_ok)
            hipLaunchKernelGGL(combine_kernel<uint16_t>, grid, dim3(C_THREADS), 0, stream,
                               static_cast<const uint16_t*>(y_perm), plan->pair_row, topk_w, G, k,
                               H, routed_scale, static_cast<uint16_t*>(out));
        else
            hipLaunchKernelGGL(combine_scalar_kernel<uint16_t>, grid, dim3(C_THREADS), 0, stream,
                               static_cast<const uint16_t*>(y_perm), plan->pair_row, topk_w, G, k,
                               H, routed_scale, static_cast<uint16_t*>(out));
    } else {
        if (vec_ok)
            hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(C_THREADS), 0, stream,
                               static_cast<const float*>(y_perm), plan->pair_row, topk_w, G, k, H,
                               routed_scale, static_cast<float*>(out));
        else
            hipLaunchKernelGGL(combine_scalar_kernel<float>, grid, dim3(C_THREADS), 0, stream,
                               static_cast<const float*>(y_perm), plan->pair_row, topk_w, G, k, H,
                               routed_scale, static_cast<float*>(out));
    }
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}
