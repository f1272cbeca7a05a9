// Combine: weighted un-permute of the expert outputs back to global-row order.
//
// vLLM walkthrough "vLLM 源码完全拆解(二十七): Dual Batch Overlap": in the modular-kernel
// block figure the top-k weights are applied by finalize after the un-permute, and the
// combine call of section "第 3 段：combine 前再交一次棒" passes no weights of its own.
// Here both happen in one pass, in gather form:
//     out[g] = scale * sum_{j ascending, pair_row[g*k+j] >= 0} w[g,j] * y_perm[pair_row[g*k+j]]
// One block owns one output row (no atomics, deterministic): each wave learns which of the
// row's k pairs are local from one ballot, then the block streams the row's columns, kUnrollC
// 16-byte vectors per thread, taking the local pairs two at a time in ascending j with both
// source rows' loads in flight before the fp32 FMAs.  Source rows are read and the output row
// written with the streaming (non-temporal) hint.
#include "moe_dev.h"

namespace moe {
namespace {

constexpr int C_THREADS = 256;
constexpr int C_WAVES = C_THREADS / kWave;
constexpr int kUnrollC = 4;  // 16-byte vectors per thread and source row in flight

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

// global row g of the combine, written to the row at dst (the block's 256 threads)
template <typename T>
__device__ __forceinline__ void combine_row(const T* __restrict__ y, const int32_t* __restrict__ pair_row,
                                            const float* __restrict__ w, int64_t g, int k, int64_t H,
                                            float scale, T* __restrict__ dst) {
    using VT = Vec<T>;
    using V = typename VT::V;
    const int lane = lane_id();
    // every wave reads the row's k pairs itself: lane j holds pair j, and the ballot of the
    // local ones is walked lowest lane first, i.e. in ascending j
    int32_t my_row = -1;
    float my_w = 0.f;
    if (lane < k) {
        my_row = pair_row[g * k + lane];
        my_w = w[g * k + lane];
    }
    const uint64_t local = __ballot(my_row >= 0);
    const int64_t vec_per_row = H / VT::N;
    const V* __restrict__ yv = reinterpret_cast<const V*>(y);
    V* __restrict__ ov = reinterpret_cast<V*>(dst);
    for (int64_t c0 = threadIdx.x; c0 < vec_per_row; c0 += C_THREADS * kUnrollC) {
        float acc[kUnrollC][VT::N];
#pragma unroll
        for (int u = 0; u < kUnrollC; ++u)
#pragma unroll
            for (int q = 0; q < VT::N; ++q) acc[u][q] = 0.f;
        uint64_t m = local;
        while (m) {
            // two pairs per step: both source rows' vectors are in flight before the FMAs
            const int j0 = __builtin_ctzll(m);
            m &= m - 1;
            const bool two = m != 0;
            const int j1 = two ? __builtin_ctzll(m) : j0;
            if (two) m &= m - 1;
            const int64_t r0 = __builtin_amdgcn_readlane(my_row, j0);
            const int64_t r1 = __builtin_amdgcn_readlane(my_row, j1);
            const float w0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j0));
            const float w1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j1));
            V v0[kUnrollC], v1[kUnrollC];
#pragma unroll
            for (int u = 0; u < kUnrollC; ++u) {
                const int64_t c = c0 + u * C_THREADS;
                if (c < vec_per_row) {
                    v0[u] = ld_stream(yv + r0 * vec_per_row + c);
                    if (two) v1[u] = ld_stream(yv + r1 * vec_per_row + c);
                }
            }
#pragma unroll
            for (int u = 0; u < kUnrollC; ++u) {
                float f[VT::N];
                VT::unpack(v0[u], f);
#pragma unroll
                for (int q = 0; q < VT::N; ++q) acc[u][q] = __builtin_fmaf(w0, f[q], acc[u][q]);
            }
            if (two) {
#pragma unroll
                for (int u = 0; u < kUnrollC; ++u) {
                    float f[VT::N];
                    VT::unpack(v1[u], f);
#pragma unroll
                    for (int q = 0; q < VT::N; ++q) acc[u][q] = __builtin_fmaf(w1, f[q], acc[u][q]);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kUnrollC; ++u) {
            const int64_t c = c0 + u * C_THREADS;
            if (c >= vec_per_row) continue;
#pragma unroll
            for (int q = 0; q < VT::N; ++q) acc[u][q] *= scale;
            st_stream(ov + c, VT::pack(acc[u]));
        }
    }
}

// Six waves per SIMD (80 registers for bf16, no spill; the compiler's default gives 81 and
// five): more rows in flight per CU.  Prefill combine 0.126 -> 0.124 ms, fused exit 0.135 ->
// 0.129 ms.  Eight waves would spill.
#define MOE_COMBINE_OCCUPANCY __attribute__((amdgpu_waves_per_eu(6)))

template <typename T>
__global__ __launch_bounds__(C_THREADS) MOE_COMBINE_OCCUPANCY void combine_kernel(
    const T* __restrict__ y, const int32_t* __restrict__ pair_row, const float* __restrict__ w,
    int64_t G, int k, int64_t H, float scale, T* __restrict__ out) {
    const int64_t g = blockIdx.x;
    combine_row(y, pair_row, w, g, k, H, scale, out + g * H);
}

// Fused exit: the combine of every real row of up to kExitBatch replicas, written straight to
// the replica's own buffer (the scatter's destination), so the global output buffer is never
// written or read again.  Blocks are numbered over the replicas' real rows back to back; a
// block finds its replica in the row prefix held in the kernel arguments.
constexpr int kExitBatch = 32;
struct ExitBatch {
    void* ptr[kExitBatch];
    int64_t off[kExitBatch];              // first global row of the replica's slot
    int64_t first[kExitBatch + 1];        // real rows of the replicas before j; [cnt] = all
    int32_t cnt;
};

template <typename T>
__global__ __launch_bounds__(C_THREADS) MOE_COMBINE_OCCUPANCY void combine_scatter_kernel(
    const T* __restrict__ y, const int32_t* __restrict__ pair_row, const float* __restrict__ w,
    int k, int64_t H, float scale, ExitBatch b) {
    const int64_t blk = blockIdx.x;
    int i = 0;
    while (i + 1 < b.cnt && blk >= b.first[i + 1]) ++i;
    const int64_t r = blk - b.first[i];
    combine_row(y, pair_row, w, b.off[i] + r, k, H, scale, static_cast<T*>(b.ptr[i]) + r * H);
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
    // vector path: one block per output row; element-wise fallback: one wave per row
    const dim3 grid_rows(static_cast<unsigned>(G));
    const dim3 grid(static_cast<unsigned>(ceil_div(G, C_WAVES)));
    const int vec = dt == MOE_BF16 ? 8 : 4;
    const bool vec_ok = (H % vec == 0) && aligned(out, 16) && (y_perm == nullptr || aligned(y_perm, 16));
    if (!grid_fits(vec_ok ? G : ceil_div(G, C_WAVES), C_THREADS)) return MOE_ERR_UNSUPPORTED;
    if (dt == MOE_BF16) {
        if (vec_ok)
            hipLaunchKernelGGL(combine_kernel<uint16_t>, grid_rows, dim3(C_THREADS), 0, stream,
                               static_cast<const uint16_t*>(y_perm), plan->pair_row, topk_w, G, k,
                               H, routed_scale, static_cast<uint16_t*>(out));
        else
            hipLaunchKernelGGL(combine_scalar_kernel<uint16_t>, grid, dim3(C_THREADS), 0, stream,
                               static_cast<const uint16_t*>(y_perm), plan->pair_row, topk_w, G, k,
                               H, routed_scale, static_cast<uint16_t*>(out));
    } else {
        if (vec_ok)
            hipLaunchKernelGGL(combine_kernel<float>, grid_rows, dim3(C_THREADS), 0, stream,
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

extern "C" moe_status moe_combine_scatter(const void* y_perm, moe_dtype dt, const moe_plan* plan,
                                          const float* topk_w, float routed_scale, int64_t H,
                                          const moe_gather_layout_t* L, void* const* replica_y,
                                          hipStream_t stream) {
    using namespace moe;
    MOE_CHECK_ARG(plan && L && replica_y && H > 0);
    MOE_CHECK_ARG(dt == MOE_F32 || dt == MOE_BF16);
    MOE_CHECK_ARG(plan->G >= 0 && plan->top_k >= 1 && plan->top_k <= 64);
    MOE_CHECK_ARG(L->num_replicas >= 1 && L->num_replicas <= MOE_MAX_REPLICAS);
    MOE_CHECK_ARG(L->rows == plan->G && L->offsets[L->num_replicas] == L->rows);
    const int64_t G = plan->G;
    const int k = plan->top_k;
    const int vec = dt == MOE_BF16 ? 8 : 4;
    int64_t real = 0;
    for (int i = 0; i < L->num_replicas; ++i) {
        MOE_CHECK_ARG(L->sizes[i] >= 0 && L->offsets[i] >= 0 && L->offsets[i + 1] >= L->offsets[i]);
        MOE_CHECK_ARG(L->sizes[i] <= L->offsets[i + 1] - L->offsets[i]);
        if (L->sizes[i] == 0) continue;
        MOE_CHECK_ARG(replica_y[i] != nullptr);
        // the fused form takes whole 16-byte vectors only; other shapes use combine + scatter
        if (!aligned(replica_y[i], 16)) return MOE_ERR_UNSUPPORTED;
        real += L->sizes[i];
    }
    if (G == 0 || real == 0) return MOE_OK;
    MOE_CHECK_ARG(plan->pair_row && topk_w);
    MOE_CHECK_ARG(plan->cap == 0 || y_perm != nullptr);
    if (H % vec != 0 || (y_perm != nullptr && !aligned(y_perm, 16))) return MOE_ERR_UNSUPPORTED;
    if (!grid_fits(real, C_THREADS)) return MOE_ERR_UNSUPPORTED;
    for (int first = 0; first < L->num_replicas; first += kExitBatch) {
        const int cnt = (L->num_replicas - first) < kExitBatch ? (L->num_replicas - first) : kExitBatch;
        ExitBatch b{};
        b.cnt = cnt;
        int64_t rows = 0;
        for (int j = 0; j < cnt; ++j) {
            b.ptr[j] = replica_y[first + j];
            b.off[j] = L->offsets[first + j];
            b.first[j] = rows;
            rows += L->sizes[first + j];
        }
        b.first[cnt] = rows;
        if (rows == 0) continue;
        const dim3 grid(static_cast<unsigned>(rows));
        if (dt == MOE_BF16)
            hipLaunchKernelGGL(combine_scatter_kernel<uint16_t>, grid, dim3(C_THREADS), 0, stream,
                               static_cast<const uint16_t*>(y_perm), plan->pair_row, topk_w, k, H,
                               routed_scale, b);
        else
            hipLaunchKernelGGL(combine_scatter_kernel<float>, grid, dim3(C_THREADS), 0, stream,
                               static_cast<const float*>(y_perm), plan->pair_row, topk_w, k, H,
                               routed_scale, b);
        MOE_LAUNCH_CHECK();
    }
    return MOE_OK;
}
