// The layer's entry step fused with the DP gather.
//
// SGLang walkthrough "SGLang 源码完全拆解(十七): DP Attention 与专家并行", section "边界判定的融合"
// (under "两层通信怎么省"): with a plain residual add and a plain RMSNorm, one pass updates the
// residual, reads the normalised FFN input from it and gathers that input.  Per row of
// replica i (the attention-TP sum that precedes it on a multi-GPU rank has no counterpart
// here):
//     residual[r] <- round(hidden[r] + residual[r])                    (stored dtype)
//     global_x[offset_i + r] = round(residual[r] * w / sqrt(mean(residual[r]^2) + eps))
// The norm reads the residual as stored.  Pad rows of the global buffer are zero, and
// row_valid marks the real rows, as in the plain gather.
//
// HBM-bound: per real row, 2 rows read and 2 written; the unfused chain (add+norm kernel,
// then gather) reads 3 and writes 3.  One block of 256 threads owns one row at a time: each
// thread loads its 16-byte chunks of both inputs at once (at most kMaxChunks, all in flight),
// keeps the rounded sum in registers across the block's sum of squares (waves, then LDS),
// then writes both outputs, all with the streaming (non-temporal) hint.  Few registers per
// thread keep many blocks resident per CU, and each thread reads its chunks of the norm
// weight once for all its rows.  Rows too wide for
// the register path, or not 16-byte aligned, take a two-pass per-element path (one wave per
// row) that re-reads the residual it has just written.
#include "moe_dev.h"

namespace moe {
namespace {

constexpr int kBatch = 32;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
// 16-byte chunks of a row one thread holds in registers (both inputs in flight at once):
// rows up to 32 KiB
constexpr int kMaxChunks = 8;

struct EntryBatch {
    const void* hid[kBatch];
    void* res[kBatch];
    int64_t off[kBatch];        // first global row of the slot
    int64_t slot_rows[kBatch];  // rows of the slot in the global buffer
    int64_t n[kBatch];          // rows of the replica (<= slot_rows)
};

template <typename T>
struct Elem;
template <>
struct Elem<uint16_t> {
    static constexpr int kPer16 = 8;
    __device__ static float load(uint16_t v) { return bf16_to_f32(v); }
    __device__ static uint16_t round(float f) { return f32_to_bf16(f); }
};
template <>
struct Elem<float> {
    static constexpr int kPer16 = 4;
    __device__ static float load(float v) { return v; }
    __device__ static float round(float f) { return f; }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

// the values of one 16-byte chunk
template <typename T>
union Chunk {
    uint4 u;
    T v[Elem<T>::kPer16];
};

template <typename T, int MAXC>
__global__ __launch_bounds__(kThreads) void entry_kernel(EntryBatch b, int64_t H,
                                                         const T* __restrict__ w, float eps,
                                                         T* __restrict__ gx,
                                                         int32_t* __restrict__ row_valid) {
    constexpr int P = Elem<T>::kPer16;
    __shared__ float part[2][kWaves];
    const int i = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int64_t chunks = H / P;
    const int64_t rows = b.slot_rows[i], n = b.n[i];
    // the input may be the residual buffer itself (each element is read before it is written)
    const uint4* hid = static_cast<const uint4*>(b.hid[i]);
    uint4* res = static_cast<uint4*>(b.res[i]);
    const float inv_h = 1.0f / static_cast<float>(H);
    // this thread's chunks of the norm weight, read from HBM once for all its rows and parked
    // in LDS (registers would hold them converted to fp32 and halve the resident blocks); each
    // thread reads back only the chunks it wrote, so no barrier is needed
    __shared__ uint4 gl[MAXC * kThreads];
#pragma unroll
    for (int u = 0; u < MAXC; ++u) {
        const int64_t c = tid + u * kThreads;
        if (c < chunks) gl[c] = reinterpret_cast<const uint4*>(w)[c];
    }
    int par = 0;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        uint4* __restrict__ out = reinterpret_cast<uint4*>(gx + (b.off[i] + r) * H);
        if (r >= n) {  // pad slot row of MAX_LEN / static layouts
            for (int64_t c = tid; c < chunks; c += kThreads) st_stream(out + c, uint4{0u, 0u, 0u, 0u});
            if (tid == 0) row_valid[b.off[i] + r] = 0;
            continue;
        }
        Chunk<T> s[MAXC], h[MAXC];
#pragma unroll
        for (int u = 0; u < MAXC; ++u) {
            const int64_t c = tid + u * kThreads;
            if (c < chunks) {
                h[u].u = ld_stream(hid + r * chunks + c);
                s[u].u = ld_stream(res + r * chunks + c);
            }
        }
        float sq = 0.f;
#pragma unroll
        for (int u = 0; u < MAXC; ++u) {
            const int64_t c = tid + u * kThreads;
            if (c < chunks) {
#pragma unroll
                for (int e = 0; e < P; ++e) {
                    s[u].v[e] = Elem<T>::round(Elem<T>::load(h[u].v[e]) + Elem<T>::load(s[u].v[e]));
                    const float q = Elem<T>::load(s[u].v[e]);
                    sq = fmaf(q, q, sq);
                }
                st_stream(res + r * chunks + c, s[u].u);
            }
        }
        // row sum of squares: waves, then the block through LDS (two buffers alternate by
        // row, so one barrier per row suffices)
        sq = wave_sum(sq);
        if (lane == 0) part[par][wave] = sq;
        __syncthreads();
        float tot = 0.f;
#pragma unroll
        for (int q = 0; q < kWaves; ++q) tot += part[par][q];
        const float scale = 1.0f / sqrtf(tot * inv_h + eps);
#pragma unroll
        for (int u = 0; u < MAXC; ++u) {
            const int64_t c = tid + u * kThreads;
            if (c < chunks) {
                Chunk<T> y, g;
                g.u = gl[c];
#pragma unroll
                for (int e = 0; e < P; ++e)
                    y.v[e] = Elem<T>::round(Elem<T>::load(s[u].v[e]) * scale * Elem<T>::load(g.v[e]));
                st_stream(out + c, y.u);
            }
        }
        if (tid == 0) row_valid[b.off[i] + r] = 1;
        par ^= 1;  // per barrier, not per row: pad rows take none
    }
}

// any H and alignment: two passes per row, the second re-reading the residual this lane wrote
template <typename T>
__global__ __launch_bounds__(kThreads) void entry_generic_kernel(EntryBatch b, int64_t H,
                                                                 const T* __restrict__ w, float eps,
                                                                 T* __restrict__ gx,
                                                                 int32_t* __restrict__ row_valid) {
    const int i = blockIdx.y;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t rows = b.slot_rows[i], n = b.n[i];
    const T* hid = static_cast<const T*>(b.hid[i]);
    T* res = static_cast<T*>(b.res[i]);
    const float inv_h = 1.0f / static_cast<float>(H);
    for (int64_t r = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6); r < rows;
         r += static_cast<int64_t>(gridDim.x) * kWaves) {
        T* __restrict__ out = gx + (b.off[i] + r) * H;
        if (r >= n) {
            for (int64_t c = lane; c < H; c += kWave) out[c] = T{};
            if (lane == 0) row_valid[b.off[i] + r] = 0;
            continue;
        }
        float sq = 0.f;
        for (int64_t c = lane; c < H; c += kWave) {
            const T v = Elem<T>::round(Elem<T>::load(hid[r * H + c]) + Elem<T>::load(res[r * H + c]));
            res[r * H + c] = v;
            const float q = Elem<T>::load(v);
            sq = fmaf(q, q, sq);
        }
        sq = wave_sum(sq);
        const float scale = 1.0f / sqrtf(sq * inv_h + eps);
        for (int64_t c = lane; c < H; c += kWave)
            out[c] = Elem<T>::round(Elem<T>::load(res[r * H + c]) * scale * Elem<T>::load(w[c]));
        if (lane == 0) row_valid[b.off[i] + r] = 1;
    }
}

template <typename T>
moe_status launch_entry(const moe_gather_layout_t* L, const void* const* hid, void* const* res,
                        const void* w, float eps, int64_t H, void* gx, int32_t* row_valid,
                        bool vec, hipStream_t stream) {
    constexpr int P = Elem<T>::kPer16;
    const int64_t per_thread = ceil_div(H / P, kThreads);
    for (int first = 0; first < L->num_replicas; first += kBatch) {
        const int cnt = (L->num_replicas - first) < kBatch ? (L->num_replicas - first) : kBatch;
        EntryBatch b{};
        int64_t max_rows = 0;
        for (int j = 0; j < cnt; ++j) {
            const int i = first + j;
            b.hid[j] = hid[i];
            b.res[j] = res[i];
            b.off[j] = L->offsets[i];
            b.slot_rows[j] = L->offsets[i + 1] - L->offsets[i];
            b.n[j] = L->sizes[i];
            if (b.slot_rows[j] > max_rows) max_rows = b.slot_rows[j];
        }
        if (max_rows == 0) continue;
        // up to 32768 blocks per launch: at the prefill shape (8 x 4096 rows) every block takes
        // one row.  8192 blocks of four rows each took 0.339 ms there, 32768 blocks 0.317 ms.
        const int64_t cap_x = (32768 / cnt) > 1 ? (32768 / cnt) : 1;
        const T* wt = static_cast<const T*>(w);
        T* out = static_cast<T*>(gx);
        if (!vec) {
            // one wave per row
            int64_t gxb = ceil_div(max_rows, kWaves);
            const dim3 grid(static_cast<unsigned>(gxb < cap_x ? gxb : cap_x), static_cast<unsigned>(cnt));
            hipLaunchKernelGGL(entry_generic_kernel<T>, grid, dim3(kThreads), 0, stream, b, H, wt, eps, out, row_valid);
        } else {
            // one block per row
            const dim3 grid(static_cast<unsigned>(max_rows < cap_x ? max_rows : cap_x), static_cast<unsigned>(cnt));
            if (per_thread <= 1)
                hipLaunchKernelGGL((entry_kernel<T, 1>), grid, dim3(kThreads), 0, stream, b, H, wt, eps, out, row_valid);
            else if (per_thread <= 2)
                hipLaunchKernelGGL((entry_kernel<T, 2>), grid, dim3(kThreads), 0, stream, b, H, wt, eps, out, row_valid);
            else if (per_thread <= 4)
                hipLaunchKernelGGL((entry_kernel<T, 4>), grid, dim3(kThreads), 0, stream, b, H, wt, eps, out, row_valid);
            else
                hipLaunchKernelGGL((entry_kernel<T, 8>), grid, dim3(kThreads), 0, stream, b, H, wt, eps, out, row_valid);
        }
        MOE_LAUNCH_CHECK();
    }
    return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_entry_gather(const moe_gather_layout_t* L, const void* const* replica_h,
                                       void* const* replica_residual, const void* norm_weight,
                                       float eps, int64_t H, moe_dtype dt, void* global_x,
                                       int32_t* row_valid, hipStream_t stream) {
    using namespace moe;
    MOE_CHECK_ARG(L && replica_h && replica_residual);
    MOE_CHECK_ARG(L->num_replicas >= 1 && L->num_replicas <= MOE_MAX_REPLICAS);
    MOE_CHECK_ARG(L->mode == MOE_PAD_MAX_LEN || L->mode == MOE_PAD_SUM_LEN);
    MOE_CHECK_ARG(H > 0);
    MOE_CHECK_ARG(dt == MOE_F32 || dt == MOE_BF16);
    MOE_CHECK_ARG(eps >= 0.0f && eps < 1e30f);  // also rejects NaN
    if (L->rows == 0) return MOE_OK;            // every replica idle: nothing runs
    MOE_CHECK_ARG(global_x && row_valid && norm_weight);
    for (int i = 0; i < L->num_replicas; ++i) {
        MOE_CHECK_ARG(L->sizes[i] >= 0);
        MOE_CHECK_ARG(L->offsets[i] >= 0 && L->offsets[i + 1] >= L->offsets[i]);
        MOE_CHECK_ARG(L->sizes[i] <= L->offsets[i + 1] - L->offsets[i]);
        MOE_CHECK_ARG(L->sizes[i] == 0 || (replica_h[i] != nullptr && replica_residual[i] != nullptr));
    }
    MOE_CHECK_ARG(L->offsets[L->num_replicas] == L->rows);
    const int es = dtype_size(dt);
    bool vec = (H * es) % 16 == 0 && aligned(global_x, 16) && aligned(norm_weight, 16) &&
               ceil_div(H * es / 16, kThreads) <= kMaxChunks;
    for (int i = 0; i < L->num_replicas && vec; ++i)
        if (L->sizes[i] > 0 && !(aligned(replica_h[i], 16) && aligned(replica_residual[i], 16))) vec = false;
    if (dt == MOE_BF16)
        return launch_entry<uint16_t>(L, replica_h, replica_residual, norm_weight, eps, H, global_x,
                                      row_valid, vec, stream);
    return launch_entry<float>(L, replica_h, replica_residual, norm_weight, eps, H, global_x, row_valid,
                               vec, stream);
}
