// DP gather / scatter between the replicas' token slices and the global buffer.
//
// SGLang walkthrough "SGLang 源码完全拆解(十七): DP Attention 与专家并行":
//   - section "两种 gather：all_reduce 与 all_gather": zero the global buffer and write each
//     replica's rows at its offset;
//   - section "scatter：把 MoE 的输出还回本副本": cut the global rows back with the same counts.
// On one GPU every replica buffer is local, so both are pure HBM streams.  One launch covers
// up to kBatch replicas.  Each block copies one contiguous chunk of one replica's slot: its
// U 16-byte loads per thread are all in flight before the stores, and both use the streaming
// (non-temporal) hint.  Chunks of 8 KB for the gather and 4 KB for the scatter timed best on
// the prefill shape (16 KB: 158.6 and 158.5 us; 8 KB: 156.1 and 156.3; 4 KB: 157.3 and 148.9).  Blocks are numbered over the replicas'
// chunks back to back; a block finds its replica in the chunk prefix held in the kernel
// arguments (a uniform, scalar walk over at most kBatch entries).  Pad rows of MAX_LEN slots
// are written as zeros in the same pass; row_valid is written alongside.
#include "moe_dev.h"

namespace moe {
namespace {

constexpr int kBatch = 32;
constexpr int kThreads = 256;
constexpr int kUnrollG = 2;  // vectors per thread: gather
constexpr int kUnrollS = 1;  // scatter

struct SliceBatch {
    const void* ptr[kBatch];
    int64_t off[kBatch];              // first global row of the slot
    int64_t slot_rows[kBatch];        // rows of the slot in the global buffer
    int64_t n[kBatch];                // rows of the replica (<= slot_rows)
    int64_t first_chunk[kBatch + 1];  // chunks of the replicas before j; [cnt] = all chunks
    int32_t cnt;
};

// replica of this block: first_chunk[i] <= blockIdx.x < first_chunk[i + 1] (empty replicas
// have equal bounds and are stepped over)
__device__ __forceinline__ int replica_of_block(const SliceBatch& b) {
    const int64_t blk = blockIdx.x;
    int i = 0;
    while (i + 1 < b.cnt && blk >= b.first_chunk[i + 1]) ++i;
    return i;
}

template <typename V>
__global__ __launch_bounds__(kThreads) void gather_kernel(SliceBatch b, int64_t row_units,
                                                          V* __restrict__ dst,
                                                          int32_t* __restrict__ row_valid) {
    constexpr int kUnroll = kUnrollG, kChunk = kThreads * kUnroll;
    const int i = replica_of_block(b);
    const V* __restrict__ src = static_cast<const V*>(b.ptr[i]);
    V* __restrict__ d = dst + b.off[i] * row_units;
    const int64_t total = b.slot_rows[i] * row_units;
    const int64_t ncopy = b.n[i] * row_units;
    const int64_t c = static_cast<int64_t>(blockIdx.x) - b.first_chunk[i];
    const int64_t base = c * kChunk + threadIdx.x;
    V v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t idx = base + u * kThreads;
        v[u] = (idx < ncopy) ? ld_stream(src + idx) : V{};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t idx = base + u * kThreads;
        if (idx < total) st_stream(d + idx, v[u]);
    }
    // row_valid of the slot: chunk c covers rows c*kThreads + m*(chunks*kThreads)
    const int64_t rows = b.slot_rows[i];
    const int64_t rstep = (b.first_chunk[i + 1] - b.first_chunk[i]) * kThreads;
    for (int64_t r = c * kThreads + threadIdx.x; r < rows; r += rstep)
        row_valid[b.off[i] + r] = r < b.n[i] ? 1 : 0;
}

template <typename V>
__global__ __launch_bounds__(kThreads) void scatter_kernel(SliceBatch b, int64_t row_units,
                                                           const V* __restrict__ src) {
    constexpr int kUnroll = kUnrollS, kChunk = kThreads * kUnroll;
    const int i = replica_of_block(b);
    V* __restrict__ d = static_cast<V*>(const_cast<void*>(b.ptr[i]));
    const V* __restrict__ s = src + b.off[i] * row_units;
    const int64_t total = b.n[i] * row_units;
    const int64_t base = (static_cast<int64_t>(blockIdx.x) - b.first_chunk[i]) * kChunk + threadIdx.x;
    V v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t idx = base + u * kThreads;
        if (idx < total) v[u] = ld_stream(s + idx);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t idx = base + u * kThreads;
        if (idx < total) st_stream(d + idx, v[u]);
    }
}

// Widest vector unit that divides the row and every base pointer.
int pick_unit(int64_t row_bytes, const void* const* ptrs, int n, const void* big) {
    for (int u : {16, 8, 4, 2}) {
        if (row_bytes % u) continue;
        if (!aligned(big, u)) continue;
        bool ok = true;
        for (int i = 0; i < n; ++i)
            if (ptrs[i] && !aligned(ptrs[i], u)) ok = false;
        if (ok) return u;
    }
    return 1;
}

template <typename V>
moe_status launch_slices(bool is_gather, const moe_gather_layout_t* L, const void* const* reps,
                         int64_t row_bytes, void* big, int32_t* row_valid, hipStream_t stream) {
    const int64_t row_units = row_bytes / static_cast<int64_t>(sizeof(V));
    const int64_t kChunk = kThreads * (is_gather ? kUnrollG : kUnrollS);  // vectors per block
    // every launch's block count fits the grid (checked before anything is enqueued)
    if (!grid_fits(ceil_div(L->rows * row_units, kChunk) + kBatch, kThreads)) return MOE_ERR_UNSUPPORTED;
    for (int first = 0; first < L->num_replicas; first += kBatch) {
        const int cnt = (L->num_replicas - first) < kBatch ? (L->num_replicas - first) : kBatch;
        SliceBatch b{};
        b.cnt = cnt;
        int64_t chunks = 0;
        for (int j = 0; j < cnt; ++j) {
            const int i = first + j;
            b.ptr[j] = reps[i];
            b.off[j] = L->offsets[i];
            b.slot_rows[j] = L->offsets[i + 1] - L->offsets[i];
            b.n[j] = L->sizes[i];
            b.first_chunk[j] = chunks;
            chunks += ceil_div((is_gather ? b.slot_rows[j] : b.n[j]) * row_units, kChunk);
        }
        b.first_chunk[cnt] = chunks;
        if (chunks == 0) continue;
        const dim3 grid(static_cast<unsigned>(chunks));
        if (is_gather) {
            hipLaunchKernelGGL(gather_kernel<V>, grid, dim3(kThreads), 0, stream, b, row_units,
                               static_cast<V*>(big), row_valid);
        } else {
            hipLaunchKernelGGL(scatter_kernel<V>, grid, dim3(kThreads), 0, stream, b, row_units,
                               static_cast<const V*>(big));
        }
        MOE_LAUNCH_CHECK();
    }
    return MOE_OK;
}

moe_status run_slices(bool is_gather, const moe_gather_layout_t* L, const void* const* reps,
                      int64_t H, moe_dtype dt, void* big, int32_t* row_valid, hipStream_t stream) {
    MOE_CHECK_ARG(L && reps);
    MOE_CHECK_ARG(L->num_replicas >= 1 && L->num_replicas <= MOE_MAX_REPLICAS);
    MOE_CHECK_ARG(L->mode == MOE_PAD_MAX_LEN || L->mode == MOE_PAD_SUM_LEN);
    MOE_CHECK_ARG(H > 0);
    MOE_CHECK_ARG(dt == MOE_F32 || dt == MOE_BF16);
    if (L->rows == 0) return MOE_OK;  // every replica idle: nothing runs
    MOE_CHECK_ARG(big != nullptr);
    MOE_CHECK_ARG(!is_gather || row_valid != nullptr);
    for (int i = 0; i < L->num_replicas; ++i) {
        MOE_CHECK_ARG(L->sizes[i] >= 0);
        MOE_CHECK_ARG(L->offsets[i] >= 0 && L->offsets[i + 1] >= L->offsets[i]);
        MOE_CHECK_ARG(L->sizes[i] <= L->offsets[i + 1] - L->offsets[i]);
        MOE_CHECK_ARG(L->sizes[i] == 0 || reps[i] != nullptr);
    }
    MOE_CHECK_ARG(L->offsets[L->num_replicas] == L->rows);
    const int64_t row_bytes = H * dtype_size(dt);
    switch (pick_unit(row_bytes, reps, L->num_replicas, big)) {
        case 16: return launch_slices<uint4>(is_gather, L, reps, row_bytes, big, row_valid, stream);
        case 8: return launch_slices<uint2>(is_gather, L, reps, row_bytes, big, row_valid, stream);
        case 4: return launch_slices<uint32_t>(is_gather, L, reps, row_bytes, big, row_valid, stream);
        case 2: return launch_slices<uint16_t>(is_gather, L, reps, row_bytes, big, row_valid, stream);
        default: return launch_slices<uint8_t>(is_gather, L, reps, row_bytes, big, row_valid, stream);
    }
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_gather(const moe_gather_layout_t* L, const void* const* replica_x,
                                 int64_t H, moe_dtype dt, void* global_x, int32_t* row_valid,
                                 hipStream_t stream) {
    return moe::run_slices(true, L, replica_x, H, dt, global_x, row_valid, stream);
}

extern "C" moe_status moe_scatter(const moe_gather_layout_t* L, const void* out, int64_t H,
                                  moe_dtype dt, void* const* replica_y, hipStream_t stream) {
    return moe::run_slices(false, L, const_cast<const void* const*>(replica_y), H, dt,
                           const_cast<void*>(out), nullptr, stream);
}
