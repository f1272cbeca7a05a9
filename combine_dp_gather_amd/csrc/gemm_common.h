// Pieces shared by the bf16 and fp8 grouped GEMMs: buffer descriptors, the device-side tile
// numbering over ragged segments, the XCD-grouped tile order, and the launch plumbing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_dev.h"

namespace moe {
namespace gemm {

constexpr int kMaxSlots = 1024;
constexpr int kThreads = 256;  // 4 waves

typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)

// Raw buffer descriptor over [base, base+bytes): loads past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(bytes), kBufferFlags);
}

// Same, with the base and size declared wave-uniform so the descriptor sits in scalar
// registers (the values are uniform by construction).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_uniform(const void* base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32));
    const void* p = reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
    return make_rsrc(p, __builtin_amdgcn_readfirstlane(bytes));
}

// Tiles are numbered (m-tile over all slots) x (column tile).  With one block per CU the
// hardware hands workgroup b to XCD b % 8, so block b takes, in round r, tile q = b / 8 of
// super-tile r*8 + b%8: the blocks of one XCD work on one SM x SN patch of tiles at a time
// and share its A rows and B columns through that XCD's L2.
struct TileOrder {
    int32_t SM, SN;  // super-tile = SM m-tiles x SN column tiles, SM*SN = blocks per XCD
};

// Slot e owns ceil(c / BM) m-tiles, c = min(counts[e], cap - seg[e]), if lo < c <= hi and none
// otherwise (two kernels can split the slots by size); tile_prefix[e] = m-tiles before slot e,
// tile_prefix[El] = total.  Called by all NTHR threads of the block (part holds NTHR ints);
// ends synced.
template <int BM, int NTHR = kThreads>
__device__ __forceinline__ int32_t number_tiles(const int32_t* counts, const int64_t* seg,
                                                int64_t cap, int El, int32_t* tile_prefix,
                                                int32_t* part, int64_t lo = 0,
                                                int64_t hi = INT64_MAX) {
    static_assert(kMaxSlots % NTHR == 0, "whole slots per thread");
    const int tid = threadIdx.x;
    int32_t loc[kMaxSlots / NTHR];
    int32_t s = 0;
#pragma unroll
    for (int q = 0; q < kMaxSlots / NTHR; ++q) {
        const int e = tid * (kMaxSlots / NTHR) + q;
        int32_t mt = 0;
        if (e < El) {
            int64_t c = counts[e];
            const int64_t room = cap - seg[e];
            c = c < room ? c : (room > 0 ? room : 0);
            if (c > lo && c <= hi) mt = static_cast<int32_t>((c + BM - 1) / BM);
        }
        loc[q] = mt;
        s += mt;
    }
    part[tid] = s;
    __syncthreads();
    for (int off = 1; off < NTHR; off <<= 1) {
        const int32_t v = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int32_t run = part[tid] - s;
#pragma unroll
    for (int q = 0; q < kMaxSlots / NTHR; ++q) {
        const int e = tid * (kMaxSlots / NTHR) + q;
        if (e < El) tile_prefix[e] = run;
        run += loc[q];
    }
    if (tid == NTHR - 1) tile_prefix[El] = part[tid];
    __syncthreads();
    return tile_prefix[El];
}

// Slot of m-tile em (tile_prefix[e] <= em < tile_prefix[e+1]), as a scalar.
__device__ __forceinline__ int slot_of_tile(const int32_t* tile_prefix, int El, int32_t em) {
    int lo = 0, hi = El;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (tile_prefix[mid] <= em) lo = mid;
        else hi = mid;
    }
    return __builtin_amdgcn_readfirstlane(lo);
}

int num_cus();
// blocks of a persistent launch on `stream`: its usable CUs, rounded down to a multiple of 8
int grid_blocks(hipStream_t stream);

// Super-tile shape for NT column tiles and `blocks` blocks (8 XCDs); false if unusable.
inline bool pick_tile_order(int NT, int blocks, TileOrder* to) {
    const int per_xcd = blocks / 8;
    if (blocks % 8 != 0 || per_xcd < 1) return false;
    to->SN = 1;
    for (int sn : {8, 4, 2}) {
        if (NT % sn == 0 && per_xcd % sn == 0) {
            to->SN = sn;
            break;
        }
    }
    to->SM = per_xcd / to->SN;
    return true;
}

// fp8 path (expert_gemm_fp8.hip): quantise the stage's activations, then the block-scaled
// fp8 GEMM.  `act` is [cap, K] bf16, or with amap != NULL (gather form, up only) the
// [arows, K] global buffer whose row amap[r] / ak is permuted row r (a negative entry is a
// zero row); workspace holds the fp8 codes and scales.
size_t fp8_stage_workspace(int64_t cap, int64_t K);
moe_status run_fp8_stage(bool up, const void* act, const moe_plan* plan,
                         const moe_expert_weights* w, int64_t H, int64_t I, void* out,
                         void* workspace, size_t ws_bytes, hipStream_t stream,
                         const int32_t* amap = nullptr, int32_t ak = 1, int64_t arows = 0);

}  // namespace gemm
}  // namespace moe
