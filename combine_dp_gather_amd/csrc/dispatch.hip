// Dispatch: the (token, k) pairs of this rank's local expert slots, counting-sorted into one
// contiguous segment per slot, and the permuted copy of the activations.
//
// SGLang walkthrough "SGLang 源码完全拆解(十七): DP Attention 与专家并行":
//   - section "normal dispatch 的调用链": get_dispatch_layout's per-expert counts come first,
//     expert_alignment rounds each expert's rows up for the grouped GEMM tiles, and the
//     dispatch "handle" records where every pair went so that combine can bring it back;
//   - section "推理时怎么“选副本”": with redundant experts every rank must pick the same
//     physical replica for a token (rank_invariant), so the pick depends only on the global
//     row index: replica g mod n_rep.
//
// Kernels (one rank, one GPU, no atomics deciding any order):
//   1. count:   each block takes 1024 consecutive pairs (256 for batches of up to
//               kSmallPairs pairs) and builds a per-slot histogram in
//               LDS (integer LDS atomics: the counts do not depend on their order);
//   2. scan:    one block turns the per-block histograms into per-block bases (column prefix
//               over blocks), per-slot counts and the aligned exclusive scan seg_offsets; when
//               the count table is small, the place blocks do this themselves instead;
//   3. place:   each wave of a block owns a quarter of the block's pairs, walks it 64 pairs
//               at a time and ranks equal slots with ballots (rank = popcount of the lanes
//               below with the same slot), so rows follow ascending pair index: stable.
//               Up to 1024 pairs, one place block takes them all and counts them itself, so
//               neither the count launch nor the scan runs;
//   4. permute: x_perm[row] = global_x[sorted_pair[row] / k], one block per row, streaming
//               16-byte vectors, rows bounded by the device-side num_rows (no host sync).
//               Skipped when the caller passes no x_perm: the gathering up GEMM then reads
//               each row from global_x through sorted_pair itself, and the copy's traffic
//               (a read and a write of every routed row) is saved.
#include <mutex>

#include "moe_dev.h"

namespace moe {
namespace {

constexpr int D_THREADS = 256;
constexpr int D_WAVES = D_THREADS / kWave;
// pairs per thread of the count and place blocks: 4 (1024 per block) for large batches, 1
// (256 per block) up to kSmallPairs, where more, shorter blocks finish sooner
constexpr int kPairsPerThread = 4;
constexpr int kChunk = D_THREADS * kPairsPerThread;  // 1024 pairs per block
constexpr int kSmallPairs = 16384;
constexpr int kMaxSlots = 1024;

struct MapArgs {
    const int32_t* phys_of;
    const int32_t* n_rep;
    int32_t E, max_rep, p0, El;
};

// local slot of pair f (global row g = f / k, logical id l), or -1
__device__ __forceinline__ int pair_slot(int32_t l, uint32_t f, uint32_t k, const MapArgs& m) {
    if (l < 0 || l >= m.E) return -1;
    int32_t p = l;
    if (m.phys_of) {
        int32_t nr = m.n_rep[l];
        nr = nr < 1 ? 1 : nr;
        // pair indices fit in 32 bits (the launcher checks G * k < 2^31): 32-bit division
        const uint32_t g = f / k;
        const int32_t r = static_cast<int32_t>(g % static_cast<uint32_t>(nr));
        if (r >= m.max_rep) return -1;
        p = m.phys_of[static_cast<int64_t>(l) * m.max_rep + r];
    }
    p -= m.p0;
    return (p >= 0 && p < m.El) ? p : -1;
}

template <int PPT>
__global__ __launch_bounds__(D_THREADS) void count_kernel(const int32_t* __restrict__ ids,
                                                          int64_t P, int k, MapArgs m,
                                                          int32_t* __restrict__ blk_counts) {
    __shared__ int32_t hist[kMaxSlots];
    for (int e = threadIdx.x; e < m.El; e += D_THREADS) hist[e] = 0;
    __syncthreads();
    const int64_t base = static_cast<int64_t>(blockIdx.x) * (PPT * D_THREADS);
    // all of the thread's ids are loaded before the first LDS add
    int32_t idv[PPT];
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
        const int64_t f = base + i * D_THREADS + threadIdx.x;
        idv[i] = f < P ? ids[f] : -1;
    }
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
        const int64_t f = base + i * D_THREADS + threadIdx.x;
        if (f < P) {
            const int s = pair_slot(idv[i], static_cast<uint32_t>(f), static_cast<uint32_t>(k), m);
            if (s >= 0) atomicAdd(&hist[s], 1);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < m.El; e += D_THREADS)
        blk_counts[static_cast<int64_t>(blockIdx.x) * m.El + e] = hist[e];
}

constexpr int SCAN_THREADS = 1024;

// stride > 0: fixed-capacity layout, slot e owns rows [e * stride, (e + 1) * stride) and keeps
// at most stride pairs; stride == 0: packed segments of the counts rounded up to align.
__global__ __launch_bounds__(SCAN_THREADS) void scan_kernel(
    const int32_t* __restrict__ blk_counts, int64_t NB, int El, int align, int64_t stride,
    int64_t cap, int32_t* __restrict__ blk_base, int32_t* __restrict__ counts,
    int64_t* __restrict__ seg, int64_t* __restrict__ num_rows, int32_t* __restrict__ error_flag,
    int32_t* __restrict__ sorted_pair) {
    __shared__ int64_t sc[SCAN_THREADS];
    __shared__ int32_t kept[kMaxSlots];
    __shared__ int32_t part_sum[SCAN_THREADS];
    __shared__ int32_t over;
    const int tid = threadIdx.x;
    if (tid == 0) over = 0;
    // per-block bases of every slot: the threads are split into `parts` groups of El_pad
    // (a power of two >= El); thread (part, e) adds slot e's counts over one contiguous range
    // of blocks, the ranges' sums are scanned over parts in LDS, and each thread then writes
    // its range's running bases
    int el_pad = 1;
    while (el_pad < El) el_pad <<= 1;
    const int parts = SCAN_THREADS / el_pad;
    const int e_of = tid & (el_pad - 1), part = tid / el_pad;
    const int64_t per = (NB + parts - 1) / parts;
    const int64_t b0 = part * per < NB ? part * per : NB;
    const int64_t b1 = b0 + per < NB ? b0 + per : NB;
    int32_t mine = 0;
    if (e_of < El)
        for (int64_t b = b0; b < b1; ++b) mine += blk_counts[b * El + e_of];
    part_sum[tid] = mine;
    __syncthreads();
    for (int off = 1; off < parts; off <<= 1) {
        const int32_t v = part >= off ? part_sum[tid - off * el_pad] : 0;
        __syncthreads();
        part_sum[tid] += v;
        __syncthreads();
    }
    if (e_of < El) {
        int32_t run = part_sum[tid] - mine;
        for (int64_t b = b0; b < b1; ++b) {
            blk_base[b * El + e_of] = run;
            run += blk_counts[b * El + e_of];
        }
    }
    const int e = tid;
    int64_t padded = 0;
    if (e < El) {
        const int32_t run = part_sum[(parts - 1) * el_pad + e];
        int32_t keep = run;
        if (stride > 0) {
            if (run > stride) {
                keep = static_cast<int32_t>(stride);
                over = 1;
            }
            padded = stride;
        } else {
            const uint32_t al = static_cast<uint32_t>(align);
            padded = static_cast<int64_t>((static_cast<uint32_t>(run) + al - 1u) / al) * al;
        }
        counts[e] = keep;
        kept[e] = keep;
    }
    // inclusive scan of the padded counts over slots (Hillis-Steele in LDS)
    sc[e] = padded;
    __syncthreads();
    for (int off = 1; off < SCAN_THREADS; off <<= 1) {
        const int64_t v = (e >= off) ? sc[e - off] : 0;
        __syncthreads();
        sc[e] += v;
        __syncthreads();
    }
    if (e < El) {
        seg[e + 1] = sc[e];
        if (e == 0) seg[0] = 0;
    }
    // rows of a segment past its pairs (alignment pad, or unused capacity) hold no pair; the
    // whole block fills them segment by segment
    for (int q = 0; q < El; ++q) {
        const int64_t end = sc[q];
        const int64_t start = (q == 0 ? 0 : sc[q - 1]) + kept[q];
        for (int64_t r = start + e; r < end && r < cap; r += SCAN_THREADS) sorted_pair[r] = -1;
    }
    if (e == 0) {
        const int64_t end = sc[El - 1];
        *num_rows = end;
        *error_flag = (end > cap || over) ? 1 : 0;
    }
}

// Layout of the plan from the per-block counts, computed inside the place kernel when the
// count table is small (FUSED): every block adds the table itself -- the slot totals over all
// blocks and its own base over the blocks before it, with integer LDS atomics whose order
// does not matter -- then runs the aligned exclusive scan over slots.  Block 0 publishes the
// plan's counts, seg_offsets, num_rows and error_flag, and all blocks share the pad-row fill.
// This saves the separate scan launch and the per-block base round trip through memory.
constexpr int64_t kFusedScanLimit = 65536;  // NB * El entries each block adds up
// Pairs one block places alone.  At 1020 pairs (170 tokens over 4 replicas, top-6) the dispatch
// took 8.1 us this way against 12.8 us with the count launch; a form with 12 pairs per lane was
// slower at 3072 pairs (14.4 against 12.4 us), so larger batches keep the count blocks.
constexpr int64_t kSoloPairs = kChunk;

struct ScanArgs {
    const int32_t* blk_counts;  // [NB][El]
    int64_t NB;
    int align;
    int64_t stride;
    int32_t* counts;
    int64_t* seg;
    int64_t* num_rows;
    int32_t* error_flag;
};

// SOLO (FUSED with one block): the block holds every pair, so the slot totals are its own wave
// histograms and no count table is read; the count launch is left out.
template <bool FUSED, bool SOLO, int PPT>
__global__ __launch_bounds__(D_THREADS) void place_kernel(
    const int32_t* __restrict__ ids, int64_t P, int k, MapArgs m,
    const int32_t* __restrict__ blk_base, const int64_t* __restrict__ seg_in, int64_t cap,
    ScanArgs sa, int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_row) {
    // a pair's row must also stay inside its slot's segment: in the fixed-capacity layout the
    // pairs past the capacity are dropped; packed segments always have room
    __shared__ int32_t whist[D_WAVES][kMaxSlots];
    __shared__ int64_t wbase[D_WAVES][kMaxSlots];
    // FUSED only: slot totals, this block's base, the segment offsets, the kept counts
    __shared__ int32_t tot[FUSED ? kMaxSlots : 1], before[FUSED ? kMaxSlots : 1];
    __shared__ int64_t seg_s[FUSED ? kMaxSlots + 1 : 1];
    __shared__ int64_t part[FUSED ? D_THREADS : 1];
    __shared__ int32_t over;
    const int tid = threadIdx.x;
    const int wv = tid / kWave;
    const int lane = lane_id();
    const int El = m.El;
    for (int w = 0; w < D_WAVES; ++w)
        for (int e = tid; e < El; e += D_THREADS) whist[w][e] = 0;
    if constexpr (FUSED) {
        for (int e = tid; e < El; e += D_THREADS) {
            tot[e] = 0;
            before[e] = 0;
        }
        if (tid == 0) over = 0;
    }
    __syncthreads();
    static_assert(!SOLO || FUSED, "the single-block form derives the layout itself");
    constexpr int STEPS = PPT;  // each wave owns PPT * 64 consecutive pairs
    const int64_t wstart = (static_cast<int64_t>(blockIdx.x) * D_WAVES + wv) * (STEPS * kWave);
    // FUSED: the first U count-table entries of this thread are loaded before the pass over
    // the ids, so the two global round trips overlap
    constexpr int U = 16;
    const int64_t n_tab = FUSED && !SOLO ? sa.NB * El : 0;
    int32_t c0[U];
    if constexpr (FUSED && !SOLO) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = tid + u * D_THREADS;
            c0[u] = i < n_tab ? sa.blk_counts[i] : 0;
        }
    }
    // per-wave histogram of its pairs; the ids are all loaded before the first LDS add, and
    // the slots stay in registers for the placement pass
    int32_t idv[STEPS];
#pragma unroll
    for (int step = 0; step < STEPS; ++step) {
        const int64_t f = wstart + step * kWave + lane;
        idv[step] = f < P ? ids[f] : -1;
    }
    int slot[STEPS];
#pragma unroll
    for (int step = 0; step < STEPS; ++step) {
        const int64_t f = wstart + step * kWave + lane;
        slot[step] = f < P ? pair_slot(idv[step], static_cast<uint32_t>(f), static_cast<uint32_t>(k), m) : -1;
        if (slot[step] >= 0) atomicAdd(&whist[wv][slot[step]], 1);
    }
    const int64_t* seg = seg_in;
    if constexpr (SOLO) {
        __syncthreads();
        for (int e = tid; e < El; e += D_THREADS) {
            int32_t t = 0;
            for (int w = 0; w < D_WAVES; ++w) t += whist[w][e];
            tot[e] = t;
        }
    }
    if constexpr (FUSED) {
        const int64_t mine_end = static_cast<int64_t>(blockIdx.x) * El;  // entries of earlier blocks
        // the thread's entries are i = tid + n * D_THREADS, n = 0, 1, ...; their slot i % El
        // advances by D_THREADS % El per entry
        const int e_step = D_THREADS % El;
        int e_cur = tid % El;
        auto add = [&](int64_t i, int32_t c) {
            if (c) {
                atomicAdd(&tot[e_cur], c);
                if (i < mine_end) atomicAdd(&before[e_cur], c);
            }
            e_cur += e_step;
            if (e_cur >= El) e_cur -= El;
        };
        if constexpr (!SOLO) {
#pragma unroll
            for (int u = 0; u < U; ++u) add(tid + u * D_THREADS, c0[u]);
        }
        for (int64_t i0 = tid + U * D_THREADS; i0 < n_tab; i0 += D_THREADS * U) {
            int32_t c[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = i0 + u * D_THREADS;
                c[u] = i < n_tab ? sa.blk_counts[i] : 0;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) add(i0 + u * D_THREADS, c[u]);
        }
        __syncthreads();
        // aligned exclusive scan over slots: thread t owns slots 4t .. 4t+3
        constexpr int SPT = kMaxSlots / D_THREADS;
        int64_t padded[SPT];
        int64_t sum = 0;
#pragma unroll
        for (int q = 0; q < SPT; ++q) {
            const int e = tid * SPT + q;
            padded[q] = 0;
            if (e < El) {
                const int32_t run = tot[e];
                if (sa.stride > 0) {
                    if (run > sa.stride) over = 1;
                    padded[q] = sa.stride;
                } else {
                    // run < 2^31 and align < 2^31: the rounding fits 32 bits
                    const uint32_t al = static_cast<uint32_t>(sa.align);
                    padded[q] = static_cast<int64_t>((static_cast<uint32_t>(run) + al - 1u) / al) * al;
                }
            }
            sum += padded[q];
        }
        int64_t incl;
        if (El <= kWave * SPT) {
            // every slot sits in wave 0: an inclusive scan by shuffles, no barriers
            incl = sum;
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const int64_t v = __shfl_up(incl, off);
                if (lane >= off) incl += v;
            }
            if (tid == kWave - 1) part[D_THREADS - 1] = incl;
        } else {
            part[tid] = sum;
            __syncthreads();
            for (int off = 1; off < D_THREADS; off <<= 1) {
                const int64_t v = tid >= off ? part[tid - off] : 0;
                __syncthreads();
                part[tid] += v;
                __syncthreads();
            }
            incl = part[tid];
        }
        int64_t run = incl - sum;
#pragma unroll
        for (int q = 0; q < SPT; ++q) {
            const int e = tid * SPT + q;
            if (e < El) seg_s[e] = run;
            run += padded[q];
        }
        __syncthreads();
        if (tid == 0) seg_s[El] = part[D_THREADS - 1];
        __syncthreads();
        seg = seg_s;
        const bool publish = blockIdx.x == 0;
        // rows of a segment past its kept pairs (alignment pad, or unused capacity) hold no
        // pair; a thread takes slots tid, tid + D_THREADS, ... and the blocks share each
        // slot's rows (block b writes rows b, b + gridDim.x, ... of the range)
        auto kept = [&](int e) -> int32_t {
            return sa.stride > 0 && tot[e] > sa.stride ? static_cast<int32_t>(sa.stride) : tot[e];
        };
        for (int e = tid; e < El; e += D_THREADS) {
            const int64_t end = seg_s[e + 1] < cap ? seg_s[e + 1] : cap;
            for (int64_t r = seg_s[e] + kept(e) + blockIdx.x; r < end; r += gridDim.x) sorted_pair[r] = -1;
        }
        if (publish) {
            for (int e = tid; e < El; e += D_THREADS) sa.counts[e] = kept(e);
            for (int e = tid; e <= El; e += D_THREADS) sa.seg[e] = seg_s[e];
            if (tid == 0) {
                *sa.num_rows = seg_s[El];
                *sa.error_flag = (seg_s[El] > cap || over) ? 1 : 0;
            }
        }
    } else {
        __syncthreads();
    }
    // first row of each wave's run of each slot
    for (int e = tid; e < El; e += D_THREADS) {
        int64_t run = seg[e] + (FUSED ? before[e] : blk_base[static_cast<int64_t>(blockIdx.x) * El + e]);
        for (int w = 0; w < D_WAVES; ++w) {
            wbase[w][e] = run;
            run += whist[w][e];
        }
    }
    __syncthreads();
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    // bits of a slot index: the lanes sharing a lane's slot are found one bit at a time (one
    // ballot per bit), whatever the number of distinct slots in the wave
    const int sbits = El > 1 ? 32 - __builtin_clz(static_cast<uint32_t>(El - 1)) : 0;
#pragma unroll
    for (int step = 0; step < STEPS; ++step) {
        const int64_t f = wstart + step * kWave + lane;
        const bool inb = f < P;
        const int s = slot[step];
        // lanes with the same slot as this one (its own included), for s >= 0
        uint64_t mine = __ballot(s >= 0);
        for (int b = 0; b < sbits; ++b) {
            const bool bit = (s >> b) & 1;
            const uint64_t ones = __ballot(s >= 0 && bit);
            mine &= bit ? ones : ~ones;
        }
        int64_t row = -1;
        if (s >= 0) row = wbase[wv][s] + __popcll(mine & below);
        // the lowest lane of each slot advances the wave's running row for it
        if (s >= 0 && (mine & below) == 0) wbase[wv][s] += __popcll(mine);
        if (inb) {
            if (row >= 0 && row < cap && row < seg[s + 1]) {
                sorted_pair[row] = static_cast<int32_t>(f);
                pair_row[f] = static_cast<int32_t>(row);
            } else {
                pair_row[f] = -1;
            }
        }
    }
}

// One block per x_perm row at a time (grid-stride over rows, bounded by the device-side
// num_rows): the row's source is one contiguous row of global_x, so the block streams a
// contiguous span in and out, kPermUnroll 16-byte loads per thread in flight before the stores.
constexpr int kPermUnroll = 4;
constexpr int kPermGrid = 8192;

template <typename V>
__global__ __launch_bounds__(D_THREADS) void permute_kernel(
    const V* __restrict__ x, const int32_t* __restrict__ sorted_pair,
    const int64_t* __restrict__ num_rows, int64_t cap, int k, int64_t row_units,
    bool zero_pads, V* __restrict__ x_perm) {
    int64_t rows = *num_rows;
    rows = rows < cap ? rows : cap;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const int32_t f = sorted_pair[r];
        if (f < 0 && !zero_pads) continue;  // unused capacity rows stay unwritten
        V* __restrict__ d = x_perm + r * row_units;
        // alignment pad rows (f < 0) are written as zeros
        const V* __restrict__ s = x + static_cast<int64_t>(f < 0 ? 0 : f / k) * row_units;
        for (int64_t c0 = threadIdx.x; c0 < row_units; c0 += D_THREADS * kPermUnroll) {
            V v[kPermUnroll];
#pragma unroll
            for (int u = 0; u < kPermUnroll; ++u) {
                const int64_t c = c0 + u * D_THREADS;
                v[u] = (f >= 0 && c < row_units) ? ld_stream(s + c) : V{};
            }
#pragma unroll
            for (int u = 0; u < kPermUnroll; ++u) {
                const int64_t c = c0 + u * D_THREADS;
                if (c < row_units) st_stream(d + c, v[u]);
            }
        }
    }
}

template <typename V>
moe_status launch_permute(const void* x, const moe_plan* plan, int64_t row_bytes, void* x_perm,
                          hipStream_t stream) {
    const int64_t row_units = row_bytes / static_cast<int64_t>(sizeof(V));
    const int64_t blocks = plan->cap < kPermGrid ? plan->cap : kPermGrid;
    hipLaunchKernelGGL(permute_kernel<V>, dim3(static_cast<unsigned>(blocks)), dim3(D_THREADS), 0,
                       stream, static_cast<const V*>(x), plan->sorted_pair, plan->num_rows,
                       plan->cap, plan->top_k, row_units, plan->seg_stride == 0, static_cast<V*>(x_perm));
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

// pairs per thread, and blocks, of the count and place launches for G * k pairs
int pairs_per_thread(int64_t P) { return P > kSoloPairs && P <= kSmallPairs ? 1 : kPairsPerThread; }
int64_t num_blocks(int64_t G, int32_t k) { return ceil_div(G * k, D_THREADS * pairs_per_thread(G * k)); }

}  // namespace
}  // namespace moe

extern "C" size_t moe_dispatch_workspace_size(int64_t G, int32_t k, int32_t num_slots) {
    if (G < 0 || k < 1 || num_slots < 1) return 0;
    const int64_t nb = moe::num_blocks(G, k);
    return static_cast<size_t>(2 * nb * num_slots) * sizeof(int32_t) + 256;
}

namespace moe {
namespace {

// Argument checks shared by both entry points; nothing is enqueued on failure.
moe_status check_dispatch_args(const void* global_x, const int32_t* topk_ids, int64_t G, int32_t k,
                               int64_t H, moe_dtype dt, const moe_expert_map* map, const moe_plan* plan,
                               const void* x_perm) {
    MOE_CHECK_ARG(map && plan);
    MOE_CHECK_ARG(G >= 0 && k >= 1 && H > 0);
    MOE_CHECK_ARG(dt == MOE_F32 || dt == MOE_BF16);
    MOE_CHECK_ARG(plan->G == G && plan->top_k == k);
    MOE_CHECK_ARG(plan->num_slots == map->num_slots);
    MOE_CHECK_ARG(map->num_slots >= 1 && map->num_slots <= kMaxSlots);
    MOE_CHECK_ARG(map->num_logical >= 1 && map->first_slot >= 0);
    MOE_CHECK_ARG(map->phys_of == nullptr || (map->n_rep != nullptr && map->max_rep >= 1));
    MOE_CHECK_ARG(plan->align >= 1 && plan->cap >= 0 && plan->seg_stride >= 0);
    // fixed-capacity layout: every segment inside the caller's rows, row indices in int32
    if (plan->seg_stride > 0)
        MOE_CHECK_ARG(plan->seg_stride <= (int64_t(1) << 31) / map->num_slots &&
                      plan->cap >= static_cast<int64_t>(map->num_slots) * plan->seg_stride);
    MOE_CHECK_ARG(plan->counts && plan->seg_offsets && plan->num_rows && plan->error_flag);
    MOE_CHECK_ARG(G * k < (int64_t(1) << 31));
    if (G > 0) MOE_CHECK_ARG(topk_ids && plan->pair_row && (global_x || !x_perm));
    if (plan->cap > 0) MOE_CHECK_ARG(plan->sorted_pair);
    return MOE_OK;
}

// The count blocks, then the place blocks (which scan a small count table themselves) or the
// scan kernel and the place blocks; NB = 0 runs the scan alone (empty plan).
template <int PPT>
moe_status count_and_place(const int32_t* topk_ids, int64_t P, int32_t k, const MapArgs& m, int64_t NB,
                           int El, const moe_plan* plan, const ScanArgs& sa, int32_t* blk_counts,
                           int32_t* blk_base, hipStream_t stream) {
    if (NB > 0) {
        hipLaunchKernelGGL(count_kernel<PPT>, dim3(static_cast<unsigned>(NB)), dim3(D_THREADS), 0, stream,
                           topk_ids, P, k, m, blk_counts);
        MOE_LAUNCH_CHECK();
    }
    if (NB > 0 && NB * El <= kFusedScanLimit) {
        hipLaunchKernelGGL((place_kernel<true, false, PPT>), dim3(static_cast<unsigned>(NB)), dim3(D_THREADS), 0,
                           stream, topk_ids, P, k, m, nullptr, nullptr, plan->cap, sa, plan->sorted_pair,
                           plan->pair_row);
        MOE_LAUNCH_CHECK();
        return MOE_OK;
    }
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(SCAN_THREADS), 0, stream, blk_counts, NB, El, plan->align,
                       static_cast<int64_t>(plan->seg_stride), plan->cap, blk_base, plan->counts,
                       plan->seg_offsets, plan->num_rows, plan->error_flag, plan->sorted_pair);
    MOE_LAUNCH_CHECK();
    if (NB == 0) return MOE_OK;
    hipLaunchKernelGGL((place_kernel<false, false, PPT>), dim3(static_cast<unsigned>(NB)), dim3(D_THREADS), 0,
                       stream, topk_ids, P, k, m, blk_base, plan->seg_offsets, plan->cap, sa, plan->sorted_pair,
                       plan->pair_row);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

// The kernels on a checked call; `workspace` holds the per-block count and base tables
// (2 * NB * E_l int32), every entry of which the count and scan kernels write before any
// kernel reads it, so its previous contents never matter.
moe_status run_dispatch(const void* global_x, const int32_t* topk_ids, int64_t G, int32_t k, int64_t H,
                        moe_dtype dt, const moe_expert_map* map, const moe_plan* plan, void* x_perm,
                        void* workspace, hipStream_t stream) {
    const int64_t P = G * k;
    const int64_t NB = num_blocks(G, k);
    const int El = map->num_slots;
    MOE_CHECK_ARG(NB == 0 || workspace != nullptr);
    MapArgs m{map->phys_of, map->n_rep, map->num_logical, map->max_rep, map->first_slot, El};
    int32_t* blk_counts = static_cast<int32_t*>(workspace);
    int32_t* blk_base = blk_counts + NB * El;
    ScanArgs sa{blk_counts, NB, plan->align, static_cast<int64_t>(plan->seg_stride), plan->counts,
                plan->seg_offsets, plan->num_rows, plan->error_flag};
    if (NB > 0 && P <= kSoloPairs) {
        // one block holds every pair: no count table, no count launch
        hipLaunchKernelGGL((place_kernel<true, true, kPairsPerThread>), dim3(1), dim3(D_THREADS), 0, stream,
                           topk_ids, P, k, m, nullptr, nullptr, plan->cap, sa, plan->sorted_pair,
                           plan->pair_row);
        MOE_LAUNCH_CHECK();
    } else {
        const moe_status st = pairs_per_thread(P) == 1
                                  ? count_and_place<1>(topk_ids, P, k, m, NB, El, plan, sa, blk_counts, blk_base, stream)
                                  : count_and_place<kPairsPerThread>(topk_ids, P, k, m, NB, El, plan, sa, blk_counts,
                                                                     blk_base, stream);
        if (st != MOE_OK || NB == 0) return st;
    }
    // no x_perm: the plan only (the gathering up GEMM reads the rows in place)
    if (plan->cap == 0 || x_perm == nullptr) return MOE_OK;
    const int64_t row_bytes = H * dtype_size(dt);
    if (row_bytes % 16 == 0 && aligned(global_x, 16) && aligned(x_perm, 16))
        return launch_permute<uint4>(global_x, plan, row_bytes, x_perm, stream);
    if (row_bytes % 4 == 0 && aligned(global_x, 4) && aligned(x_perm, 4))
        return launch_permute<uint32_t>(global_x, plan, row_bytes, x_perm, stream);
    return launch_permute<uint16_t>(global_x, plan, row_bytes, x_perm, stream);
}

// ---- the no-allocation variant's scratch: a fixed device array, one copy per GPU, kept
// until the process ends.  In host code `scratch` names a host-side stand-in, never the
// device memory: its device address is looked up once per device with that device current
// and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[MOE_DISPATCH_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

moe_status scratch_for_current_device(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ERR_HIP;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_dispatch(const void* global_x, const int32_t* topk_ids, int64_t G,
                                   int32_t k, int64_t H, moe_dtype dt, const moe_expert_map* map,
                                   const moe_plan* plan, void* x_perm, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
    const moe_status st = moe::check_dispatch_args(global_x, topk_ids, G, k, H, dt, map, plan, x_perm);
    if (st != MOE_OK) return st;
    if (workspace_bytes < moe_dispatch_workspace_size(G, k, map->num_slots)) return MOE_ERR_CAPACITY;
    return moe::run_dispatch(global_x, topk_ids, G, k, H, dt, map, plan, x_perm, workspace, stream);
}

extern "C" moe_status moe_dispatch_noalloc(const void* global_x, const int32_t* topk_ids, int64_t G,
                                           int32_t k, int64_t H, moe_dtype dt, const moe_expert_map* map,
                                           const moe_plan* plan, void* x_perm, hipStream_t stream) {
    moe_status st = moe::check_dispatch_args(global_x, topk_ids, G, k, H, dt, map, plan, x_perm);
    if (st != MOE_OK) return st;
    if (moe_dispatch_workspace_size(G, k, map->num_slots) > MOE_DISPATCH_NOALLOC_SCRATCH_BYTES)
        return MOE_ERR_SCRATCH_LIMIT;
    void* ws = nullptr;
    st = moe::scratch_for_current_device(&ws);
    if (st != MOE_OK) return st;
    return moe::run_dispatch(global_x, topk_ids, G, k, H, dt, map, plan, x_perm, ws, stream);
}
