// Expert-load statistics and expert placement (EPLB).
//
// SGLang walkthrough "SGLang 源码完全拆解(十七): DP Attention 与专家并行", section "EPLB:专家分布不均
// 怎么办" and its subsections:
//   - "统计:把物理计数还原成逻辑计数": per-step token counts per physical expert slot, turned into
//     per-logical-expert load by adding each slot's count to the expert it holds;
//   - "不均衡的代价与冗余专家的思路": balancedness = (mean + 1e-5) / (max + 1e-5) of the per-GPU
//     token counts;
//   - "三步算法:分组、复制、再打包": the hierarchical placement (whole groups to nodes, replicas
//     inside a node, slots to the node's GPUs);
//   - "逻辑与物理的两套映射": the logical -> physical table that dispatch reads.
//
// Counting runs on the device every step.  Without an all-to-all back end every rank routes
// every token and picks replicas rank-invariantly (section "推理时怎么“选副本”"), so one rank
// can count the load of every physical slot from its own top-k ids: no collective is needed
// to assemble the global view.  Placement is a host algorithm run between windows.
#include <algorithm>
#include <vector>

#include "moe_dev.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxPhysical = 8192;  // LDS bins of the count kernel (32 KiB of int32)
constexpr int kMaxLogical = 4096;   // LDS bins of the scatter-add kernel (32 KiB of int64)

// Block histogram of the rank-invariant picks over a grid-stride share of the pairs, then one
// 64-bit atomic add per non-zero bin.  Integer only: the result does not depend on order.
__global__ __launch_bounds__(kThreads) void load_count_kernel(const int32_t* __restrict__ ids, int64_t pairs,
                                                              int32_t k, const int32_t* __restrict__ phys_of,
                                                              const int32_t* __restrict__ n_rep, int32_t E,
                                                              int32_t max_rep, int32_t P,
                                                              unsigned long long* __restrict__ out) {
    __shared__ uint32_t bins[kMaxPhysical];
    for (int b = threadIdx.x; b < P; b += kThreads) bins[b] = 0u;
    __syncthreads();
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    for (int64_t f = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; f < pairs; f += stride) {
        const int32_t e = ids[f];
        if (e < 0 || e >= E) continue;
        const int64_t g = f / k;
        const int32_t nr = n_rep[e];
        if (nr < 1 || nr > max_rep) continue;  // malformed row: counted nowhere
        const int32_t p = phys_of[static_cast<int64_t>(e) * max_rep + g % nr];
        if (p >= 0 && p < P) atomicAdd(&bins[p], 1u);
    }
    __syncthreads();
    for (int b = threadIdx.x; b < P; b += kThreads) {
        const uint32_t c = bins[b];
        if (c) atomicAdd(&out[b], static_cast<unsigned long long>(c));
    }
}

// One block per layer: logical[l, phy2log[l, p]] += phys[l, p], written in full.
__global__ __launch_bounds__(kThreads) void phys_to_logical_kernel(const int64_t* __restrict__ phys,
                                                                   const int32_t* __restrict__ phy2log,
                                                                   int32_t P, int32_t E,
                                                                   int64_t* __restrict__ logical) {
    __shared__ unsigned long long acc[kMaxLogical];
    const int64_t l = blockIdx.x;
    for (int e = threadIdx.x; e < E; e += kThreads) acc[e] = 0ull;
    __syncthreads();
    for (int p = threadIdx.x; p < P; p += kThreads) {
        const int32_t e = phy2log[l * P + p];
        if (e >= 0 && e < E) atomicAdd(&acc[e], static_cast<unsigned long long>(phys[l * P + p]));
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kThreads) logical[l * E + e] = static_cast<int64_t>(acc[e]);
}

// ------------------------------------------------------------------ host placement
// Greedy balanced packing: items heaviest first (ties: lower index), each into the lightest
// pack that still has room (ties: lower pack), n / m items per pack.  pos is the order in
// which the pack received the item.
void pack_balanced(const std::vector<double>& w, int m, std::vector<int>& pack, std::vector<int>& pos) {
    const int n = static_cast<int>(w.size());
    const int per = n / m;
    std::vector<int> order(n);
    for (int i = 0; i < n; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return w[a] > w[b]; });
    std::vector<double> load(m, 0.0);
    std::vector<int> size(m, 0);
    pack.assign(n, 0);
    pos.assign(n, 0);
    for (int i : order) {
        int q = -1;
        for (int c = 0; c < m; ++c)
            if (size[c] < per && (q < 0 || load[c] < load[q])) q = c;
        pack[i] = q;
        pos[i] = size[q]++;
        load[q] += w[i];
    }
}

// Replication: one slot per expert in index order, then each extra slot to the expert with
// the largest load per replica (ties: lower index).
void replicate(const std::vector<double>& w, int slots, std::vector<int>& slot_expert,
               std::vector<int>& slot_rank, std::vector<int>& count) {
    const int n = static_cast<int>(w.size());
    slot_expert.resize(slots);
    slot_rank.resize(slots);
    count.assign(n, 1);
    for (int i = 0; i < n; ++i) {
        slot_expert[i] = i;
        slot_rank[i] = 0;
    }
    for (int s = n; s < slots; ++s) {
        int best = 0;
        double best_v = w[0] / count[0];
        for (int e = 1; e < n; ++e) {
            const double v = w[e] / count[e];
            if (v > best_v) {
                best = e;
                best_v = v;
            }
        }
        slot_expert[s] = best;
        slot_rank[s] = count[best]++;
    }
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_expert_load(const int32_t* topk_ids, int64_t G, int32_t k, const moe_expert_map* map,
                                      int32_t num_physical, int64_t* phys_count, hipStream_t stream) {
    using namespace moe;
    MOE_CHECK_ARG(map && G >= 0 && k >= 1 && k <= 64);
    MOE_CHECK_ARG(num_physical >= 1 && num_physical <= kMaxPhysical);
    MOE_CHECK_ARG(map->num_logical >= 1 && map->max_rep >= 1 && map->phys_of && map->n_rep);
    if (G == 0) return MOE_OK;
    MOE_CHECK_ARG(topk_ids && phys_count);
    const int64_t pairs = G * k;
    int64_t blocks = ceil_div(pairs, static_cast<int64_t>(kThreads) * 8);
    if (blocks > 1024) blocks = 1024;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(load_count_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream, topk_ids,
                       pairs, k, map->phys_of, map->n_rep, map->num_logical, map->max_rep, num_physical,
                       reinterpret_cast<unsigned long long*>(phys_count));
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

extern "C" moe_status moe_physical_to_logical_count(const int64_t* phys_count, const int32_t* phy2log,
                                                    int32_t num_layers, int32_t num_physical,
                                                    int32_t num_logical, int64_t* logical_count,
                                                    hipStream_t stream) {
    using namespace moe;
    MOE_CHECK_ARG(num_layers >= 0 && num_physical >= 1 && num_logical >= 1 && num_logical <= kMaxLogical);
    if (num_layers == 0) return MOE_OK;
    MOE_CHECK_ARG(phys_count && phy2log && logical_count);
    hipLaunchKernelGGL(phys_to_logical_kernel, dim3(static_cast<unsigned>(num_layers)), dim3(kThreads), 0, stream,
                       phys_count, phy2log, num_physical, num_logical, logical_count);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

extern "C" moe_status moe_eplb_balancedness(const int64_t* phys_count, int32_t num_layers, int32_t num_physical,
                                            int32_t num_gpus, double* out) {
    MOE_CHECK_ARG(phys_count && out && num_layers >= 0 && num_physical >= 1 && num_gpus >= 1);
    MOE_CHECK_ARG(num_physical % num_gpus == 0);
    const int per = num_physical / num_gpus;
    for (int32_t l = 0; l < num_layers; ++l) {
        double sum = 0.0, mx = 0.0;
        for (int32_t r = 0; r < num_gpus; ++r) {
            int64_t c = 0;
            for (int s = 0; s < per; ++s) c += phys_count[static_cast<int64_t>(l) * num_physical + r * per + s];
            const double v = static_cast<double>(c);
            sum += v;
            mx = (r == 0 || v > mx) ? v : mx;
        }
        out[l] = (sum / num_gpus + 1e-5) / (mx + 1e-5);
    }
    return MOE_OK;
}

extern "C" moe_status moe_eplb_rebalance(const double* weight, int32_t num_layers, int32_t num_logical,
                                         int32_t num_physical, int32_t num_groups, int32_t num_nodes,
                                         int32_t num_gpus, int32_t* phy2log, int32_t* phy_rank,
                                         int32_t* log_count) {
    MOE_CHECK_ARG(weight && phy2log && phy_rank && log_count);
    MOE_CHECK_ARG(num_layers >= 0 && num_logical >= 1 && num_physical >= 1);
    MOE_CHECK_ARG(num_groups >= 1 && num_nodes >= 1 && num_gpus >= 1);
    MOE_CHECK_ARG(num_logical % num_groups == 0 && num_groups % num_nodes == 0);
    MOE_CHECK_ARG(num_gpus % num_nodes == 0 && num_physical % num_gpus == 0);
    const int E = num_logical, P = num_physical;
    const int gsize = E / num_groups;
    const int e_node = E / num_nodes, p_node = P / num_nodes;
    const int gpus_node = num_gpus / num_nodes, per_gpu = P / num_gpus;
    MOE_CHECK_ARG(p_node >= e_node);
    for (int64_t i = 0; i < static_cast<int64_t>(num_layers) * E; ++i)
        MOE_CHECK_ARG(weight[i] >= 0.0 && weight[i] < 1e300);  // finite, non-negative loads
    std::vector<double> gload(num_groups), wl(e_node), share(p_node);
    std::vector<int> gnode, gpos, members(E), s_exp, s_rank, cnt, gpu, pos;
    for (int32_t l = 0; l < num_layers; ++l) {
        const double* w = weight + static_cast<int64_t>(l) * E;
        // 1. groups to nodes by group load (summed in ascending expert order)
        for (int q = 0; q < num_groups; ++q) {
            double s = 0.0;
            for (int t = 0; t < gsize; ++t) s += w[q * gsize + t];
            gload[q] = s;
        }
        moe::pack_balanced(gload, num_nodes, gnode, gpos);
        // members[node * e_node + j]: the node's logical experts, group by group in the order
        // the node received them, ascending id inside a group
        for (int q = 0; q < num_groups; ++q)
            for (int t = 0; t < gsize; ++t) members[gnode[q] * e_node + gpos[q] * gsize + t] = q * gsize + t;
        for (int nd = 0; nd < num_nodes; ++nd) {
            const int* ex = &members[nd * e_node];
            for (int j = 0; j < e_node; ++j) wl[j] = w[ex[j]];
            // 2. the node's slots to its experts
            moe::replicate(wl, p_node, s_exp, s_rank, cnt);
            // 3. the node's slots to its GPUs by per-replica load
            for (int i = 0; i < p_node; ++i) share[i] = wl[s_exp[i]] / cnt[s_exp[i]];
            moe::pack_balanced(share, gpus_node, gpu, pos);
            for (int i = 0; i < p_node; ++i) {
                const int64_t slot = static_cast<int64_t>(l) * P + nd * p_node + gpu[i] * per_gpu + pos[i];
                phy2log[slot] = ex[s_exp[i]];
                phy_rank[slot] = s_rank[i];
            }
            for (int j = 0; j < e_node; ++j) log_count[static_cast<int64_t>(l) * E + ex[j]] = cnt[j];
        }
    }
    return MOE_OK;
}

extern "C" moe_status moe_eplb_logical_to_physical(const int32_t* phy2log, const int32_t* phy_rank,
                                                   int32_t num_physical, int32_t num_logical, int32_t max_rep,
                                                   int32_t* phys_of, int32_t* n_rep) {
    MOE_CHECK_ARG(phy2log && phy_rank && phys_of && n_rep);
    MOE_CHECK_ARG(num_physical >= 1 && num_logical >= 1 && max_rep >= 1);
    for (int64_t i = 0; i < static_cast<int64_t>(num_logical) * max_rep; ++i) phys_of[i] = -1;
    for (int32_t e = 0; e < num_logical; ++e) n_rep[e] = 0;
    for (int32_t p = 0; p < num_physical; ++p) {
        const int32_t e = phy2log[p], r = phy_rank[p];
        MOE_CHECK_ARG(e >= 0 && e < num_logical && r >= 0);
        if (r >= max_rep) return MOE_ERR_CAPACITY;
        MOE_CHECK_ARG(phys_of[static_cast<int64_t>(e) * max_rep + r] < 0);  // each replica once
        phys_of[static_cast<int64_t>(e) * max_rep + r] = p;
        ++n_rep[e];
    }
    for (int32_t e = 0; e < num_logical; ++e) {
        MOE_CHECK_ARG(n_rep[e] >= 1);
        for (int32_t r = 0; r < n_rep[e]; ++r) MOE_CHECK_ARG(phys_of[static_cast<int64_t>(e) * max_rep + r] >= 0);
    }
    return MOE_OK;
}
