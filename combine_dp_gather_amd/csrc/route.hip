// Routing: gate logits (op_gate) and top-k selection (op_select_experts) of the SGLang
// walkthrough "SGLang 源码完全拆解(十七): DP Attention 与专家并行", section "operations 与
// yield"; output is the TopKOutput (topk_ids, topk_weights) of section "normal dispatch 的
// 调用链".  The pages do not define the selection arithmetic; the rule implemented is
// DeepSeek-V3's grouped sigmoid with a correction bias (the bias that the "fake" dispatch of
// section "推理时怎么“选副本”" zeroes) and plain softmax top-k.
//
// Exact-order gate.  The integer routing decision depends on the logits bit for bit, so
// the gate fixes one accumulation order: per (row, expert) an fp32 fma chain over h in
// ascending order from +0.  The kernel is a register-tiled fp32 FMA GEMM whose K loop runs
// in that order: a 128x128 output tile per 256-thread block, 8x8 outputs per thread, 32-deep
// K slices staged through LDS as fp32 (bf16 widened exactly), double-buffered.
#include <float.h>

#include "moe_dev.h"

namespace moe {
namespace {

// ------------------------------------------------------------------ gate logits
constexpr int GB_M = 128, GB_N = 128, GB_K = 32, G_THREADS = 256;
constexpr int G_PAD = 4;  // LDS row padding (floats)

template <typename T>
struct GateLoad;

// bf16: one 16-byte load = 8 consecutive h of one row
template <>
struct GateLoad<uint16_t> {
    static constexpr int kPerThread = (GB_M * GB_K) / (8 * G_THREADS);  // 2
    __device__ static void load(const uint16_t* __restrict__ src, int64_t rows, int64_t H,
                                int64_t r0, int64_t k0, uint4 (&buf)[kPerThread]) {
#pragma unroll
        for (int p = 0; p < kPerThread; ++p) {
            const int idx = threadIdx.x + p * G_THREADS;  // 0..511
            const int r = idx >> 2, c = (idx & 3) * 8;
            const int64_t gr = r0 + r, gk = k0 + c;
            uint4 v = {0, 0, 0, 0};
            if (gr < rows) {
                const uint16_t* ptr = src + gr * H + gk;
                if (gk + 8 <= H && ((reinterpret_cast<uintptr_t>(ptr) & 15) == 0)) {
                    v = *reinterpret_cast<const uint4*>(ptr);
                } else {
                    uint16_t t[8];
#pragma unroll
                    for (int q = 0; q < 8; ++q) t[q] = (gk + q < H) ? ptr[q] : 0;
                    v.x = t[0] | (uint32_t(t[1]) << 16);
                    v.y = t[2] | (uint32_t(t[3]) << 16);
                    v.z = t[4] | (uint32_t(t[5]) << 16);
                    v.w = t[6] | (uint32_t(t[7]) << 16);
                }
            }
            buf[p] = v;
        }
    }
    __device__ static void store(float (*lds)[GB_M + G_PAD], const uint4 (&buf)[kPerThread]) {
#pragma unroll
        for (int p = 0; p < kPerThread; ++p) {
            const int idx = threadIdx.x + p * G_THREADS;
            const int r = idx >> 2, c = (idx & 3) * 8;
            const uint32_t w[4] = {buf[p].x, buf[p].y, buf[p].z, buf[p].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                lds[c + 2 * q][r] = __uint_as_float(w[q] << 16);
                lds[c + 2 * q + 1][r] = __uint_as_float(w[q] & 0xffff0000u);
            }
        }
    }
};

// fp32: one 16-byte load = 4 consecutive h of one row
template <>
struct GateLoad<float> {
    static constexpr int kPerThread = (GB_M * GB_K) / (4 * G_THREADS);  // 4
    __device__ static void load(const float* __restrict__ src, int64_t rows, int64_t H, int64_t r0,
                                int64_t k0, float4 (&buf)[kPerThread]) {
#pragma unroll
        for (int p = 0; p < kPerThread; ++p) {
            const int idx = threadIdx.x + p * G_THREADS;  // 0..1023
            const int r = idx >> 3, c = (idx & 7) * 4;
            const int64_t gr = r0 + r, gk = k0 + c;
            float4 v = {0.f, 0.f, 0.f, 0.f};
            if (gr < rows) {
                const float* ptr = src + gr * H + gk;
                if (gk + 4 <= H && ((reinterpret_cast<uintptr_t>(ptr) & 15) == 0)) {
                    v = *reinterpret_cast<const float4*>(ptr);
                } else {
                    v.x = (gk + 0 < H) ? ptr[0] : 0.f;
                    v.y = (gk + 1 < H) ? ptr[1] : 0.f;
                    v.z = (gk + 2 < H) ? ptr[2] : 0.f;
                    v.w = (gk + 3 < H) ? ptr[3] : 0.f;
                }
            }
            buf[p] = v;
        }
    }
    __device__ static void store(float (*lds)[GB_M + G_PAD], const float4 (&buf)[kPerThread]) {
#pragma unroll
        for (int p = 0; p < kPerThread; ++p) {
            const int idx = threadIdx.x + p * G_THREADS;
            const int r = idx >> 3, c = (idx & 7) * 4;
            lds[c + 0][r] = buf[p].x;
            lds[c + 1][r] = buf[p].y;
            lds[c + 2][r] = buf[p].z;
            lds[c + 3][r] = buf[p].w;
        }
    }
};

template <typename T>
using GateBuf = typename std::conditional<std::is_same<T, float>::value, float4, uint4>::type;

template <typename T>
__global__ __launch_bounds__(G_THREADS) void gate_exact_kernel(const T* __restrict__ x,
                                                               const T* __restrict__ w,
                                                               const int32_t* __restrict__ row_valid,
                                                               int64_t G, int64_t E, int64_t H,
                                                               float* __restrict__ logits) {
    __shared__ float As[2][GB_K][GB_M + G_PAD];
    __shared__ float Bs[2][GB_K][GB_N + G_PAD];
    using L = GateLoad<T>;
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * GB_M;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * GB_N;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;

    GateBuf<T> abuf[L::kPerThread], bbuf[L::kPerThread];
    float acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;

    const int64_t KT = (H + GB_K - 1) / GB_K;
    L::load(x, G, H, m0, 0, abuf);
    L::load(w, E, H, n0, 0, bbuf);
    L::store(As[0], abuf);
    L::store(Bs[0], bbuf);
    __syncthreads();
    for (int64_t kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) {
            L::load(x, G, H, m0, (kt + 1) * GB_K, abuf);
            L::load(w, E, H, n0, (kt + 1) * GB_K, bbuf);
        }
#pragma unroll 4
        for (int kk = 0; kk < GB_K; ++kk) {
            const float4 a0 = *reinterpret_cast<const float4*>(&As[cur][kk][ty * 8]);
            const float4 a1 = *reinterpret_cast<const float4*>(&As[cur][kk][ty * 8 + 4]);
            const float4 b0 = *reinterpret_cast<const float4*>(&Bs[cur][kk][tx * 8]);
            const float4 b1 = *reinterpret_cast<const float4*>(&Bs[cur][kk][tx * 8 + 4]);
            const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            const float b[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
        if (kt + 1 < KT) {
            L::store(As[cur ^ 1], abuf);
            L::store(Bs[cur ^ 1], bbuf);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t g = m0 + ty * 8 + i;
        if (g >= G) break;
        const bool valid = row_valid == nullptr || row_valid[g] != 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t e = n0 + tx * 8 + j;
            if (e < E) logits[g * E + e] = valid ? acc[i][j] : 0.f;
        }
    }
}

// ------------------------------------------------------------------ selection
// One wave per global row.  Lane l holds experts e = l + 64*j, j < kMaxPerLane.
constexpr int S_THREADS = 256;
constexpr int kMaxE = 1024;
constexpr int kMaxPerLane = kMaxE / kWave;  // 16
constexpr int kMaxTopK = 32;
constexpr int kMaxGroups = 64;
constexpr int kMaxGroupTopn = 8;

// exp by Cody-Waite reduction and a degree-13 Taylor polynomial (Horner with fused steps):
//   n = rint(x / ln2), r = x - n*ln2 (ln2 split in a 32-bit head and a tail),
//   exp(x) = 2^n * sum_{i<=13} r^i / i!
// A fixed recipe, so that the fp64 routing keys do not depend on a libm.
__device__ double exp_cody_waite(double x) {
    const double kInvLn2 = 0x1.71547652b82fep+0;
    const double kLn2Hi = 0x1.62e42fee00000p-1;
    const double kLn2Lo = 0x1.a39ef35793c76p-33;
    if (x != x) return x;
    if (x > 709.8) return __builtin_huge_val();
    if (x < -745.2) return 0.0;
    const double n = rint(x * kInvLn2);
    double r = fma(-n, kLn2Hi, x);
    r = fma(-n, kLn2Lo, r);
    double inv_fact[14];
    double f = 1.0;
#pragma unroll
    for (int i = 0; i < 14; ++i) {
        if (i > 0) f *= static_cast<double>(i);
        inv_fact[i] = 1.0 / f;
    }
    double p = inv_fact[13];
#pragma unroll
    for (int i = 12; i >= 0; --i) p = fma(p, r, inv_fact[i]);
    return ldexp(p, static_cast<int>(n));
}

__device__ __forceinline__ double sigmoid64(double l) { return 1.0 / (1.0 + exp_cody_waite(-l)); }

// (value, index) wave argmax: larger value wins, equal values go to the lower index.
// Lanes without a candidate pass idx = INT32_MAX.
__device__ __forceinline__ void wave_argmax(double& v, int& idx) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const double ov = __shfl_xor(v, off);
        const int oi = __shfl_xor(idx, off);
        const bool take = (oi != INT32_MAX) &&
                          (idx == INT32_MAX || ov > v || (ov == v && oi < idx));
        if (take) {
            v = ov;
            idx = oi;
        }
    }
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

struct SelectArgs {
    const float* logits;
    const int32_t* row_valid;
    const float* bias;
    int64_t G;
    int E, k, kind, n_group, topk_group, group_topn, renorm;
    int32_t* ids;
    float* w;
};

__global__ __launch_bounds__(S_THREADS) void select_kernel(SelectArgs a) {
    __shared__ double keys_lds[S_THREADS / kWave][kMaxE];
    const int wv = threadIdx.x / kWave;
    const int lane = lane_id();
    const int64_t g = static_cast<int64_t>(blockIdx.x) * (S_THREADS / kWave) + wv;
    const int E = a.E, k = a.k;
    // every wave stays to the end (the grouped path has a block barrier); rows past G and
    // pad rows only skip the work
    const bool in_range = g < a.G;
    const bool active = in_range && (a.row_valid == nullptr || a.row_valid[g] != 0);
    const float* lg = a.logits + (in_range ? g : 0) * E;
    const int per_lane = (E + kWave - 1) / kWave;
    double key[kMaxPerLane];
    double score[kMaxPerLane];  // sigmoid (grouped) or logit (softmax)
    bool allow[kMaxPerLane];
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
        const int e = lane + j * kWave;
        allow[j] = false;
        key[j] = 0.0;
        score[j] = 0.0;
        if (active && j < per_lane && e < E) {
            const double l = static_cast<double>(lg[e]);
            if (a.kind == MOE_ROUTE_SOFTMAX) {
                score[j] = l;
                key[j] = l;
            } else {
                score[j] = sigmoid64(l);
                key[j] = score[j] + (a.bias ? static_cast<double>(a.bias[e]) : 0.0);
            }
            allow[j] = true;
        }
    }
    double den = 1.0, mx = 0.0;
    if (a.kind == MOE_ROUTE_SOFTMAX) {
        double m = -DBL_MAX;
#pragma unroll
        for (int j = 0; j < kMaxPerLane; ++j)
            if (allow[j] && key[j] > m) m = key[j];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) m = fmax(m, __shfl_xor(m, off));
        mx = m;
        double s = 0.0;
#pragma unroll
        for (int j = 0; j < kMaxPerLane; ++j)
            if (allow[j]) s += exp(key[j] - mx);
        den = wave_sum(s);
    } else {
        double* kl = keys_lds[wv];
#pragma unroll
        for (int j = 0; j < kMaxPerLane; ++j) {
            const int e = lane + j * kWave;
            if (allow[j]) kl[e] = key[j];
        }
        __syncthreads();
        // group scores: lane q < n_group scans group q's keys in ascending expert order and
        // keeps the group_topn largest (a strictly larger key displaces, so equal keys keep
        // the lower id first); the score adds them largest first
        const int per = E / a.n_group;
        double gscore = 0.0;
        int gidx = INT32_MAX;
        if (active && lane < a.n_group) {
            double top[kMaxGroupTopn];
            int cnt = 0;
            for (int e = lane * per; e < (lane + 1) * per; ++e) {
                const double v = kl[e];
                int p;
                if (cnt < a.group_topn) {
                    p = cnt++;
                } else if (v > top[a.group_topn - 1]) {
                    p = a.group_topn - 1;
                } else {
                    continue;
                }
                while (p > 0 && v > top[p - 1]) {
                    top[p] = top[p - 1];
                    --p;
                }
                top[p] = v;
            }
            double acc = 0.0;
            for (int j = 0; j < a.group_topn; ++j) acc += top[j];
            gscore = acc;
            gidx = lane;
        }
        // keep the topk_group best groups (ties to the lower group)
        uint64_t kept = 0;
        bool mine_taken = false;
        if (active) {
            for (int t = 0; t < a.topk_group; ++t) {
                double v = mine_taken ? 0.0 : gscore;
                int i = mine_taken ? INT32_MAX : gidx;
                wave_argmax(v, i);
                kept |= (1ull << i);
                if (i == gidx) mine_taken = true;
            }
        }
#pragma unroll
        for (int j = 0; j < kMaxPerLane; ++j) {
            const int e = lane + j * kWave;
            if (allow[j]) allow[j] = (kept >> (e / per)) & 1ull;
        }
    }
    if (!in_range) return;
    int32_t* ids = a.ids + g * k;
    float* wout = a.w + g * k;
    if (!active) {
        for (int j = lane; j < k; j += kWave) {
            ids[j] = -1;
            wout[j] = 0.f;
        }
        return;
    }
    // top-k over the allowed keys, descending, ties to the lower id; lane t keeps pick t
    double my_score = 0.0;
    int my_id = -1;
    for (int t = 0; t < k; ++t) {
        double v = 0.0;
        int i = INT32_MAX;
#pragma unroll
        for (int j = 0; j < kMaxPerLane; ++j) {
            if (!allow[j]) continue;
            if (i == INT32_MAX || key[j] > v) {  // ascending e per lane: ties keep the lower id
                v = key[j];
                i = lane + j * kWave;
            }
        }
        wave_argmax(v, i);
        double sc = 0.0;
#pragma unroll
        for (int j = 0; j < kMaxPerLane; ++j) {
            if (allow[j] && lane + j * kWave == i) {
                allow[j] = false;
                sc = score[j];
            }
        }
        sc = __shfl(sc, i & (kWave - 1));
        if (lane == t) {
            my_score = sc;
            my_id = i;
        }
    }
    const double p = (a.kind == MOE_ROUTE_SOFTMAX) ? exp(my_score - mx) / den : my_score;
    double sum = 0.0;
    for (int t = 0; t < k; ++t) sum += __shfl(p, t);  // slot order
    if (lane < k) {
        ids[lane] = my_id;
        wout[lane] = static_cast<float>(a.renorm ? p / sum : p);
    }
}

moe_status check_route_cfg(const moe_route_cfg* c) {
    MOE_CHECK_ARG(c);
    MOE_CHECK_ARG(c->kind == MOE_ROUTE_SOFTMAX || c->kind == MOE_ROUTE_GROUPED_SIGMOID);
    MOE_CHECK_ARG(c->num_experts >= 1 && c->num_experts <= kMaxE);
    MOE_CHECK_ARG(c->top_k >= 1 && c->top_k <= kMaxTopK && c->top_k <= c->num_experts);
    if (c->kind == MOE_ROUTE_GROUPED_SIGMOID) {
        MOE_CHECK_ARG(c->n_group >= 1 && c->n_group <= kMaxGroups);
        MOE_CHECK_ARG(c->num_experts % c->n_group == 0);
        const int per = c->num_experts / c->n_group;
        MOE_CHECK_ARG(c->topk_group >= 1 && c->topk_group <= c->n_group);
        MOE_CHECK_ARG(c->group_topn >= 1 && c->group_topn <= kMaxGroupTopn && c->group_topn <= per);
        MOE_CHECK_ARG(c->top_k <= c->topk_group * per);
    }
    return MOE_OK;
}

moe_status launch_select(const float* logits, const int32_t* row_valid, int64_t G,
                         const float* bias, const moe_route_cfg* c, int32_t* ids, float* w,
                         hipStream_t stream) {
    SelectArgs a;
    a.logits = logits;
    a.row_valid = row_valid;
    a.bias = c->kind == MOE_ROUTE_GROUPED_SIGMOID ? bias : nullptr;
    a.G = G;
    a.E = c->num_experts;
    a.k = c->top_k;
    a.kind = c->kind;
    a.n_group = c->n_group;
    a.topk_group = c->topk_group;
    a.group_topn = c->group_topn;
    a.renorm = c->renormalize;
    a.ids = ids;
    a.w = w;
    const int rows_per_block = S_THREADS / kWave;
    const int64_t blocks = ceil_div(G, rows_per_block);
    hipLaunchKernelGGL(select_kernel, dim3(static_cast<unsigned>(blocks)), dim3(S_THREADS), 0,
                       stream, a);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_route_from_logits(const float* logits, const int32_t* row_valid,
                                            int64_t G, const float* bias, const moe_route_cfg* cfg,
                                            int32_t* topk_ids, float* topk_w, hipStream_t stream) {
    moe_status st = moe::check_route_cfg(cfg);
    if (st != MOE_OK) return st;
    MOE_CHECK_ARG(G >= 0);
    if (G == 0) return MOE_OK;
    MOE_CHECK_ARG(logits && topk_ids && topk_w);
    MOE_CHECK_ARG(G <= (int64_t)1 << 31);
    return moe::launch_select(logits, row_valid, G, bias, cfg, topk_ids, topk_w, stream);
}

extern "C" moe_status moe_route(const void* global_x, const int32_t* row_valid, int64_t G,
                                int64_t H, moe_dtype dt, const void* w_router, const float* bias,
                                const moe_route_cfg* cfg, float* logits, int32_t* topk_ids,
                                float* topk_w, hipStream_t stream) {
    moe_status st = moe::check_route_cfg(cfg);
    if (st != MOE_OK) return st;
    MOE_CHECK_ARG(G >= 0 && H > 0);
    MOE_CHECK_ARG(dt == MOE_F32 || dt == MOE_BF16);
    if (G == 0) return MOE_OK;
    MOE_CHECK_ARG(global_x && w_router && logits && topk_ids && topk_w);
    MOE_CHECK_ARG(G <= (int64_t)1 << 31);
    const int64_t E = cfg->num_experts;
    dim3 grid(static_cast<unsigned>(moe::ceil_div(E, moe::GB_N)),
              static_cast<unsigned>(moe::ceil_div(G, moe::GB_M)));
    if (dt == MOE_BF16) {
        hipLaunchKernelGGL(moe::gate_exact_kernel<uint16_t>, grid, dim3(moe::G_THREADS), 0, stream,
                           static_cast<const uint16_t*>(global_x),
                           static_cast<const uint16_t*>(w_router), row_valid, G, E, H, logits);
    } else {
        hipLaunchKernelGGL(moe::gate_exact_kernel<float>, grid, dim3(moe::G_THREADS), 0, stream,
                           static_cast<const float*>(global_x), static_cast<const float*>(w_router),
                           row_valid, G, E, H, logits);
    }
    MOE_LAUNCH_CHECK();
    return moe::launch_select(logits, row_valid, G, bias, cfg, topk_ids, topk_w, stream);
}
