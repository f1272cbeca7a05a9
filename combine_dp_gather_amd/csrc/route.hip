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
// One wave per global row.  Lane l holds the V consecutive experts e = l*V + j (V = E/64
// rounded up to a power of two), so a group of E/n_group experts covers E/(n_group*V)
// neighbouring lanes and group statistics reduce with xor shuffles inside those lanes.
constexpr int S_THREADS = 256;
constexpr int S_WAVES = S_THREADS / kWave;
constexpr int kMaxE = 1024;
constexpr int kMaxTopK = 32;
constexpr int kMaxGroups = 64;
constexpr int kMaxGroupTopn = 4;
constexpr int kNone = INT32_MAX;

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

// a ranks before b: larger key, equal keys by lower id; kNone never ranks first
__device__ __forceinline__ bool ranks_before(double ka, int ia, double kb, int ib) {
    return ia != kNone && (ib == kNone || ka > kb || (ka == kb && ia < ib));
}

// (key, id) wave argmax with the same order; every lane ends with the winner
__device__ __forceinline__ void wave_argmax(double& v, int& idx) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const double ov = __shfl_xor(v, off);
        const int oi = __shfl_xor(idx, off);
        if (ranks_before(ov, oi, v, idx)) {
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

__device__ __forceinline__ double readlane_f64(double v, int l) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane(static_cast<int>(b & 0xffffffffll), l);
    const int hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), l);
    return __longlong_as_double((static_cast<long long>(hi) << 32) |
                                static_cast<long long>(static_cast<unsigned>(lo)));
}

// sort a lane's V entries best-first (odd-even transposition: static indices only)
template <int V>
__device__ __forceinline__ void sort_lane(double (&k)[V], double (&s)[V], int (&id)[V]) {
#pragma unroll
    for (int r = 0; r < V; ++r) {
#pragma unroll
        for (int i = r & 1; i + 1 < V; i += 2) {
            if (ranks_before(k[i + 1], id[i + 1], k[i], id[i])) {
                const double tk = k[i], ts = s[i];
                const int ti = id[i];
                k[i] = k[i + 1]; s[i] = s[i + 1]; id[i] = id[i + 1];
                k[i + 1] = tk; s[i + 1] = ts; id[i + 1] = ti;
            }
        }
    }
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

template <int V>
__global__ __launch_bounds__(S_THREADS) void select_kernel(SelectArgs a) {
    const int lane = lane_id();
    const int64_t g = static_cast<int64_t>(blockIdx.x) * S_WAVES + threadIdx.x / kWave;
    if (g >= a.G) return;  // no block barrier below
    const int E = a.E, k = a.k;
    int32_t* ids = a.ids + g * k;
    float* wout = a.w + g * k;
    if (a.row_valid && a.row_valid[g] == 0) {  // pad row: no expert load
        if (lane < k) {
            ids[lane] = -1;
            wout[lane] = 0.f;
        }
        return;
    }
    const float* lg = a.logits + g * E;
    const bool grouped = a.kind == MOE_ROUTE_GROUPED_SIGMOID;
    double key[V], score[V];
    int id[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const int e = lane * V + j;
        key[j] = -__builtin_huge_val();
        score[j] = 0.0;
        id[j] = kNone;
        if (e < E) {
            const double l = static_cast<double>(lg[e]);
            if (grouped) {
                score[j] = sigmoid64(l);
                key[j] = score[j] + (a.bias ? static_cast<double>(a.bias[e]) : 0.0);
            } else {
                score[j] = l;
                key[j] = l;
            }
            id[j] = e;
        }
    }
    double mx = 0.0, den = 1.0;
    if (!grouped) {
        double m = -__builtin_huge_val();
#pragma unroll
        for (int j = 0; j < V; ++j)
            if (id[j] != kNone && key[j] > m) m = key[j];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) m = fmax(m, __shfl_xor(m, off));
        mx = m;
        double s = 0.0;
#pragma unroll
        for (int j = 0; j < V; ++j)
            if (id[j] != kNone) s += exp(key[j] - mx);
        den = wave_sum(s);
    }
    sort_lane<V>(key, score, id);
    if (grouped) {
        const int per = E / a.n_group;
        const int lpg = per / V;  // lanes per group (the launcher checks this path applies)
        const int mygroup = (lane * V) / per;
        // the group's group_topn largest keys, largest first: merge the lanes' sorted
        // top-4 lists pairwise (bitonic: elementwise max against the reversed partner,
        // then a 2-stage half-cleaner)
        double t[kMaxGroupTopn];
#pragma unroll
        for (int j = 0; j < kMaxGroupTopn; ++j) t[j] = j < V ? key[j < V ? j : 0] : -__builtin_huge_val();
        for (int off = 1; off < lpg; off <<= 1) {
            double o[kMaxGroupTopn];
#pragma unroll
            for (int j = 0; j < kMaxGroupTopn; ++j) o[j] = __shfl_xor(t[j], off);
            double c[kMaxGroupTopn];
#pragma unroll
            for (int j = 0; j < kMaxGroupTopn; ++j) c[j] = fmax(t[j], o[kMaxGroupTopn - 1 - j]);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const double hi = fmax(c[j], c[j + 2]), lo = fmin(c[j], c[j + 2]);
                c[j] = hi;
                c[j + 2] = lo;
            }
#pragma unroll
            for (int j = 0; j < 4; j += 2) {
                const double hi = fmax(c[j], c[j + 1]), lo = fmin(c[j], c[j + 1]);
                c[j] = hi;
                c[j + 1] = lo;
            }
#pragma unroll
            for (int j = 0; j < kMaxGroupTopn; ++j) t[j] = c[j];
        }
        double gscore = 0.0;
#pragma unroll
        for (int j = 0; j < kMaxGroupTopn; ++j)
            if (j < a.group_topn) gscore += t[j];
        // rank of this lane's group among all groups (higher score first, ties: lower group)
        int rank = 0;
        for (int q = 0; q < a.n_group; ++q) {
            const double sq = readlane_f64(gscore, q * lpg);
            rank += (sq > gscore || (sq == gscore && q < mygroup)) ? 1 : 0;
        }
        if (rank >= a.topk_group || lane * V >= E) {
#pragma unroll
            for (int j = 0; j < V; ++j) {
                key[j] = -__builtin_huge_val();
                id[j] = kNone;
            }
        }
    }
    // k picks, best first: the wave argmax of the lanes' heads; the owner pops its head
    double my_score = 0.0;
    int my_id = -1;
    for (int t = 0; t < k; ++t) {
        double v = key[0];
        int i = id[0];
        wave_argmax(v, i);
        const int owner = i / V;
        const double sc = readlane_f64(score[0], owner);
        if (lane == owner) {
#pragma unroll
            for (int j = 0; j + 1 < V; ++j) {
                key[j] = key[j + 1];
                score[j] = score[j + 1];
                id[j] = id[j + 1];
            }
            key[V - 1] = -__builtin_huge_val();
            id[V - 1] = kNone;
        }
        if (lane == t) {
            my_score = sc;
            my_id = i;
        }
    }
    const double p = grouped ? my_score : exp(my_score - mx) / den;
    double sum = 0.0;
    for (int t = 0; t < k; ++t) sum += readlane_f64(p, t);  // slot order
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

int lanes_per_expert_chunk(int E) {
    int v = 1;
    while (v * kWave < E) v <<= 1;
    return v;
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
    const int V = lanes_per_expert_chunk(a.E);
    if (a.kind == MOE_ROUTE_GROUPED_SIGMOID) {
        // groups must be whole lanes: per % V == 0, per / V a power of two
        const int per = a.E / a.n_group;
        const int lpg = per / V;
        if (per % V != 0 || lpg < 1 || (lpg & (lpg - 1)) != 0) return MOE_ERR_UNSUPPORTED;
    }
    const dim3 grid(static_cast<unsigned>(ceil_div(G, S_WAVES)));
    switch (V) {
        case 1: hipLaunchKernelGGL(select_kernel<1>, grid, dim3(S_THREADS), 0, stream, a); break;
        case 2: hipLaunchKernelGGL(select_kernel<2>, grid, dim3(S_THREADS), 0, stream, a); break;
        case 4: hipLaunchKernelGGL(select_kernel<4>, grid, dim3(S_THREADS), 0, stream, a); break;
        case 8: hipLaunchKernelGGL(select_kernel<8>, grid, dim3(S_THREADS), 0, stream, a); break;
        default: hipLaunchKernelGGL(select_kernel<16>, grid, dim3(S_THREADS), 0, stream, a); break;
    }
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
