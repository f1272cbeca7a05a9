// Routing: gate logits (op_gate) and top-k selection (op_select_experts) of the SGLang
// walkthrough "SGLang 源码完全拆解(十七): DP Attention 与专家并行", section "operations 与
// yield"; output is the TopKOutput (topk_ids, topk_weights) of section "normal dispatch 的
// 调用链".  The pages do not define the selection arithmetic; the rule implemented is
// DeepSeek-V3's grouped sigmoid with a correction bias (the bias that the "fake" dispatch of
// section "推理时怎么“选副本”" zeroes) and plain softmax top-k.
//
// Exact-order gate.  The integer routing decision depends on the logits bit for bit, so
// the gate fixes one accumulation order (below) and runs it on the fp32 matrix cores, with
// slices of h staged through LDS as fp32 (bf16 widened exactly), double-buffered.
#include <float.h>

#include "gemm_common.h"
#include "moe_dev.h"

namespace moe {
namespace {

// ------------------------------------------------------------------ gate logits
// Exact-order gate.  Reading of the gate's arithmetic (the pages fix none): the plain dot
// product as one chain of fp32 fused multiply-adds in ascending h, starting from +0:
//     acc = +0;  for h = 0 .. H-1:  acc = fmaf(x[g,h], w[e,h], acc)
// Two matrix-core instructions run this chain bit for bit; both were checked against the
// sequential fma chain, and shown to differ from other orders and from a single rounding,
// on full-range fp32, bf16-valued and subnormal operands:
//   - v_mfma_f32_32x32x2f32 adds two products to each accumulator of a 32x32 block per
//     instruction as two fused multiply-adds in sequence, the lower half-wave's k first;
//   - v_mfma_f32_16x16x4f32 adds four products to each accumulator of a 16x16 block as four
//     fused multiply-adds in sequence, lane group 0 (lanes 0-15) first, then 1, 2, 3.
// A chain therefore advances 2 h per 64-cycle instruction on the first and 4 h per 32-cycle
// instruction on the second: whatever the batch, one chain costs at least about 8 cycles
// per h on the 16x16 form.  Large batches use 32x32 chains (fewer LDS reads per flop, x read
// from HBM once per 256 experts); small and medium batches give every wave one 16x16 block
// so that the chains of a small batch spread over as many SIMDs as it has blocks.
// Padding: operand columns past H are staged as x = -0 and w = +0.  Their product is -0,
// and adding -0 leaves every fp32 value in place, +0 and -0 included, so a padded chain has
// the bits of the unpadded one.
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
constexpr int GB_N = 256, GB_K = 32;
constexpr int G_THREADS = 256;
constexpr int G_PAD = 4;

template <typename T>
struct GateIO;

template <>
struct GateIO<uint16_t> {  // bf16 rows; 16-byte piece = 8 k values
    static constexpr int kChunk = 8;
    static constexpr uint16_t kNegZero = 0x8000u;
};
template <>
struct GateIO<float> {  // fp32 rows; 16-byte piece = 4 k values
    static constexpr int kChunk = 4;
    static constexpr float kNegZero = -0.0f;
};

// element t (0..3) of a float4
__device__ __forceinline__ float f4_at(const float4& q, int t) {
    return t == 0 ? q.x : (t == 1 ? q.y : (t == 2 ? q.z : q.w));
}

// 16 bytes of row r starting at column k; columns at or past H read `pad`, rows past `rows`
// read 0 (those rows' outputs are never stored)
template <typename T>
__device__ __forceinline__ uint4 load_piece(const T* __restrict__ src, int64_t rows, int64_t H,
                                            int64_t r, int64_t k, T pad) {
    constexpr int C = GateIO<T>::kChunk;
    uint4 v = {0, 0, 0, 0};
    if (r >= rows) return v;
    const T* p = src + r * H + k;
    T t[C];
#pragma unroll
    for (int q = 0; q < C; ++q) t[q] = (k + q < H) ? p[q] : pad;
    __builtin_memcpy(&v, t, 16);
    return v;
}

typedef unsigned int gate_u32x4 __attribute__((ext_vector_type(4)));

// ---- large batches: 32x32 chains
// Staging of one 32-wide slice of h: x rows [m0, m0+BM) and w rows [n0, n0+256), in LDS as
// fp32 [row][k] with row stride LD, each row split by parity (evens, then odds) so that one
// 16-byte read gives a lane its operands for four consecutive 32x32x2 instructions (lanes
// 0-31 carry the even k of each pair, lanes 32-63 the odd k).  The loads are 16-byte buffer
// loads from descriptors over the block's rows only, so rows past G (or E) read as zeros.
template <typename T, int BM, int NT>
struct GateStage {
    static constexpr int C = GateIO<T>::kChunk;
    static constexpr int LD = GB_K + G_PAD;
    static constexpr int PER_ROW = GB_K / C;  // 16-byte pieces per row
    static constexpr int XCH = BM * PER_ROW / NT;
    static constexpr int WCH = GB_N * PER_ROW / NT;
    static_assert(XCH * NT == BM * PER_ROW && WCH * NT == GB_N * PER_ROW, "whole pieces per thread");
    uint4 xr[XCH], wr[WCH];
    __device__ void load_fast(__amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t rw,
                              const uint32_t (&xoff)[XCH], const uint32_t (&woff)[WCH], int64_t k0) {
        const int so = static_cast<int>(k0 * static_cast<int64_t>(sizeof(T)));
#pragma unroll
        for (int p = 0; p < XCH; ++p) {
            const gate_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rx, static_cast<int>(xoff[p]), so, 0);
            xr[p] = make_uint4(v.x, v.y, v.z, v.w);
        }
#pragma unroll
        for (int p = 0; p < WCH; ++p) {
            const gate_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rw, static_cast<int>(woff[p]), so, 0);
            wr[p] = make_uint4(v.x, v.y, v.z, v.w);
        }
    }
    // slice column k of a row sits at k / 2 (even k) or GB_K / 2 + k / 2 (odd k); `kk` is the
    // piece's first column in the slice
    __device__ static void put(float* row, int kk, const uint4& v) {
        if constexpr (sizeof(T) == 2) {
            reinterpret_cast<float4*>(row + kk / 2)[0] =
                make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.y << 16),
                            __uint_as_float(v.z << 16), __uint_as_float(v.w << 16));
            reinterpret_cast<float4*>(row + GB_K / 2 + kk / 2)[0] =
                make_float4(__uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y & 0xffff0000u),
                            __uint_as_float(v.z & 0xffff0000u), __uint_as_float(v.w & 0xffff0000u));
        } else {
            reinterpret_cast<float2*>(row + kk / 2)[0] = make_float2(__uint_as_float(v.x), __uint_as_float(v.z));
            reinterpret_cast<float2*>(row + GB_K / 2 + kk / 2)[0] =
                make_float2(__uint_as_float(v.y), __uint_as_float(v.w));
        }
    }
    __device__ void store(float* xs, float* ws) {
#pragma unroll
        for (int p = 0; p < XCH; ++p) {
            const int idx = threadIdx.x + p * NT;
            put(xs + (idx / PER_ROW) * LD, (idx % PER_ROW) * C, xr[p]);
        }
#pragma unroll
        for (int p = 0; p < WCH; ++p) {
            const int idx = threadIdx.x + p * NT;
            put(ws + (idx / PER_ROW) * LD, (idx % PER_ROW) * C, wr[p]);
        }
    }
};

// A block of 32 WMR rows x 256 experts with 2 WMR waves, for 16-byte aligned inputs with H
// a multiple of 64: WMR = 4 (128 rows, 8 waves, two per SIMD) for batches that fill the GPU
// with such blocks, WMR = 2 (64 rows, 4 waves) for batches half that size.  Each wave owns
// 32 rows x 128 experts as four 32x32 chains (wave wv: rows 32 (wv / 2), experts 128
// (wv % 2)) that run over all of h.  Slices are loaded from HBM two slices ahead (two
// staging register sets) and the LDS fragments one k-quad ahead.
constexpr int G8_CB = 4;  // 32-expert chains per wave

template <typename T, int WMR>
__global__ __launch_bounds__(128 * WMR, 1) void gate_exact8_kernel(const T* __restrict__ x,
                                                                   const T* __restrict__ w,
                                                                   const int32_t* __restrict__ row_valid,
                                                                   int64_t G, int64_t E, int64_t H,
                                                                   float* __restrict__ logits) {
    constexpr int G8_BM = 32 * WMR;
    constexpr int G8_THREADS = 128 * WMR;
    typedef GateStage<T, G8_BM, G8_THREADS> S;
    constexpr int LD = S::LD;
    __shared__ __attribute__((aligned(16))) float xs[2 * G8_BM * LD];
    __shared__ __attribute__((aligned(16))) float ws[2 * GB_N * LD];
    const int64_t m0 = static_cast<int64_t>(blockIdx.x) * G8_BM;
    const int64_t n0 = static_cast<int64_t>(blockIdx.y) * GB_N;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int wm = wv >> 1, wn = wv & 1;
    const int par = (lane >> 5) * (GB_K / 2);
    const int arow = wm * 32 + (lane & 31);
    const int brow = wn * 128 + (lane & 31);
    const int64_t xrows = G - m0 < G8_BM ? G - m0 : G8_BM;
    const int64_t wrows = E - n0 < GB_N ? E - n0 : GB_N;
    const __amdgpu_buffer_rsrc_t rx =
        gemm::make_rsrc_uniform(x + m0 * H, static_cast<uint32_t>(xrows * H * static_cast<int64_t>(sizeof(T))));
    const __amdgpu_buffer_rsrc_t rw =
        gemm::make_rsrc_uniform(w + n0 * H, static_cast<uint32_t>(wrows * H * static_cast<int64_t>(sizeof(T))));
    uint32_t xoff[S::XCH], woff[S::WCH];
#pragma unroll
    for (int p = 0; p < S::XCH; ++p) {
        const int idx = threadIdx.x + p * G8_THREADS;
        xoff[p] = static_cast<uint32_t>(((idx / S::PER_ROW) * H + (idx % S::PER_ROW) * S::C) * sizeof(T));
    }
#pragma unroll
    for (int p = 0; p < S::WCH; ++p) {
        const int idx = threadIdx.x + p * G8_THREADS;
        woff[p] = static_cast<uint32_t>(((idx / S::PER_ROW) * H + (idx % S::PER_ROW) * S::C) * sizeof(T));
    }
    floatx16_t acc[G8_CB];
#pragma unroll
    for (int c = 0; c < G8_CB; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[c][v] = 0.f;
    // Pipeline.  Slice j is held in staging registers st[j % 2] from the top of slice j - 2
    // (its global loads) to the second half of slice j - 1 (its LDS stores), so a load has a
    // slice and a half to arrive.  Inside a slice the LDS fragments of k-quad kq + 1 are read
    // while the MFMAs of k-quad kq run.
    S st[2];
    const int64_t s_end = H / GB_K;  // even
    st[0].load_fast(rx, rw, xoff, woff, 0);
    st[0].store(xs, ws);
    st[1].load_fast(rx, rw, xoff, woff, GB_K);
    __syncthreads();
    float4 fa[2], fb[2][G8_CB];
    auto read_frag = [&](int buf, int kq, float4& a, float4 (&b)[G8_CB]) {
        const float* xc = xs + buf * (G8_BM * LD) + arow * LD + par + kq * 4;
        const float* wc = ws + buf * (GB_N * LD) + brow * LD + par + kq * 4;
        a = *reinterpret_cast<const float4*>(xc);
#pragma unroll
        for (int cb = 0; cb < G8_CB; ++cb) b[cb] = *reinterpret_cast<const float4*>(wc + cb * 32 * LD);
    };
    // the k-quad's 16 MFMAs: 4 k pairs in order, each over the wave's G8_CB chains
    auto mfma_quad = [&](const float4& a, const float4 (&b)[G8_CB]) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float av = f4_at(a, t);
#pragma unroll
            for (int cb = 0; cb < G8_CB; ++cb)
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, f4_at(b[cb], t), acc[cb], 0, 0, 0);
        }
    };
    read_frag(0, 0, fa[0], fb[0]);
    for (int64_t s2 = 0; s2 < s_end; s2 += 2) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int64_t sl = s2 + q;
            const int cur = q;
            const int64_t n2 = sl + 2 < s_end ? sl + 2 : s_end - 1;
            __builtin_amdgcn_sched_barrier(0);
            st[q].load_fast(rx, rw, xoff, woff, n2 * GB_K);  // slice sl + 2
            read_frag(cur, 1, fa[1], fb[1]);
            mfma_quad(fa[0], fb[0]);
#pragma unroll
            for (int g = 0; g < 1 + G8_CB; ++g) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
                __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);  // then MFMAs
            }
            __builtin_amdgcn_sched_barrier(0);
            read_frag(cur, 2, fa[0], fb[0]);
            mfma_quad(fa[1], fb[1]);
#pragma unroll
            for (int g = 0; g < 1 + G8_CB; ++g) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            read_frag(cur, 3, fa[1], fb[1]);
            st[q ^ 1].store(xs + (cur ^ 1) * (G8_BM * LD), ws + (cur ^ 1) * (GB_N * LD));  // slice sl + 1
            mfma_quad(fa[0], fb[0]);
#pragma unroll
            for (int g = 0; g < 1 + G8_CB; ++g) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // one LDS store
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            mfma_quad(fa[1], fb[1]);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            // k-quad 0 of slice sl + 1 (past the last slice: a stale stage, never used)
            read_frag(cur ^ 1, 0, fa[0], fb[0]);
        }
    }
#pragma unroll
    for (int c = 0; c < G8_CB; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t e = n0 + wn * 128 + 32 * c + (lane & 31);
            const int64_t g = m0 + wm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (g < G && e < E) {
                const bool valid = row_valid == nullptr || row_valid[g] != 0;
                logits[g * E + e] = valid ? acc[c][v] : 0.f;
            }
        }
}

// ---- small and medium batches, and any shape or alignment: 16x16 chains, one per wave
// Each wave owns 16 rows x 16 experts and stages its own operands, so no wave waits for
// another: a block is four independent waves (2 x 2 tiles, neighbours in x and w for the
// L2).  Lane l of a wave holds row (or expert) l % 16 and k group j = l / 16, so instruction
// t needs column 4t + j of its row.  LDS keeps each staged row of a 64-wide slice of h as
// fp32 in [j][t] order (column 4t + j at j * 16 + t, rows C16_RS floats apart): one 16-byte
// read gives a lane its operands for four consecutive instructions.  A wave's LDS accesses
// complete in order, so a slice's stores and the reads that follow them need no barrier.
// A dependent 16x16x4 step takes 32-33 cycles (its issue time), so a slice of 16 steps is
// ~530 cycles while an operand fetch from HBM can take ~1000: slices are loaded C16_D ahead
// into as many register sets, and the stores of the next slice and the reads of its
// fragments are spread between this slice's MFMAs.
constexpr int C16_K = 64;           // h per slice
constexpr int C16_RS = C16_K + 4;   // LDS row stride in floats
constexpr int C16_D = 4;            // slices in flight (register sets), even
constexpr int C16_WAVES = 4;        // independent waves per block, as 2 x 2 tiles

template <typename T>
struct Chain16Stage {
    static constexpr int C = GateIO<T>::kChunk;  // values per 16-byte piece
    static constexpr int PPR = C16_K / C;        // pieces per row and slice
    static constexpr int NP = 16 * PPR / 64;     // pieces per lane for each of x and w
    static_assert(NP * 64 == 16 * PPR, "whole pieces per lane");
    uint4 xr[NP], wr[NP];
    // x rows [m0, m0 + 16) and w rows [n0, n0 + 16) of the slice starting at column k0.
    // FAST: whole slices (H a multiple of C16_K), 16-byte aligned rows; the descriptors
    // cover the wave's own rows, so rows past G (or E) read zeros
    template <bool FAST>
    __device__ void load(__amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t rw, const T* x, const T* w,
                         int64_t G, int64_t E, int64_t H, int64_t m0, int64_t n0, int64_t k0, int lane) {
        if constexpr (FAST) {
            const int so = static_cast<int>(k0 * static_cast<int64_t>(sizeof(T)));
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const int idx = lane + 64 * p;
                const int off = static_cast<int>(((idx / PPR) * H + (idx % PPR) * C) * sizeof(T));
                const gate_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rx, off, so, 0);
                const gate_u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(rw, off, so, 0);
                xr[p] = make_uint4(v.x, v.y, v.z, v.w);
                wr[p] = make_uint4(u.x, u.y, u.z, u.w);
            }
        } else {
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const int idx = lane + 64 * p;
                xr[p] = load_piece<T>(x, G, H, m0 + idx / PPR, k0 + (idx % PPR) * C, GateIO<T>::kNegZero);
                wr[p] = load_piece<T>(w, E, H, n0 + idx / PPR, k0 + (idx % PPR) * C, T(0));
            }
        }
    }
    // piece q of a row covers slice columns q*C .. q*C + C - 1; column c goes to
    // (c % 4) * 16 + c / 4
    __device__ static void put(float* row, int q, const uint4& v) {
        if constexpr (sizeof(T) == 2) {  // columns 8q + u: u and u + 4 share j = u, at t = 2q, 2q + 1
            reinterpret_cast<float2*>(row + 0 * 16 + 2 * q)[0] =
                make_float2(__uint_as_float(v.x << 16), __uint_as_float(v.z << 16));
            reinterpret_cast<float2*>(row + 1 * 16 + 2 * q)[0] =
                make_float2(__uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.z & 0xffff0000u));
            reinterpret_cast<float2*>(row + 2 * 16 + 2 * q)[0] =
                make_float2(__uint_as_float(v.y << 16), __uint_as_float(v.w << 16));
            reinterpret_cast<float2*>(row + 3 * 16 + 2 * q)[0] =
                make_float2(__uint_as_float(v.y & 0xffff0000u), __uint_as_float(v.w & 0xffff0000u));
        } else {  // columns 4q + u: j = u, t = q
            row[0 * 16 + q] = __uint_as_float(v.x);
            row[1 * 16 + q] = __uint_as_float(v.y);
            row[2 * 16 + q] = __uint_as_float(v.z);
            row[3 * 16 + q] = __uint_as_float(v.w);
        }
    }
    // stage layout: x rows 0 .. 15, then w rows 16 .. 31
    __device__ void store(float* stage, int lane) const {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int idx = lane + 64 * p;
            put(stage + (idx / PPR) * C16_RS, idx % PPR, xr[p]);
            put(stage + (16 + idx / PPR) * C16_RS, idx % PPR, wr[p]);
        }
    }
};

template <int Q>
struct SliceIdx {
    static constexpr int kValue = Q;
};

// Slices sl + Q .. sl + D - 1 in order, each with its register set Q fixed at compile time:
// all of them (full), or those before ns (tail).
template <int Q, int D>
struct SliceRun {
    template <typename F>
    __device__ static void full(F& f, int64_t sl) {
        f(SliceIdx<Q>(), sl + Q);
        SliceRun<Q + 1, D>::full(f, sl);
    }
    template <typename F>
    __device__ static void tail(F& f, int64_t sl, int64_t ns) {
        if (sl + Q < ns) {
            f(SliceIdx<Q>(), sl + Q);
            SliceRun<Q + 1, D>::tail(f, sl, ns);
        }
    }
};
template <int D>
struct SliceRun<D, D> {
    template <typename F>
    __device__ static void full(F&, int64_t) {}
    template <typename F>
    __device__ static void tail(F&, int64_t, int64_t) {}
};

// FAST (whole slices, aligned rows) is a template parameter: a run-time branch around the
// loads leaves them in conditional blocks, and the wait counts the compiler then places
// drain every load in flight once per loop trip.
template <typename T, bool FAST>
__global__ __launch_bounds__(64 * C16_WAVES) void gate_chain16_kernel(const T* __restrict__ x,
                                                                     const T* __restrict__ w,
                                                                     const int32_t* __restrict__ row_valid,
                                                                     int64_t G, int64_t E, int64_t H,
                                                                     float* __restrict__ logits) {
    typedef Chain16Stage<T> S;
    constexpr int STAGE = 32 * C16_RS;
    constexpr int D = C16_D;
    static_assert(D % 2 == 0, "the LDS stage of a slice is its register set's parity");
    __shared__ __attribute__((aligned(16))) float lds_all[C16_WAVES * 2 * STAGE];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    float* lds = lds_all + wv * 2 * STAGE;
    const int64_t m0 = static_cast<int64_t>(blockIdx.x) * 32 + (wv >> 1) * 16;
    const int64_t n0 = static_cast<int64_t>(blockIdx.y) * 32 + (wv & 1) * 16;
    if (m0 >= G || n0 >= E) return;  // a wave past the edge has no rows (no block barrier below)
    const int i16 = lane & 15, j = lane >> 4;
    const int64_t xrows = G - m0 < 16 ? G - m0 : 16;
    const int64_t wrows = E - n0 < 16 ? E - n0 : 16;
    // descriptors over the wave's own rows (used by the fast loads only)
    const __amdgpu_buffer_rsrc_t rx =
        gemm::make_rsrc_uniform(x + m0 * H, static_cast<uint32_t>(xrows * H * static_cast<int64_t>(sizeof(T))));
    const __amdgpu_buffer_rsrc_t rw =
        gemm::make_rsrc_uniform(w + n0 * H, static_cast<uint32_t>(wrows * H * static_cast<int64_t>(sizeof(T))));
    // this lane's fragment rows in a stage, at its k group
    const int aoff = i16 * C16_RS + j * 16;
    const int boff = (16 + i16) * C16_RS + j * 16;
    floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
    const int64_t ns = ceil_div(H, C16_K);
    // register set q holds slice q (mod D) from its global loads, issued D slices ahead, to
    // its LDS stores in the slice before
    S st[D];
#pragma unroll
    for (int q = 0; q < D; ++q)
        st[q].template load<FAST>(rx, rw, x, w, G, E, H, m0, n0, (q < ns ? q : ns - 1) * C16_K, lane);
    st[0].store(lds, lane);
    float4 fa[2][4], fb[2][4];
    auto read_frag = [&](int buf, float4 (&a)[4], float4 (&b)[4]) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            a[s] = *reinterpret_cast<const float4*>(lds + buf * STAGE + aoff + 4 * s);
            b[s] = *reinterpret_cast<const float4*>(lds + buf * STAGE + boff + 4 * s);
        }
    };
    // instructions 4s .. 4s+3 of a slice: h = 16 s + 4 u + j for u = 0..3
    auto mfma4 = [&](const float4& a, const float4& b) {
#pragma unroll
        for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(f4_at(a, u), f4_at(b, u), acc, 0, 0, 0);
    };
    read_frag(0, fa[0], fb[0]);
    // slice sl, with Q = sl mod D fixed at compile time: its fragments are in set Q % 2 and
    // its LDS stage is Q % 2.  The chain issues one MFMA per ~44 cycles; the slice's other
    // instructions go between them.
    auto slice = [&](auto QC, int64_t sl) {
        constexpr int Q = decltype(QC)::kValue;
        constexpr int P = Q & 1;
        const int64_t nd = sl + D < ns ? sl + D : ns - 1;
        __builtin_amdgcn_sched_barrier(0);
        st[Q].template load<FAST>(rx, rw, x, w, G, E, H, m0, n0, nd * C16_K, lane);  // slice sl + D
        st[(Q + 1) % D].store(lds + (P ^ 1) * STAGE, lane);  // slice sl + 1 (past the end: never read)
        mfma4(fa[P][0], fb[P][0]);
        mfma4(fa[P][1], fb[P][1]);
        __builtin_amdgcn_sched_barrier(0);
        read_frag(P ^ 1, fa[P ^ 1], fb[P ^ 1]);
        __builtin_amdgcn_sched_barrier(0);
        mfma4(fa[P][2], fb[P][2]);
        mfma4(fa[P][3], fb[P][3]);
        __builtin_amdgcn_sched_barrier(0);
    };
    int64_t sl = 0;
    for (; sl + D <= ns; sl += D) SliceRun<0, D>::full(slice, sl);
    SliceRun<0, D>::tail(slice, sl, ns);
    // lane l, register r: row 4 (l / 16) + r, expert l % 16 of the wave's block
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t g = m0 + 4 * j + r;
        const int64_t e = n0 + i16;
        if (g < G && e < E) {
            const bool valid = row_valid == nullptr || row_valid[g] != 0;
            logits[g * E + e] = valid ? acc[r] : 0.f;
        }
    }
}

// ---- small batches with chains on their own SIMDs
// When a batch has at most one block per CU, each chain's time is the whole kernel's, and a
// dependent 16x16x4 step costs its ~32-cycle issue plus every other instruction the wave
// issues between steps: a vector-ALU or LDS instruction in the MFMA wave's stream is not
// hidden behind the step but adds ~5 cycles to it (measured on this part: 13.4 ns per step
// alone, 22.4 ns with four VALU instructions between steps).  Widening a slice to fp32 and
// storing it takes ~80 such instructions per 16 steps.  So here a block of four waves (one
// per SIMD) has two chain waves, which only read fragments and issue MFMAs, and two helper
// waves, which load each slice from HBM, widen it and store it to the LDS.  The block covers
// 16 rows x 32 experts (chain wave c: experts 16 c .. + 15); the LDS holds three stages of two
// slices, each slice 16 x rows and 32 w rows in the layout of gate_chain16_kernel, and one
// barrier per stage (a handover) passes slices from the helpers to the chains.  The MFMAs see
// the operands and the order of gate_chain16_kernel: the same bits.  At 384 rows and 256
// experts (H = 7168) the kernel takes 35 us against 59 us for gate_chain16_kernel; ~33 cycles
// of its ~42 per step are the MFMA itself, the rest the chains' fragment reads and the LDS and
// memory traffic of the helpers beside them.
constexpr int C16P_STAGES = 3;
constexpr int C16P_SPH = 2;  // slices per handover (stage)
constexpr int C16P_LEAD = 3;  // handovers of helper loads in flight
constexpr int C16P_D = C16P_LEAD * C16P_SPH;  // helper register sets (slice s in set s mod D)
static_assert(C16P_LEAD >= 2, "the prologue fills two stages");

template <typename T, bool FAST>
__global__ __launch_bounds__(256, 1) void gate_chain16p_kernel(const T* __restrict__ x,
                                                               const T* __restrict__ w,
                                                               const int32_t* __restrict__ row_valid,
                                                               int64_t G, int64_t E, int64_t H,
                                                               float* __restrict__ logits) {
    constexpr int C = GateIO<T>::kChunk;      // values per 16-byte piece
    constexpr int PPR = C16_K / C;            // pieces per row and slice (8 bf16, 16 fp32)
    constexpr int RPI = 64 / PPR;             // rows per load instruction (8, 4)
    constexpr int NI = (16 + 32) / RPI / 2;   // load instructions per helper and slice (3, 6)
    constexpr int XI = 16 / RPI;              // the first XI instructions of the block are x rows
    constexpr int ROWS = 48;                  // stage rows: 16 x, then 32 w
    constexpr int STAGE = ROWS * C16_RS;      // one slice
    __shared__ __attribute__((aligned(16))) float lds[C16P_STAGES * C16P_SPH * STAGE];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int64_t m0 = static_cast<int64_t>(blockIdx.x) * 16;
    const int64_t n0 = static_cast<int64_t>(blockIdx.y) * 32;
    const int64_t ns = ceil_div(H, C16_K);
    const int64_t nh = ceil_div(ns, C16P_SPH);  // handovers
    const bool helper = wv >= 2;
    // LDS slot of slice s: stage (s / SPH) mod 3, position s mod SPH in it
    auto slot = [](int64_t s) {
        return static_cast<int>(((s / C16P_SPH) % C16P_STAGES) * C16P_SPH + s % C16P_SPH);
    };

    // ---- helper state: instruction q of this helper is block instruction hq = NI (wv - 2) + q,
    // rows RPI hq .. + RPI - 1 of the stage (x rows first, then w rows)
    const int64_t xrows = G - m0 < 16 ? G - m0 : 16;
    const int64_t wrows = E - n0 < 32 ? E - n0 : 32;
    const __amdgpu_buffer_rsrc_t rx = gemm::make_rsrc_uniform(
        x + m0 * H, static_cast<uint32_t>((xrows > 0 ? xrows : 0) * H * static_cast<int64_t>(sizeof(T))));
    const __amdgpu_buffer_rsrc_t rw = gemm::make_rsrc_uniform(
        w + n0 * H, static_cast<uint32_t>((wrows > 0 ? wrows : 0) * H * static_cast<int64_t>(sizeof(T))));
    const int prow = lane / PPR, ppiece = lane % PPR;  // this lane's row in an instruction, piece
    uint4 reg[C16P_D][NI];
    // a slice past the last is staged as x = -0, w = +0: each of its steps adds a -0
    // product, which leaves every accumulator's bits in place, so the chains run it blindly
    const uint32_t xpad = sizeof(T) == 2 ? 0x80008000u : 0x80000000u;
    auto hload = [&](int set, int64_t sl) {
        // slices past the last re-read the last one (no branch around the loads: the
        // compiler's wait counts would then drain every load in flight once per loop trip);
        // hstore writes the padding in their place
        const int64_t k0 = (sl < ns ? sl : ns - 1) * C16_K;
#pragma unroll
        for (int q = 0; q < NI; ++q) {
            const int hq = NI * (wv - 2) + q;
            const bool isx = hq < XI;
            const int r = (isx ? hq : hq - XI) * RPI + prow;  // row within x (0..15) or w (0..31)
            if constexpr (FAST) {
                const int off = static_cast<int>((r * H + ppiece * C) * static_cast<int64_t>(sizeof(T)));
                const int so = static_cast<int>(k0 * static_cast<int64_t>(sizeof(T)));
                const gate_u32x4 v = isx ? __builtin_amdgcn_raw_buffer_load_b128(rx, off, so, 0)
                                         : __builtin_amdgcn_raw_buffer_load_b128(rw, off, so, 0);
                reg[set][q] = make_uint4(v.x, v.y, v.z, v.w);
            } else {
                reg[set][q] = isx ? load_piece<T>(x, G, H, m0 + r, k0 + ppiece * C, GateIO<T>::kNegZero)
                                  : load_piece<T>(w, E, H, n0 + r, k0 + ppiece * C, T(0));
            }
        }
    };
    auto hstore = [&](int set, int sslot, int64_t sl) {
        const uint32_t keep = sl < ns ? 0xffffffffu : 0u;
#pragma unroll
        for (int q = 0; q < NI; ++q) {
            const int hq = NI * (wv - 2) + q;
            const int srow = hq * RPI + prow;  // slice rows: x rows 0..15, w rows 16..47
            const uint32_t pad = (hq < XI ? xpad : 0u) & ~keep;
            const uint4 r = reg[set][q];
            const uint4 v = make_uint4((r.x & keep) | pad, (r.y & keep) | pad, (r.z & keep) | pad,
                                       (r.w & keep) | pad);
            Chain16Stage<T>::put(lds + sslot * STAGE + srow * C16_RS, ppiece, v);
        }
    };

    // ---- chain state: lane (i16, j) of chain wave c, as in gate_chain16_kernel
    const int c = wv & 1;
    const int i16 = lane & 15, j = lane >> 4;
    const int aoff = i16 * C16_RS + j * 16;
    const int boff = (16 + 16 * c + i16) * C16_RS + j * 16;
    floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
    float4 fa[2][4], fb[2][4];
    auto read_frag = [&](int sslot, float4 (&a)[4], float4 (&b)[4]) {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            a[s4] = *reinterpret_cast<const float4*>(lds + sslot * STAGE + aoff + 4 * s4);
            b[s4] = *reinterpret_cast<const float4*>(lds + sslot * STAGE + boff + 4 * s4);
        }
    };
    auto mfma16 = [&](const float4 (&a)[4], const float4 (&b)[4]) {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
            for (int u = 0; u < 4; ++u)
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(f4_at(a[s4], u), f4_at(b[s4], u), acc, 0, 0, 0);
    };

    // the barrier that hands slices over: the helpers' stores are in the LDS (and the chains'
    // reads done) before it; a plain barrier, since a block-wide fence would also drain the
    // helpers' loads in flight
    auto handover = [&]() {
        __builtin_amdgcn_sched_barrier(0);  // a slice's MFMAs stay before its barrier
        // lgkmcnt(0) (vmcnt and expcnt left at their maxima), as a builtin so that the
        // compiler's own wait counts know every LDS access before it is done
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        // no work of one slice moves across a handover (the widening of a later slice's
        // registers would otherwise be hoisted and wait for loads still in flight)
        __builtin_amdgcn_sched_barrier(0);
    };
    // The two roles run separate loops (so that the compiler's wait counts see each role's
    // loads alone) with the same barriers: one after the prologue, one per handover of
    // SPH = 2 slices.  Slice s sits in register set s mod D (D = 6 = 3 handovers) and in LDS
    // slot slot(s); handover h stores slices 2h + 4, 2h + 5 (the stage read last in handover
    // h - 1) and runs slices 2h, 2h + 1.
    if (helper) {
        // prologue: slices 0 .. 3 stored (handovers 0, 1), slices 4 .. 9 in flight
#pragma unroll
        for (int q = 0; q < C16P_D; ++q) hload(q, q);
#pragma unroll
        for (int q = 0; q < 2 * C16P_SPH; ++q) {
            hstore(q, slot(q), q);
            hload(q, q + C16P_D);
        }
        handover();
        int stg = 2;  // stage of handover h + 2 (32-bit counters: the loop's scalar work counts)
        auto hstep = [&](auto QC, int64_t h) {
            // set of slice 2h + 4 (h mod LEAD is QC)
            constexpr int base = ((decltype(QC)::kValue + 2) % C16P_LEAD) * C16P_SPH;
#pragma unroll
            for (int i = 0; i < C16P_SPH; ++i) {
                const int64_t sl = C16P_SPH * (h + 2) + i;
                hstore(base + i, stg * C16P_SPH + i, sl);
                hload(base + i, sl + C16P_D);
            }
            stg = stg == C16P_STAGES - 1 ? 0 : stg + 1;
            handover();
        };
        int64_t h = 0;
        for (; h + C16P_LEAD <= nh; h += C16P_LEAD) SliceRun<0, C16P_LEAD>::full(hstep, h);
        SliceRun<0, C16P_LEAD>::tail(hstep, h, nh);
        return;
    }
    handover();
    read_frag(slot(0), fa[0], fb[0]);
    // slice 0's fragments in place before the loop: at every loop entry no LDS read is then
    // outstanding, so the wait counts the compiler places in the loop stay off its MFMAs
    __builtin_amdgcn_s_waitcnt(0xC07F);
    // Handover h reads the fragments of slices 2h + 1 and 2h + 2 (stages h and h + 1, both
    // stored before its barrier) at its start, then runs the steps of slice 2h (read in
    // handover h - 1) and of slice 2h + 1.  Reading everything at the start keeps the chains'
    // LDS reads apart from the helpers' stores, which come once their loads land: reading
    // slice 2h + 2 after slice 2h's steps instead took the decode route from 46 to 52 us.
    // Slice 2h + 2 lands in the set slice 2h used on odd h and in fa2 on even h, so the loop
    // runs handovers in pairs; slices past the last are padding (see xpad), so the body is
    // straight-line code.
    float4 fa2[4], fb2[4];
    int stg = 0;  // stage of handover h
    auto step = [&](auto PAR) {
        constexpr bool odd = decltype(PAR)::value;
        const int nxt = stg == C16P_STAGES - 1 ? 0 : stg + 1;
        // all of the handover's reads at its start: slice 2h + 1, and slice 2h + 2 for the next
        read_frag(stg * C16P_SPH + 1, fa[1], fb[1]);
        if (odd) read_frag(nxt * C16P_SPH, fa[0], fb[0]);
        else read_frag(nxt * C16P_SPH, fa2, fb2);
        __builtin_amdgcn_sched_barrier(0);
        if (odd) mfma16(fa2, fb2);
        else mfma16(fa[0], fb[0]);
        __builtin_amdgcn_sched_barrier(0);
        mfma16(fa[1], fb[1]);
        stg = nxt;
        handover();
    };
    int h = 0;
    for (; h + 2 <= static_cast<int>(nh); h += 2) {
        step(std::false_type());
        step(std::true_type());
    }
    if (h < static_cast<int>(nh)) step(std::false_type());
    // lane l, register r: row 4 (l / 16) + r, expert l % 16 of the wave's block
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t g = m0 + 4 * j + r;
        const int64_t e = n0 + 16 * c + i16;
        if (g < G && e < E) {
            const bool valid = row_valid == nullptr || row_valid[g] != 0;
            logits[g * E + e] = valid ? acc[r] : 0.f;
        }
    }
}

// ------------------------------------------------------------------ fast gate
// FAST mode: logits on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulate).
// Products of bf16 values are exact in fp32, so only the summation order differs from the
// exact gate.  A block computes 128 rows x 256 experts (x read from HBM once), 4 waves of
// 64 x 128 (eight 32x32 accumulators each), 64-deep K slices staged through LDS as bf16
// with rows padded to 144 bytes (16 consecutive rows of a 16-byte fragment read land on
// distinct bank groups); the next slice is loaded into registers while this one computes.
typedef __bf16 gate_bf16x8_t __attribute__((ext_vector_type(8)));
constexpr int FB_M = 128, FB_N = 256, FB_K = 64, FB_LD = FB_K + 8;

struct FastStage {
    static constexpr int PER_ROW = FB_K / 8;                 // 16-byte pieces per row
    static constexpr int XCH = FB_M * PER_ROW / G_THREADS;   // 4
    static constexpr int WCH = FB_N * PER_ROW / G_THREADS;   // 8
    uint4 xr[XCH], wr[WCH];
    __device__ void load(const uint16_t* x, const uint16_t* w, __amdgpu_buffer_rsrc_t rx,
                         __amdgpu_buffer_rsrc_t rw, bool fast, int64_t G, int64_t E, int64_t H,
                         int64_t m0, int64_t n0, int64_t k0) {
        if (fast && k0 + FB_K <= H) {
            const int so = static_cast<int>(k0 * 2);
#pragma unroll
            for (int p = 0; p < XCH; ++p) {
                const int idx = threadIdx.x + p * G_THREADS;
                const uint32_t off = static_cast<uint32_t>(((idx / PER_ROW) * H + (idx % PER_ROW) * 8) * 2);
                const gate_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rx, static_cast<int>(off), so, 0);
                xr[p] = make_uint4(v.x, v.y, v.z, v.w);
            }
#pragma unroll
            for (int p = 0; p < WCH; ++p) {
                const int idx = threadIdx.x + p * G_THREADS;
                const uint32_t off = static_cast<uint32_t>(((idx / PER_ROW) * H + (idx % PER_ROW) * 8) * 2);
                const gate_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rw, static_cast<int>(off), so, 0);
                wr[p] = make_uint4(v.x, v.y, v.z, v.w);
            }
        } else {
#pragma unroll
            for (int p = 0; p < XCH; ++p) {
                const int idx = threadIdx.x + p * G_THREADS;
                xr[p] = load_piece<uint16_t>(x, G, H, m0 + idx / PER_ROW, k0 + (idx % PER_ROW) * 8, 0);
            }
#pragma unroll
            for (int p = 0; p < WCH; ++p) {
                const int idx = threadIdx.x + p * G_THREADS;
                wr[p] = load_piece<uint16_t>(w, E, H, n0 + idx / PER_ROW, k0 + (idx % PER_ROW) * 8, 0);
            }
        }
    }
    __device__ void store(uint16_t* xs, uint16_t* ws) {
#pragma unroll
        for (int p = 0; p < XCH; ++p) {
            const int idx = threadIdx.x + p * G_THREADS;
            *reinterpret_cast<uint4*>(xs + (idx / PER_ROW) * FB_LD + (idx % PER_ROW) * 8) = xr[p];
        }
#pragma unroll
        for (int p = 0; p < WCH; ++p) {
            const int idx = threadIdx.x + p * G_THREADS;
            *reinterpret_cast<uint4*>(ws + (idx / PER_ROW) * FB_LD + (idx % PER_ROW) * 8) = wr[p];
        }
    }
};

__global__ __launch_bounds__(G_THREADS) void gate_fast_kernel(const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ w,
                                                              const int32_t* __restrict__ row_valid,
                                                              int64_t G, int64_t E, int64_t H, bool fast,
                                                              float* __restrict__ logits) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][FB_M * FB_LD];
    __shared__ __attribute__((aligned(16))) uint16_t ws[2][FB_N * FB_LD];
    const int64_t m0 = static_cast<int64_t>(blockIdx.x) * FB_M;
    const int64_t n0 = static_cast<int64_t>(blockIdx.y) * FB_N;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int wm = wv >> 1, wn = wv & 1;
    const int64_t xrows = G - m0 < FB_M ? G - m0 : FB_M;
    const int64_t wrows = E - n0 < FB_N ? E - n0 : FB_N;
    const __amdgpu_buffer_rsrc_t rx = gemm::make_rsrc_uniform(x + m0 * H, static_cast<uint32_t>(xrows * H * 2));
    const __amdgpu_buffer_rsrc_t rw = gemm::make_rsrc_uniform(w + n0 * H, static_cast<uint32_t>(wrows * H * 2));
    floatx16_t acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[c][v] = 0.f;
    // fragment reads: row lane%32 of each 32-row block, k 8*(lane/32) .. +8 of each 16-deep step
    const int arow = wm * 64 + (lane & 31), brow = wn * 128 + (lane & 31);
    const int kof = (lane >> 5) * 8;
    const int64_t KT = ceil_div(H, FB_K);
    FastStage st;
    st.load(x, w, rx, rw, fast, G, E, H, m0, n0, 0);
    st.store(xs[0], ws[0]);
    __syncthreads();
    for (int64_t kt = 0; kt < KT; ++kt) {
        const int cur = static_cast<int>(kt & 1);
        const bool more = kt + 1 < KT;
        if (more) st.load(x, w, rx, rw, fast, G, E, H, m0, n0, (kt + 1) * FB_K);
        const uint16_t* xa = xs[cur] + arow * FB_LD + kof;
        const uint16_t* wb = ws[cur] + brow * FB_LD + kof;
#pragma unroll
        for (int ks = 0; ks < FB_K / 16; ++ks) {
            gate_bf16x8_t fa[2], fb[4];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) fa[rb] = *reinterpret_cast<const gate_bf16x8_t*>(xa + rb * 32 * FB_LD + ks * 16);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) fb[cb] = *reinterpret_cast<const gate_bf16x8_t*>(wb + cb * 32 * FB_LD + ks * 16);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int cb = 0; cb < 4; ++cb)
                    acc[rb * 4 + cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[rb], fb[cb], acc[rb * 4 + cb], 0, 0, 0);
        }
        if (more) st.store(xs[cur ^ 1], ws[cur ^ 1]);
        __syncthreads();
    }
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            // accumulator c = 4 rb + cb, register v: row block rb, expert block cb
            const int64_t e = n0 + wn * 128 + 32 * (c & 3) + (lane & 31);
            const int64_t g = m0 + wm * 64 + 32 * (c >> 2) + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (g < G && e < E) {
                const bool valid = row_valid == nullptr || row_valid[g] != 0;
                logits[g * E + e] = valid ? acc[c][v] : 0.f;
            }
        }
}

// The same tile and the same K order (so the same logits) for H a multiple of 64 with 16-byte
// aligned rows: 64-deep slices DMA'd straight into the LDS (`buffer_load ... lds`, whole
// 128-byte lines per row and slice; the token rows, read once, with the non-temporal hint)
// through three stages, two slices in flight, one barrier per slice.  The register-staged
// form above keeps one slice in flight, which bounds its rate at ~21 GB/s per CU.  LDS rows
// are 128 bytes with chunk c of row r stored at c xor ((r / 2) mod 8), so a fragment read (16
// consecutive rows, one 16-byte chunk each) touches 16 distinct 16-byte slots of 256 bytes.
// Eight waves, two per SIMD: waves 0-3 run the MFMAs of the 128 x 256 tile (64 x 128 each)
// and waves 4-7 issue every DMA.  A vector-memory instruction in a wave that streams MFMAs
// costs it tens of cycles of matrix-core time, and each slice takes 48 of them; a wave beside
// it on the same SIMD issues them at little cost to the MFMAs.
constexpr int FD_STAGES = 3;
constexpr int FD_THREADS = 512;
constexpr int FD_CPR = FB_K / 8;                     // 16-byte chunks per row (8)
constexpr int FD_RPB = 64 / FD_CPR;                  // rows per 1 KB DMA block (8)
constexpr int FD_XDMA = FB_M / FD_RPB / 4;           // token-row DMAs per DMA wave and slice (4)
constexpr int FD_WDMA = FB_N / FD_RPB / 4;           // weight-row DMAs per DMA wave and slice (8)
constexpr int FD_VPS = FD_XDMA + FD_WDMA;
__device__ __forceinline__ int fd_swz(int row) { return (row >> 1) & 7; }

__global__ __launch_bounds__(FD_THREADS, 1) void gate_fast_dma_kernel(const uint16_t* __restrict__ x,
                                                                      const uint16_t* __restrict__ w,
                                                                      const int32_t* __restrict__ row_valid,
                                                                      int64_t G, int64_t E, int64_t H,
                                                                      float* __restrict__ logits) {
    __shared__ __attribute__((aligned(1024))) uint16_t xs[FD_STAGES][FB_M * FB_K];
    __shared__ __attribute__((aligned(1024))) uint16_t ws[FD_STAGES][FB_N * FB_K];
    const int64_t m0 = static_cast<int64_t>(blockIdx.x) * FB_M;
    const int64_t n0 = static_cast<int64_t>(blockIdx.y) * FB_N;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int64_t KT = H / FB_K;
    if (wv >= 4) {
        // ---- DMA wave d = wv - 4: the DMAs the four waves of a 4-wave block would split
        const int d = wv - 4;
        const int64_t xrows = G - m0 < FB_M ? G - m0 : FB_M;
        const int64_t wrows = E - n0 < FB_N ? E - n0 : FB_N;
        const uint32_t row_bytes = static_cast<uint32_t>(H) * 2u;
        // rows past G or E fall outside the resources and read as zeros
        const __amdgpu_buffer_rsrc_t rx = gemm::make_rsrc_uniform(x + m0 * H, static_cast<uint32_t>(xrows) * row_bytes);
        const __amdgpu_buffer_rsrc_t rw = gemm::make_rsrc_uniform(w + n0 * H, static_cast<uint32_t>(wrows) * row_bytes);
        // DMA p: token rows 32 d + 8 p + lane / 8, weight rows 64 d + 8 p + lane / 8; the global
        // chunk (lane mod 8) xor swizzle, whose value depends on p only through p mod 2
        const int dr = lane / FD_CPR;
        const int xr0 = 32 * d + dr, wr0 = 64 * d + dr;
        uint32_t xoff[2], woff[2];
#pragma unroll
        for (int par = 0; par < 2; ++par) {
            xoff[par] = static_cast<uint32_t>(xr0) * row_bytes + static_cast<uint32_t>(((lane % FD_CPR) ^ fd_swz(xr0 + 8 * par)) * 16);
            woff[par] = static_cast<uint32_t>(wr0) * row_bytes + static_cast<uint32_t>(((lane % FD_CPR) ^ fd_swz(wr0 + 8 * par)) * 16);
        }
        const uint32_t rstep = static_cast<uint32_t>(FD_RPB) * row_bytes;
        auto issue = [&](int stage, int64_t kt) {
            gemm::lds_void_t* xd = (gemm::lds_void_t*)(&xs[0][0] + stage * (FB_M * FB_K) + d * FD_XDMA * 512);
            gemm::lds_void_t* wd = (gemm::lds_void_t*)(&ws[0][0] + stage * (FB_N * FB_K) + d * FD_WDMA * 512);
            uint32_t x0 = xoff[0], x1 = xoff[1], w0 = woff[0], w1 = woff[1];
            asm volatile("" : "+s"(xd), "+s"(wd), "+v"(x0), "+v"(x1), "+v"(w0), "+v"(w1));
            const int so = static_cast<int>(kt * FB_K * 2);
#pragma unroll
            for (int p = 0; p < FD_XDMA; ++p)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rx, (gemm::lds_void_t*)((char __attribute__((address_space(3)))*)xd + p * 1024), 16,
                    ((p & 1) ? x1 : x0) + static_cast<uint32_t>(p) * rstep, so, 0, 2 /* non-temporal */);
#pragma unroll
            for (int p = 0; p < FD_WDMA; ++p)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rw, (gemm::lds_void_t*)((char __attribute__((address_space(3)))*)wd + p * 1024), 16,
                    ((p & 1) ? w1 : w0) + static_cast<uint32_t>(p) * rstep, so, 0, 0);
        };
        auto clamp = [&](int64_t kt) { return kt < KT ? kt : KT - 1; };
        // slice s goes to stage s mod 3; one barrier before the loop (slice 0 landed), then
        // one per slice kt (slice kt + 1 landed), after which slice kt's stage is refilled:
        // the MFMA waves read it before that barrier
        issue(0, 0);
        issue(1, clamp(1));
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(FD_VPS) : "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue(2, clamp(2));
        int st = 0;  // stage of slice kt
        for (int64_t kt = 0; kt < KT; ++kt) {
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(FD_VPS) : "memory");  // slice kt + 2 in flight
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            issue(st, clamp(kt + 3));
            st = st == FD_STAGES - 1 ? 0 : st + 1;
        }
        // no DMA into LDS may outlive the workgroup
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        return;
    }
    // ---- MFMA wave: 64 rows (wm) x 128 experts (wn) of the tile
    const int wm = wv >> 1, wn = wv & 1;
    floatx16_t acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[c][v] = 0.f;
    // fragment reads: row lane mod 32 of each 32-row block, logical chunk 2 ks + lane / 32 of
    // each 16-deep step (the K order of gate_fast_kernel)
    const int fr = lane & 31;
    int fch[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) fch[ks] = ((2 * ks + (lane >> 5)) ^ fd_swz(fr)) * 8;
    // k steps 0, 1 of a slice sit in fragment set 0, steps 2, 3 in set 1
    gate_bf16x8_t fa[2][2][2], fb[2][2][4];
    auto read = [&](int stage, int set) {
        const uint16_t* xa = &xs[0][0] + stage * (FB_M * FB_K) + (wm * 64 + fr) * FB_K;
        const uint16_t* wb = &ws[0][0] + stage * (FB_N * FB_K) + (wn * 128 + fr) * FB_K;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int ks = 2 * set + h;
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) fa[set][h][rb] = *reinterpret_cast<const gate_bf16x8_t*>(xa + rb * 32 * FB_K + fch[ks]);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) fb[set][h][cb] = *reinterpret_cast<const gate_bf16x8_t*>(wb + cb * 32 * FB_K + fch[ks]);
        }
    };
    auto mfma = [&](int set) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int cb = 0; cb < 4; ++cb)
                    acc[rb * 4 + cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][h][rb], fb[set][h][cb], acc[rb * 4 + cb], 0, 0, 0);
    };
    // the barrier that pairs with the DMA waves': this wave's reads are done before it (the
    // DMA waves refill a stage it read after it); the compiler's own wait counts see the wait
    auto barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    // Each slice's fragment reads run under the MFMAs of the half slice before them: steps 2, 3
    // of slice kt under steps 0, 1, and, after the barrier that finds slice kt + 1 landed,
    // steps 0, 1 of slice kt + 1 under steps 2, 3 of slice kt.  The MFMA order per
    // accumulator is that of gate_fast_kernel.
    barrier();
    read(0, 0);
    int st = 0;  // stage of slice kt
    for (int64_t kt = 0; kt < KT; ++kt) {
        const int nx = st == FD_STAGES - 1 ? 0 : st + 1;
        read(st, 1);
        __builtin_amdgcn_sched_barrier(0);
        mfma(0);
        barrier();
        read(nx, 0);
        __builtin_amdgcn_sched_barrier(0);
        mfma(1);
        st = nx;
    }
    // the lane's 32 rows (row block rb, register v): their flags first, in one batch of loads
    // (rows past G load row G - 1's flag, unused), then keep = -1 past G, else the flag
    int keep[2][16];
    if (row_valid != nullptr) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t g = m0 + wm * 64 + 32 * rb + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                keep[rb][v] = row_valid[g < G ? g : G - 1];
            }
    } else {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int v = 0; v < 16; ++v) keep[rb][v] = 1;
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t g = m0 + wm * 64 + 32 * rb + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            keep[rb][v] = g >= G ? -1 : keep[rb][v] != 0 ? 1 : 0;
        }
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            // accumulator c = 4 rb + cb, register v: row block rb, expert block cb
            const int64_t e = n0 + wn * 128 + 32 * (c & 3) + (lane & 31);
            const int64_t g = m0 + wm * 64 + 32 * (c >> 2) + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            const int k = keep[c >> 2][v];
            if (k >= 0 && e < E) logits[g * E + e] = k ? acc[c][v] : 0.f;
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

// 32-bit code of a head for the fast pick: the key rounded to fp32 (round to nearest is
// monotone, so a strictly larger code means a strictly larger fp64 key), -0 folded into +0
// (they are equal keys), mapped to an unsigned integer that orders like the float; 0 for an
// empty head.  Equal codes fall back to the exact (key, id) order.
__device__ __forceinline__ uint32_t head_code(double k, int id) {
    if (id == kNone) return 0u;
    float f = static_cast<float>(k);
    if (f == 0.0f) f = 0.0f;
    const uint32_t b = __float_as_uint(f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// wave maximum of an unsigned value, as a scalar: within each 16-lane row by DPP (the quad
// butterflies, then the half-row and row mirrors), then the four row maxima
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    auto step = [](uint32_t x, uint32_t y) { return x > y ? x : y; };
    v = step(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
    v = step(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
    v = step(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0x141, 0xF, 0xF, false)));
    v = step(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0x140, 0xF, 0xF, false)));
    const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    return step(step(r0, r1), step(r2, r3));
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

// up to 256 experts (V <= 4) the kernel fits 64 registers without spilling, and eight waves
// per SIMD instead of six took the prefill select (32768 rows, 256 experts) from ~74 to ~65 us;
// wider rows keep the compiler's default
template <int V>
__global__ __launch_bounds__(S_THREADS) __attribute__((amdgpu_waves_per_eu(V <= 4 ? 8 : 1)))
void select_kernel(SelectArgs a) {
    const int lane = lane_id();
    const int64_t g = static_cast<int64_t>(blockIdx.x) * S_WAVES + threadIdx.x / kWave;
    if (g >= a.G) return;  // no block barrier below
    const int E = a.E, k = a.k;
    int32_t* ids = a.ids + g * k;
    float* wout = a.w + g * k;
    const bool pad = a.row_valid && a.row_valid[g] == 0;
    float lv[V];
#pragma unroll
    for (int j = 0; j < V; ++j) lv[j] = lane * V + j < E ? a.logits[g * E + lane * V + j] : 0.f;
    if (pad) {  // pad row: no expert load
        if (lane < k) {
            ids[lane] = -1;
            wout[lane] = 0.f;
        }
        return;
    }
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
            const double l = static_cast<double>(lv[j]);
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
    // k picks, best first: the best of the lanes' heads, whose owner pops it.  The heads'
    // 32-bit codes find it in one wave maximum; only when several heads share the largest
    // code does the exact (key, id) argmax run among them.
    double my_score = 0.0;
    int my_id = -1;
    for (int t = 0; t < k; ++t) {
        const uint32_t code = head_code(key[0], id[0]);
        const uint32_t top = wave_max_u32(code);
        const uint64_t cand = __ballot(code == top);
        int i;
        if (__popcll(cand) == 1) {
            i = __builtin_amdgcn_readlane(id[0], __ffsll(static_cast<long long>(cand)) - 1);
        } else {
            const bool in = (cand >> lane) & 1ull;
            double v = in ? key[0] : -__builtin_huge_val();
            i = in ? id[0] : kNone;
            wave_argmax(v, i);
        }
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
    MOE_CHECK_ARG(c->gate_mode == MOE_GATE_EXACT || c->gate_mode == MOE_GATE_FAST);
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
    // the select launch (one wave per row) has the most work-items per row of any route launch
    if (!moe::grid_fits(moe::ceil_div(G, moe::S_WAVES), moe::S_THREADS)) return MOE_ERR_UNSUPPORTED;
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
    if (cfg->gate_mode == MOE_GATE_FAST && dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (G == 0) return MOE_OK;
    MOE_CHECK_ARG(global_x && w_router && logits && topk_ids && topk_w);
    MOE_CHECK_ARG(G <= (int64_t)1 << 31);
    // the select launch (one wave per row) has the most work-items per row of any route launch
    if (!moe::grid_fits(moe::ceil_div(G, moe::S_WAVES), moe::S_THREADS)) return MOE_ERR_UNSUPPORTED;
    const int64_t E = cfg->num_experts;
    const int64_t esz = dt == MOE_BF16 ? 2 : 4;
    const bool aligned = moe::aligned(global_x, 16) && moe::aligned(w_router, 16) && (H * esz) % 16 == 0;
    // A batch is large when its 128-row (or 64-row) x 256-expert blocks fill every CU (one
    // block holds a CU's LDS); smaller batches spread 16x16 chains instead.  FAST mode on a
    // batch too small for its 128-row tiles to cover half the CUs takes the exact gate: its
    // few tiles would run the whole of h in sequence on part of the GPU, and the exact
    // logits are the better ones anyway.
    const int64_t ncu = moe::stream_cus(stream);
    const int64_t etiles = moe::ceil_div(E, moe::GB_N);
    const bool fills128 = moe::ceil_div(G, 128) * etiles >= ncu;
    const bool fills64 = moe::ceil_div(G, 64) * etiles >= ncu;
    const bool exact32 = aligned && H % (2 * moe::GB_K) == 0 &&
                         static_cast<int64_t>(moe::GB_N) * H * esz < ((int64_t)1 << 31);
    const bool fast_large = moe::ceil_div(G, moe::FB_M) * moe::ceil_div(E, moe::FB_N) * 2 >= ncu;
    if (cfg->gate_mode == MOE_GATE_FAST && fast_large) {
        const bool fast = aligned && static_cast<int64_t>(moe::FB_N) * H * 2 < ((int64_t)1 << 31);
        const dim3 grid(static_cast<unsigned>(moe::ceil_div(G, moe::FB_M)),
                        static_cast<unsigned>(moe::ceil_div(E, moe::FB_N)));
        if (fast && H % moe::FB_K == 0)
            hipLaunchKernelGGL(moe::gate_fast_dma_kernel, grid, dim3(moe::FD_THREADS), 0, stream,
                               static_cast<const uint16_t*>(global_x), static_cast<const uint16_t*>(w_router),
                               row_valid, G, E, H, logits);
        else
            hipLaunchKernelGGL(moe::gate_fast_kernel, grid, dim3(moe::G_THREADS), 0, stream,
                               static_cast<const uint16_t*>(global_x), static_cast<const uint16_t*>(w_router),
                               row_valid, G, E, H, fast, logits);
    } else if (exact32 && (fills128 || fills64)) {
        // 32x32 chains; the kernel's descriptors span up to 256 rows, which must stay below
        // 2 GiB
        const int rows = fills128 ? 128 : 64;
        const dim3 grid(static_cast<unsigned>(moe::ceil_div(G, rows)), static_cast<unsigned>(etiles));
        const uint16_t* xb = static_cast<const uint16_t*>(global_x);
        const uint16_t* wb = static_cast<const uint16_t*>(w_router);
        const float* xf = static_cast<const float*>(global_x);
        const float* wf = static_cast<const float*>(w_router);
        if (dt == MOE_BF16 && fills128)
            hipLaunchKernelGGL((moe::gate_exact8_kernel<uint16_t, 4>), grid, dim3(512), 0, stream, xb, wb, row_valid,
                               G, E, H, logits);
        else if (dt == MOE_BF16)
            hipLaunchKernelGGL((moe::gate_exact8_kernel<uint16_t, 2>), grid, dim3(256), 0, stream, xb, wb, row_valid,
                               G, E, H, logits);
        else if (fills128)
            hipLaunchKernelGGL((moe::gate_exact8_kernel<float, 4>), grid, dim3(512), 0, stream, xf, wf, row_valid, G,
                               E, H, logits);
        else
            hipLaunchKernelGGL((moe::gate_exact8_kernel<float, 2>), grid, dim3(256), 0, stream, xf, wf, row_valid, G,
                               E, H, logits);
    } else if (moe::ceil_div(G, 16) * moe::ceil_div(E, 32) <= ncu) {
        // at most one block per CU: chains on their own SIMDs, fed by helper waves
        const dim3 grid(static_cast<unsigned>(moe::ceil_div(G, 16)), static_cast<unsigned>(moe::ceil_div(E, 32)));
        const bool fast = aligned && H % moe::C16_K == 0 && 32 * H * esz < ((int64_t)1 << 31);
        const uint16_t* xb = static_cast<const uint16_t*>(global_x);
        const uint16_t* wb = static_cast<const uint16_t*>(w_router);
        const float* xf = static_cast<const float*>(global_x);
        const float* wf = static_cast<const float*>(w_router);
        if (dt == MOE_BF16 && fast)
            hipLaunchKernelGGL((moe::gate_chain16p_kernel<uint16_t, true>), grid, dim3(256), 0, stream, xb, wb,
                               row_valid, G, E, H, logits);
        else if (dt == MOE_BF16)
            hipLaunchKernelGGL((moe::gate_chain16p_kernel<uint16_t, false>), grid, dim3(256), 0, stream, xb, wb,
                               row_valid, G, E, H, logits);
        else if (fast)
            hipLaunchKernelGGL((moe::gate_chain16p_kernel<float, true>), grid, dim3(256), 0, stream, xf, wf,
                               row_valid, G, E, H, logits);
        else
            hipLaunchKernelGGL((moe::gate_chain16p_kernel<float, false>), grid, dim3(256), 0, stream, xf, wf,
                               row_valid, G, E, H, logits);
    } else {
        const dim3 grid(static_cast<unsigned>(moe::ceil_div(G, 32)), static_cast<unsigned>(moe::ceil_div(E, 32)));
        // whole 64-wide slices and aligned rows take 16-byte buffer loads, whose per-wave
        // descriptors span 16 rows; anything else loads element by element
        const bool fast = aligned && H % moe::C16_K == 0 && 16 * H * esz < ((int64_t)1 << 31);
        const uint16_t* xb = static_cast<const uint16_t*>(global_x);
        const uint16_t* wb = static_cast<const uint16_t*>(w_router);
        const float* xf = static_cast<const float*>(global_x);
        const float* wf = static_cast<const float*>(w_router);
        const dim3 block(64 * moe::C16_WAVES);
        if (dt == MOE_BF16 && fast)
            hipLaunchKernelGGL((moe::gate_chain16_kernel<uint16_t, true>), grid, block, 0, stream, xb, wb, row_valid,
                               G, E, H, logits);
        else if (dt == MOE_BF16)
            hipLaunchKernelGGL((moe::gate_chain16_kernel<uint16_t, false>), grid, block, 0, stream, xb, wb, row_valid,
                               G, E, H, logits);
        else if (fast)
            hipLaunchKernelGGL((moe::gate_chain16_kernel<float, true>), grid, block, 0, stream, xf, wf, row_valid, G,
                               E, H, logits);
        else
            hipLaunchKernelGGL((moe::gate_chain16_kernel<float, false>), grid, block, 0, stream, xf, wf, row_valid,
                               G, E, H, logits);
    }
    MOE_LAUNCH_CHECK();
    return moe::launch_select(logits, row_valid, G, bias, cfg, topk_ids, topk_w, stream);
}
