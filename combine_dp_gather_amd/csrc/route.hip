// Routing: gate logits (op_gate) and top-k selection (op_select_experts) of the SGLang
// walkthrough "SGLang 源码完全拆解(十七): DP Attention 与专家并行", section "operations 与
// yield"; output is the TopKOutput (topk_ids, topk_weights) of section "normal dispatch 的
// 调用链".  The pages do not define the selection arithmetic; the rule implemented is
// DeepSeek-V3's grouped sigmoid with a correction bias (the bias that the "fake" dispatch of
// section "推理时怎么“选副本”" zeroes) and plain softmax top-k.
//
// Exact-order gate.  The integer routing decision depends on the logits bit for bit, so
// the gate fixes one accumulation order (below) and runs it on the fp32 matrix cores, with
// 32-deep K slices staged through LDS as fp32 (bf16 widened exactly), double-buffered.
#include <float.h>

#include "gemm_common.h"
#include "moe_dev.h"

namespace moe {
namespace {

// ------------------------------------------------------------------ gate logits
// Exact-order gate.  Reading of the gate's arithmetic (the pages fix none): fp32 fused
// multiply-adds in ascending h inside each 128-wide chunk of h, starting from +0; the chunk
// sums are added left to right to a running fp32 total starting from +0.
//
// On the matrix cores: v_mfma_f32_32x32x2f32 adds two products to each 32x32 accumulator
// per instruction as two fused multiply-adds in sequence (the lower half-wave's k first), each
// with one rounding -- bit for bit the fmaf chain of the definition (checked against the
// sequential fma chain, and shown to differ from a single-rounding pair, on bf16-valued and
// full fp32 operands).  Lanes 0-31 therefore carry the even k of each pair and lanes 32-63
// the odd k; LDS keeps every row's slice split by parity (evens, then odds) so that one
// 16-byte read gives a lane its operands for four consecutive instructions.  A wave owns
// 32*RB rows x 128 experts as 4*RB 32x32 chains (RB row blocks x 4 expert blocks).
//   - large batches: a block of 64*RB rows x 256 experts (x read from HBM once) walks all
//     of h in 32-wide slices, prefetching across chunk boundaries; after a chunk's last slice
//     its sums are added to the running total and the chains restart from +0.  RB = 1 (64
//     rows) when those blocks fit in one round on the CUs, else RB = 2 (128 rows), so a
//     batch of half the prefill size still fills the chip;
//   - small batches: one block per (row tile, expert tile, chunk) writes the chunk's sums to
//     a workspace and the top-k kernel adds them left to right as it reads them -- chunks
//     run in parallel, so the latency is one chunk's chain, not the whole row's.
// Zero operands past H (ragged last chunk) change nothing: a chain started at +0 never holds
// -0, so adding a +-0 product leaves every bit in place.
typedef float floatx16_t __attribute__((ext_vector_type(16)));
constexpr int GATE_CHUNK = 128;
constexpr int GB_M = 128, GB_N = 256, GB_K = 32, G_THREADS = 256;
constexpr int G_PAD = 4;
constexpr int SLICES_PER_CHUNK = GATE_CHUNK / GB_K;
static_assert(GATE_CHUNK % GB_K == 0, "a slice never straddles two chunks");

template <typename T>
struct GateIO;

template <>
struct GateIO<uint16_t> {  // bf16 rows; 16-byte piece = 8 k values
    static constexpr int kChunk = 8;
    typedef uint2 Quad;  // 4 consecutive k
    __device__ static float val(const Quad& q, int t) {
        const uint32_t w = t < 2 ? q.x : q.y;
        return __uint_as_float((t & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};
template <>
struct GateIO<float> {  // fp32 rows; 16-byte piece = 4 k values
    static constexpr int kChunk = 4;
    typedef float4 Quad;
    __device__ static float val(const Quad& q, int t) {
        return t == 0 ? q.x : (t == 1 ? q.y : (t == 2 ? q.z : q.w));
    }
};

// 16 bytes of row r starting at column k; columns at or past H (or rows past `rows`) are 0
template <typename T>
__device__ __forceinline__ uint4 load_piece(const T* __restrict__ src, int64_t rows, int64_t H,
                                            int64_t r, int64_t k) {
    constexpr int C = GateIO<T>::kChunk;
    uint4 v = {0, 0, 0, 0};
    if (r >= rows || k >= H) return v;
    const T* p = src + r * H + k;
    T t[C];
#pragma unroll
    for (int q = 0; q < C; ++q) t[q] = (k + q < H) ? p[q] : T(0);
    __builtin_memcpy(&v, t, 16);
    return v;
}

typedef unsigned int gate_u32x4 __attribute__((ext_vector_type(4)));

// Staging of one slice: x rows [m0, m0+BM) and w rows [n0, n0+256), columns k0 .. k0+GB_K,
// in LDS as [row][k] with row stride LD.  The fast load is a 16-byte buffer load per piece
// from a descriptor over the block's rows only, so rows past G (or E) read as zeros; the
// element-wise load covers a slice that runs past H and unaligned inputs.
template <typename T, int BM = GB_M, int NT = G_THREADS>
struct GateStage {
    static constexpr int C = GateIO<T>::kChunk;
    static constexpr int LD = GB_K + G_PAD;
    static constexpr int PER_ROW = GB_K / C;  // 16-byte pieces per row
    static constexpr int XCH = BM * PER_ROW / NT;
    static constexpr int WRITES = (XCH + GB_N * PER_ROW / NT) * 2;  // LDS stores per thread
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
    __device__ void load_slow(const T* x, const T* w, int64_t G, int64_t E,
                              int64_t H, int64_t m0, int64_t n0, int64_t k0) {
#pragma unroll
        for (int p = 0; p < XCH; ++p) {
            const int idx = threadIdx.x + p * NT;
            xr[p] = load_piece(x, G, H, m0 + idx / PER_ROW, k0 + (idx % PER_ROW) * C);
        }
#pragma unroll
        for (int p = 0; p < WCH; ++p) {
            const int idx = threadIdx.x + p * NT;
            wr[p] = load_piece(w, E, H, n0 + idx / PER_ROW, k0 + (idx % PER_ROW) * C);
        }
    }
    // LDS holds fp32 (bf16 widens here, once per element) split by parity: slice column k
    // of a row sits at k / 2 (even k) or GB_K / 2 + k / 2 (odd k).  `kk` is the piece's
    // first column in the slice.
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

// Chunks [ch0, ch1) of h for the block's 128 x 256 tile (chunk c = slices 4c .. 4c+3, slice
// s = columns 32s .. 32s+31).  Each chunk's chains start from +0 and see only matrix-core
// adds, so they stay in the accumulator registers; with TOTAL the chunk's sums are then
// added to `total`, else (a single chunk) they are left in acc.  `fast` (block-uniform): the
// inputs are 16-byte aligned with rows a multiple of 16 bytes.
template <typename T, bool TOTAL, int RB = 2>
__device__ __forceinline__ void gate_chunks(const T* x, const T* w, int64_t G, int64_t E, int64_t H,
                                            int64_t m0, int64_t n0, int64_t ch0, int64_t ch1,
                                            bool fast, float* xs, float* ws, floatx16_t (&acc)[4 * RB],
                                            floatx16_t (&total)[4 * RB]) {
    constexpr int BM = 64 * RB;
    typedef GateStage<T, BM> S;
    typedef typename GateIO<float>::Quad Quad;
    constexpr int LD = S::LD;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int wm = wv >> 1, wn = wv & 1;
    // lane's operand rows: x rows wm*32*RB + 32 rb + lane%32, w rows wn*128 + 32 cb + lane%32;
    // its k parity (lane / 32) picks the even or odd half of the row
    const int par = (lane >> 5) * (GB_K / 2);
    const int arow = wm * 32 * RB + (lane & 31);
    const int brow = wn * 128 + (lane & 31);
    // descriptors over the block's own rows: byte offsets stay below 256 * H * sizeof(T)
    const int64_t xrows = G - m0 < BM ? G - m0 : BM;
    const int64_t wrows = E - n0 < GB_N ? E - n0 : GB_N;
    const __amdgpu_buffer_rsrc_t rx =
        gemm::make_rsrc_uniform(x + m0 * H, static_cast<uint32_t>(xrows * H * static_cast<int64_t>(sizeof(T))));
    const __amdgpu_buffer_rsrc_t rw =
        gemm::make_rsrc_uniform(w + n0 * H, static_cast<uint32_t>(wrows * H * static_cast<int64_t>(sizeof(T))));
    uint32_t xoff[S::XCH], woff[S::WCH];
#pragma unroll
    for (int p = 0; p < S::XCH; ++p) {
        const int idx = threadIdx.x + p * G_THREADS;
        xoff[p] = static_cast<uint32_t>(((idx / S::PER_ROW) * H + (idx % S::PER_ROW) * S::C) * sizeof(T));
    }
#pragma unroll
    for (int p = 0; p < S::WCH; ++p) {
        const int idx = threadIdx.x + p * G_THREADS;
        woff[p] = static_cast<uint32_t>(((idx / S::PER_ROW) * H + (idx % S::PER_ROW) * S::C) * sizeof(T));
    }
    S st;
    const int64_t s_begin = ch0 * SLICES_PER_CHUNK, s_end = ch1 * SLICES_PER_CHUNK;
    auto load = [&](int64_t sl) {
        const int64_t k0 = sl * GB_K;
        if (fast && k0 + GB_K <= H)
            st.load_fast(rx, rw, xoff, woff, k0);
        else
            st.load_slow(x, w, G, E, H, m0, n0, k0);
    };
    load(s_begin);
    st.store(xs, ws);
    __syncthreads();
    for (int64_t ch = ch0; ch < ch1; ++ch) {
#pragma unroll
        for (int c = 0; c < 4 * RB; ++c)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[c][v] = 0.f;
#pragma unroll 1
        for (int q = 0; q < SLICES_PER_CHUNK; ++q) {
            const int64_t sl = ch * SLICES_PER_CHUNK + q;
            const int cur = static_cast<int>((sl - s_begin) & 1);
            const float* xc = xs + cur * (BM * LD) + arow * LD + par;
            const float* wc = ws + cur * (GB_N * LD) + brow * LD + par;
            const bool more = sl + 1 < s_end;
            if (more) load(sl + 1);
#pragma unroll
            for (int kq = 0; kq < GB_K / 8; ++kq) {  // four k pairs per 16-byte read
                float4 qa[RB], qb[4];
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) qa[rb] = *reinterpret_cast<const float4*>(xc + rb * 32 * LD + kq * 4);
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) qb[cb] = *reinterpret_cast<const float4*>(wc + cb * 32 * LD + kq * 4);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) {
                        const float av = GateIO<float>::val(qa[rb], t);
#pragma unroll
                        for (int cb = 0; cb < 4; ++cb)
                            acc[rb * 4 + cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                                av, GateIO<float>::val(qb[cb], t), acc[rb * 4 + cb], 0, 0, 0);
                    }
                }
            }
            if (more) st.store(xs + (cur ^ 1) * (BM * LD), ws + (cur ^ 1) * (GB_N * LD));
            __syncthreads();
        }
        if (TOTAL) {
#pragma unroll
            for (int c = 0; c < 4 * RB; ++c)
#pragma unroll
                for (int v = 0; v < 16; ++v) total[c][v] = total[c][v] + acc[c][v];
        }
    }
}

// Fast path of gate_chunks: 16-byte aligned inputs and H a multiple of the chunk width, so
// every slice is whole.  The slice loop has no branches (the last slice re-stages itself into
// the idle buffer, which nothing reads), the refill's global loads are issued at the top of
// a slice, and its LDS stores are spread between the MFMAs of the slice's second half: with
// one wave per SIMD the matrix pipe keeps issuing while the next slice is staged.  Each
// chain's MFMAs keep their k order, so the bits are those of gate_chunks.
template <typename T, bool TOTAL, int RB>
__device__ __forceinline__ void gate_chunks_pipe(const T* x, const T* w, int64_t G, int64_t E, int64_t H,
                                                 int64_t m0, int64_t n0, int64_t ch0, int64_t ch1,
                                                 float* xs, float* ws, floatx16_t (&acc)[4 * RB],
                                                 floatx16_t (&total)[4 * RB]) {
    constexpr int BM = 64 * RB;
    typedef GateStage<T, BM> S;
    constexpr int LD = S::LD;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int wm = wv >> 1, wn = wv & 1;
    const int par = (lane >> 5) * (GB_K / 2);
    const int arow = wm * 32 * RB + (lane & 31);
    const int brow = wn * 128 + (lane & 31);
    const int64_t xrows = G - m0 < BM ? G - m0 : BM;
    const int64_t wrows = E - n0 < GB_N ? E - n0 : GB_N;
    const __amdgpu_buffer_rsrc_t rx =
        gemm::make_rsrc_uniform(x + m0 * H, static_cast<uint32_t>(xrows * H * static_cast<int64_t>(sizeof(T))));
    const __amdgpu_buffer_rsrc_t rw =
        gemm::make_rsrc_uniform(w + n0 * H, static_cast<uint32_t>(wrows * H * static_cast<int64_t>(sizeof(T))));
    uint32_t xoff[S::XCH], woff[S::WCH];
#pragma unroll
    for (int p = 0; p < S::XCH; ++p) {
        const int idx = threadIdx.x + p * G_THREADS;
        xoff[p] = static_cast<uint32_t>(((idx / S::PER_ROW) * H + (idx % S::PER_ROW) * S::C) * sizeof(T));
    }
#pragma unroll
    for (int p = 0; p < S::WCH; ++p) {
        const int idx = threadIdx.x + p * G_THREADS;
        woff[p] = static_cast<uint32_t>(((idx / S::PER_ROW) * H + (idx % S::PER_ROW) * S::C) * sizeof(T));
    }
    // the second half of a slice issues 2 * 4 * RB * 4 MFMAs; spread the stores over them
    constexpr int HALF_MFMA = 32 * RB;
    constexpr int PER_STORE = HALF_MFMA / S::WRITES > 0 ? HALF_MFMA / S::WRITES : 1;
    S st;
    const int64_t s_end = ch1 * SLICES_PER_CHUNK;
    st.load_fast(rx, rw, xoff, woff, ch0 * SLICES_PER_CHUNK * GB_K);
    st.store(xs, ws);
    __syncthreads();
    static_assert(SLICES_PER_CHUNK % 2 == 0, "the stage of a slice is its index inside the chunk, mod 2");
    for (int64_t ch = ch0; ch < ch1; ++ch) {
#pragma unroll
        for (int c = 0; c < 4 * RB; ++c)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[c][v] = 0.f;
#pragma unroll
        for (int q = 0; q < SLICES_PER_CHUNK; ++q) {
            const int64_t sl = ch * SLICES_PER_CHUNK + q;
            const int cur = q & 1;
            const int64_t nxt = sl + 1 < s_end ? sl + 1 : sl;
            const float* xc = xs + cur * (BM * LD) + arow * LD + par;
            const float* wc = ws + cur * (GB_N * LD) + brow * LD + par;
            __builtin_amdgcn_sched_barrier(0);
            st.load_fast(rx, rw, xoff, woff, nxt * GB_K);
            // four k pairs per 16-byte read of each operand row
#define MOE_GATE_KQ(KQ)                                                                         \
    do {                                                                                        \
        float4 qa[RB], qb[4];                                                                   \
        _Pragma("unroll") for (int rb = 0; rb < RB; ++rb) qa[rb] =                              \
            *reinterpret_cast<const float4*>(xc + rb * 32 * LD + (KQ) * 4);                     \
        _Pragma("unroll") for (int cb = 0; cb < 4; ++cb) qb[cb] =                               \
            *reinterpret_cast<const float4*>(wc + cb * 32 * LD + (KQ) * 4);                     \
        _Pragma("unroll") for (int t = 0; t < 4; ++t)                                           \
            _Pragma("unroll") for (int rb = 0; rb < RB; ++rb) {                                 \
                const float av = GateIO<float>::val(qa[rb], t);                                 \
                _Pragma("unroll") for (int cb = 0; cb < 4; ++cb) acc[rb * 4 + cb] =             \
                    __builtin_amdgcn_mfma_f32_32x32x2f32(av, GateIO<float>::val(qb[cb], t),     \
                                                         acc[rb * 4 + cb], 0, 0, 0);            \
            }                                                                                   \
    } while (0)
            MOE_GATE_KQ(0);
            MOE_GATE_KQ(1);
            __builtin_amdgcn_sched_barrier(0);
            st.store(xs + (cur ^ 1) * (BM * LD), ws + (cur ^ 1) * (GB_N * LD));
            MOE_GATE_KQ(2);
            MOE_GATE_KQ(3);
#undef MOE_GATE_KQ
#pragma unroll
            for (int g = 0; g < S::WRITES; ++g) {
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);          // one LDS store
                __builtin_amdgcn_sched_group_barrier(0x008, PER_STORE, 0);  // then MFMAs
            }
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
        }
        if (TOTAL) {
#pragma unroll
            for (int c = 0; c < 4 * RB; ++c)
#pragma unroll
                for (int v = 0; v < 16; ++v) total[c][v] = total[c][v] + acc[c][v];
        }
    }
}

// out[g, e] for the lane's accumulator element (chain c = 4 rb + cb, register v)
template <int RB = 2>
__device__ __forceinline__ void chain_coords(int c, int v, int lane, int64_t m0, int64_t n0, int64_t& g,
                                             int64_t& e) {
    const int wv = threadIdx.x >> 6, wm = wv >> 1, wn = wv & 1;
    e = n0 + wn * 128 + 32 * (c & 3) + (lane & 31);
    g = m0 + wm * 32 * RB + 32 * (c >> 2) + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

// large batches: all chunks in one block of 64*RB rows, running total in registers
template <typename T, int RB>
__global__ __launch_bounds__(G_THREADS) void gate_exact_kernel(const T* __restrict__ x,
                                                               const T* __restrict__ w,
                                                               const int32_t* __restrict__ row_valid,
                                                               int64_t G, int64_t E, int64_t H,
                                                               bool fast, float* __restrict__ logits) {
    constexpr int BM = 64 * RB;
    constexpr int LD = GateStage<T, BM>::LD;
    __shared__ __attribute__((aligned(16))) float xs[2 * BM * LD];
    __shared__ __attribute__((aligned(16))) float ws[2 * GB_N * LD];
    const int64_t m0 = static_cast<int64_t>(blockIdx.x) * BM;
    const int64_t n0 = static_cast<int64_t>(blockIdx.y) * GB_N;
    const int lane = threadIdx.x & 63;
    floatx16_t acc[4 * RB], total[4 * RB];
#pragma unroll
    for (int c = 0; c < 4 * RB; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) total[c][v] = 0.f;
    if (fast && H % GATE_CHUNK == 0)
        gate_chunks_pipe<T, true, RB>(x, w, G, E, H, m0, n0, 0, H / GATE_CHUNK, xs, ws, acc, total);
    else  // the last chunk may be ragged: its columns past H read zeros, which add +0 products
        gate_chunks<T, true, RB>(x, w, G, E, H, m0, n0, 0, ceil_div(H, GATE_CHUNK), fast, xs, ws, acc, total);
#pragma unroll
    for (int c = 0; c < 4 * RB; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            int64_t g, e;
            chain_coords<RB>(c, v, lane, m0, n0, g, e);
            if (g < G && e < E) {
                const bool valid = row_valid == nullptr || row_valid[g] != 0;
                logits[g * E + e] = valid ? total[c][v] : 0.f;
            }
        }
}

// Large batches with whole chunks and aligned inputs: the same 128-row x 256-expert block
// with 8 waves, two per SIMD.  Each wave owns 32 rows x 128 experts as four 32x32 chains
// (wave wv: rows 32 (wv / 2), experts 128 (wv % 2)), so a wave needs half the accumulator
// registers of the 4-wave block and its SIMD partner issues MFMAs while it waits on LDS
// reads, staging or the slice barrier.  Slices are loaded from HBM two slices ahead and the
// LDS fragments one k-quad ahead; the per-chain k order is that of gate_chunks_pipe, so the
// bits are the same.
constexpr int G8_THREADS = 512;
constexpr int G8_BM = 128;
constexpr int G8_CB = 4;  // 32-expert chains per wave

template <typename T>
__global__ __launch_bounds__(G8_THREADS, 1) void gate_exact8_kernel(const T* __restrict__ x,
                                                                    const T* __restrict__ w,
                                                                    const int32_t* __restrict__ row_valid,
                                                                    int64_t G, int64_t E, int64_t H,
                                                                    float* __restrict__ logits) {
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
    floatx16_t acc[G8_CB], total[G8_CB];
#pragma unroll
    for (int c = 0; c < G8_CB; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) total[c][v] = 0.f;
    // Pipeline.  Slice j is held in staging registers st[j % 2] from the top of slice j - 2
    // (its global loads) to the second half of slice j - 1 (its LDS stores), so a load has a
    // slice and a half to arrive.  Inside a slice the LDS fragments of k-quad kq + 1 are read
    // while the MFMAs of k-quad kq run.
    S st[2];
    const int64_t nch = H / GATE_CHUNK;
    const int64_t s_end = nch * SLICES_PER_CHUNK;
    st[0].load_fast(rx, rw, xoff, woff, 0);
    st[0].store(xs, ws);
    st[1].load_fast(rx, rw, xoff, woff, (s_end > 1 ? 1 : 0) * GB_K);
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
            const float av = GateIO<float>::val(a, t);
#pragma unroll
            for (int cb = 0; cb < G8_CB; ++cb)
                acc[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, GateIO<float>::val(b[cb], t), acc[cb], 0, 0, 0);
        }
    };
    read_frag(0, 0, fa[0], fb[0]);
    for (int64_t ch = 0; ch < nch; ++ch) {
#pragma unroll
        for (int c = 0; c < G8_CB; ++c)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[c][v] = 0.f;
#pragma unroll
        for (int q = 0; q < SLICES_PER_CHUNK; ++q) {
            const int64_t sl = ch * SLICES_PER_CHUNK + q;
            const int cur = q & 1;
            const int64_t n2 = sl + 2 < s_end ? sl + 2 : s_end - 1;
            __builtin_amdgcn_sched_barrier(0);
            st[q & 1].load_fast(rx, rw, xoff, woff, n2 * GB_K);  // slice sl + 2
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
            st[(q + 1) & 1].store(xs + (cur ^ 1) * (G8_BM * LD), ws + (cur ^ 1) * (GB_N * LD));  // slice sl + 1
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
#pragma unroll
        for (int c = 0; c < G8_CB; ++c)
#pragma unroll
            for (int v = 0; v < 16; ++v) total[c][v] = total[c][v] + acc[c][v];
    }
#pragma unroll
    for (int c = 0; c < G8_CB; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t e = n0 + wn * 128 + 32 * c + (lane & 31);
            const int64_t g = m0 + wm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (g < G && e < E) {
                const bool valid = row_valid == nullptr || row_valid[g] != 0;
                logits[g * E + e] = valid ? total[c][v] : 0.f;
            }
        }
}

// small batches: blockIdx.z = chunk; writes the chunk's sums to parts[chunk][G][E]
template <typename T>
__global__ __launch_bounds__(G_THREADS) void gate_chunk_kernel(const T* __restrict__ x,
                                                               const T* __restrict__ w, int64_t G,
                                                               int64_t E, int64_t H, bool fast,
                                                               float* __restrict__ parts) {
    constexpr int LD = GateStage<T>::LD;
    __shared__ __attribute__((aligned(16))) float xs[2 * GB_M * LD];
    __shared__ __attribute__((aligned(16))) float ws[2 * GB_N * LD];
    const int64_t m0 = static_cast<int64_t>(blockIdx.x) * GB_M;
    const int64_t n0 = static_cast<int64_t>(blockIdx.y) * GB_N;
    const int64_t ch = blockIdx.z;
    const int lane = threadIdx.x & 63;
    floatx16_t acc[8], unused[8];
    gate_chunks<T, false>(x, w, G, E, H, m0, n0, ch, ch + 1, fast, xs, ws, acc, unused);
    float* out = parts + ch * G * E;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            int64_t g, e;
            chain_coords(c, v, lane, m0, n0, g, e);
            if (g < G && e < E) out[g * E + e] = acc[c][v];
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
                xr[p] = load_piece(x, G, H, m0 + idx / PER_ROW, k0 + (idx % PER_ROW) * 8);
            }
#pragma unroll
            for (int p = 0; p < WCH; ++p) {
                const int idx = threadIdx.x + p * G_THREADS;
                wr[p] = load_piece(w, E, H, n0 + idx / PER_ROW, k0 + (idx % PER_ROW) * 8);
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
            int64_t g, e;
            chain_coords(c, v, lane, m0, n0, g, e);
            if (g < G && e < E) {
                const bool valid = row_valid == nullptr || row_valid[g] != 0;
                logits[g * E + e] = valid ? acc[c][v] : 0.f;
            }
        }
}

int gate_num_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            v = 256;
        cus[dev] = v;
    }
    return cus[dev];
}

// workspace the chunk-parallel gate needs; 0 when the batch is large enough for the
// running-total kernel to fill the GPU
size_t gate_split_bytes(int64_t G, int64_t E, int64_t H) {
    const int64_t tiles = ceil_div(G, GB_M) * ceil_div(E, GB_N);
    if (tiles * 2 >= gate_num_cus()) return 0;
    return static_cast<size_t>(ceil_div(H, GATE_CHUNK) * G * E) * sizeof(float);
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
    // small-batch exact gate: the chunk partial sums [nchunks][G][E]; the kernel then adds
    // them in chunk order (the logits' definition) and writes the logits itself
    const float* parts;
    int64_t nchunks;
    float* logits_out;
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
    const bool pad = a.row_valid && a.row_valid[g] == 0;
    float lv[V];
    if (a.parts) {
        // logits = ((+0 + part_0) + part_1) + ... in chunk order; pad rows get 0
        const int64_t GE = a.G * E;
        const float* pp = a.parts + g * E + lane * V;
#pragma unroll
        for (int j = 0; j < V; ++j) lv[j] = 0.f;
        if (!pad) {
            bool done = false;
            if constexpr (V == 4) {
                if ((E & 3) == 0) {  // 16-byte loads: every offset is a multiple of 4 floats
                    if (lane * V < E) {
                        // kLoads loads in flight, then their adds in chunk order
                        constexpr int kLoads = 8;
                        int64_t c = 0;
                        for (; c + kLoads <= a.nchunks; c += kLoads) {
                            float4 q[kLoads];
#pragma unroll
                            for (int u = 0; u < kLoads; ++u)
                                q[u] = *reinterpret_cast<const float4*>(pp + (c + u) * GE);
#pragma unroll
                            for (int u = 0; u < kLoads; ++u) {
                                lv[0] = lv[0] + q[u].x;
                                lv[1] = lv[1] + q[u].y;
                                lv[2] = lv[2] + q[u].z;
                                lv[3] = lv[3] + q[u].w;
                            }
                        }
                        for (; c < a.nchunks; ++c) {
                            const float4 q = *reinterpret_cast<const float4*>(pp + c * GE);
                            lv[0] = lv[0] + q.x;
                            lv[1] = lv[1] + q.y;
                            lv[2] = lv[2] + q.z;
                            lv[3] = lv[3] + q.w;
                        }
                    }
                    done = true;
                }
            }
            if (!done)
                for (int64_t c = 0; c < a.nchunks; ++c)
#pragma unroll
                    for (int j = 0; j < V; ++j)
                        if (lane * V + j < E) lv[j] = lv[j] + pp[c * GE + j];
        }
#pragma unroll
        for (int j = 0; j < V; ++j)
            if (lane * V + j < E) a.logits_out[g * E + lane * V + j] = lv[j];
    } else {
#pragma unroll
        for (int j = 0; j < V; ++j) lv[j] = lane * V + j < E ? a.logits[g * E + lane * V + j] : 0.f;
    }
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
                         hipStream_t stream, const float* parts = nullptr, int64_t nchunks = 0) {
    SelectArgs a;
    a.logits = logits;
    a.parts = parts;
    a.nchunks = nchunks;
    a.logits_out = const_cast<float*>(logits);
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

extern "C" size_t moe_route_workspace_size(int64_t G, int32_t num_experts, int64_t H) {
    if (G <= 0 || num_experts <= 0 || H <= 0) return 0;
    return moe::gate_split_bytes(G, num_experts, H);
}

extern "C" moe_status moe_route(const void* global_x, const int32_t* row_valid, int64_t G,
                                int64_t H, moe_dtype dt, const void* w_router, const float* bias,
                                const moe_route_cfg* cfg, float* logits, int32_t* topk_ids,
                                float* topk_w, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
    moe_status st = moe::check_route_cfg(cfg);
    if (st != MOE_OK) return st;
    MOE_CHECK_ARG(G >= 0 && H > 0);
    MOE_CHECK_ARG(dt == MOE_F32 || dt == MOE_BF16);
    if (G == 0) return MOE_OK;
    MOE_CHECK_ARG(global_x && w_router && logits && topk_ids && topk_w);
    MOE_CHECK_ARG(G <= (int64_t)1 << 31);
    const int64_t E = cfg->num_experts;
    const size_t split = moe::gate_split_bytes(G, E, H);
    const bool use_split = split > 0 && workspace != nullptr && workspace_bytes >= split &&
                           moe::aligned(workspace, 16);
    // FAST mode on a batch small enough for the chunk-parallel exact gate takes that gate:
    // it is faster there (a handful of 128-row tiles would run the whole of h in sequence),
    // and its logits are the exact ones
    if (cfg->gate_mode == MOE_GATE_FAST && dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (cfg->gate_mode == MOE_GATE_FAST && !use_split) {
        const bool fast = moe::aligned(global_x, 16) && moe::aligned(w_router, 16) && (H * 2) % 16 == 0 &&
                          static_cast<int64_t>(moe::FB_N) * H * 2 < ((int64_t)1 << 31);
        const dim3 grid(static_cast<unsigned>(moe::ceil_div(G, moe::FB_M)),
                        static_cast<unsigned>(moe::ceil_div(E, moe::FB_N)));
        hipLaunchKernelGGL(moe::gate_fast_kernel, grid, dim3(moe::G_THREADS), 0, stream,
                           static_cast<const uint16_t*>(global_x), static_cast<const uint16_t*>(w_router),
                           row_valid, G, E, H, fast, logits);
        MOE_LAUNCH_CHECK();
        return moe::launch_select(logits, row_valid, G, bias, cfg, topk_ids, topk_w, stream);
    }
    const dim3 tiles(static_cast<unsigned>(moe::ceil_div(G, moe::GB_M)),
                     static_cast<unsigned>(moe::ceil_div(E, moe::GB_N)));
    // 64-row blocks when they all fit in one round on the CUs (a 64-row block takes a bit
    // over half a 128-row block's time), else 128-row blocks
    const dim3 tiles64(static_cast<unsigned>(moe::ceil_div(G, 64)), tiles.y);
    const bool rows128 = static_cast<int64_t>(tiles64.x) * tiles64.y > moe::gate_num_cus();
    // 16-byte buffer loads need aligned bases and rows; the per-block descriptors span at
    // most 256 rows, which must stay below 2 GiB
    const size_t esz = dt == MOE_BF16 ? 2 : 4;
    const bool fast = moe::aligned(global_x, 16) && moe::aligned(w_router, 16) && (H * esz) % 16 == 0 &&
                      static_cast<int64_t>(moe::GB_N) * H * static_cast<int64_t>(esz) < ((int64_t)1 << 31);
    if (use_split) {
        const int64_t nch = moe::ceil_div(H, moe::GATE_CHUNK);
        const dim3 grid(tiles.x, tiles.y, static_cast<unsigned>(nch));
        float* parts = static_cast<float*>(workspace);
        if (dt == MOE_BF16)
            hipLaunchKernelGGL(moe::gate_chunk_kernel<uint16_t>, grid, dim3(moe::G_THREADS), 0, stream,
                               static_cast<const uint16_t*>(global_x), static_cast<const uint16_t*>(w_router),
                               G, E, H, fast, parts);
        else
            hipLaunchKernelGGL(moe::gate_chunk_kernel<float>, grid, dim3(moe::G_THREADS), 0, stream,
                               static_cast<const float*>(global_x), static_cast<const float*>(w_router),
                               G, E, H, fast, parts);
        MOE_LAUNCH_CHECK();
        // the select kernel adds the chunk partials in chunk order and writes the logits
        return moe::launch_select(logits, row_valid, G, bias, cfg, topk_ids, topk_w, stream, parts, nch);
    } else if (rows128 && fast && H % moe::GATE_CHUNK == 0) {
        if (dt == MOE_BF16)
            hipLaunchKernelGGL(moe::gate_exact8_kernel<uint16_t>, tiles, dim3(moe::G8_THREADS), 0, stream,
                               static_cast<const uint16_t*>(global_x), static_cast<const uint16_t*>(w_router),
                               row_valid, G, E, H, logits);
        else
            hipLaunchKernelGGL(moe::gate_exact8_kernel<float>, tiles, dim3(moe::G8_THREADS), 0, stream,
                               static_cast<const float*>(global_x), static_cast<const float*>(w_router),
                               row_valid, G, E, H, logits);
    } else if (dt == MOE_BF16) {
        const uint16_t* xb = static_cast<const uint16_t*>(global_x);
        const uint16_t* wb = static_cast<const uint16_t*>(w_router);
        if (rows128)
            hipLaunchKernelGGL((moe::gate_exact_kernel<uint16_t, 2>), tiles, dim3(moe::G_THREADS), 0, stream, xb,
                               wb, row_valid, G, E, H, fast, logits);
        else
            hipLaunchKernelGGL((moe::gate_exact_kernel<uint16_t, 1>), tiles64, dim3(moe::G_THREADS), 0, stream, xb,
                               wb, row_valid, G, E, H, fast, logits);
    } else {
        const float* xf = static_cast<const float*>(global_x);
        const float* wf = static_cast<const float*>(w_router);
        if (rows128)
            hipLaunchKernelGGL((moe::gate_exact_kernel<float, 2>), tiles, dim3(moe::G_THREADS), 0, stream, xf, wf,
                               row_valid, G, E, H, fast, logits);
        else
            hipLaunchKernelGGL((moe::gate_exact_kernel<float, 1>), tiles64, dim3(moe::G_THREADS), 0, stream, xf,
                               wf, row_valid, G, E, H, fast, logits);
    }
    MOE_LAUNCH_CHECK();
    return moe::launch_select(logits, row_valid, G, bias, cfg, topk_ids, topk_w, stream);
}
