// SwiGLU experts as two grouped GEMMs over the dispatch segments.
//
// Per local slot e and every row r of its segment (SGLang walkthrough "SGLang 源码完全拆解
// (十七): DP Attention 与专家并行", section "EP 下专家权重切不均匀的问题": gate_proj and up_proj
// are [I, H], down_proj [H, I], and experts stay whole per rank so each GEMM keeps its full
// size; vLLM walkthrough "vLLM 源码完全拆解(二十七)", modular-kernel figure: MM1, activation,
// MM2 between permute and unpermute):
//     h[r, i] = silu(sum_h x[r,h] Wg[e][i,h]) * (sum_h x[r,h] Wu[e][i,h])
//     y[r, c] = sum_i h[r,i] Wd[e][c,i]
//
// Three kernels, all on gfx950 v_mfma_f32_32x32x16_bf16 with fp32 accumulation, all with the
// weight fragment as the MFMAs' first operand (each accumulator block holds its output block
// transposed, so a lane writes four consecutive columns of one row per 8-byte store), the
// up GEMM's 256 weight rows being 128 gate rows and the same 128 up rows (SiLU * up in
// registers, only h written), operands moved global -> LDS by buffer DMA, rows past a
// segment's end read as zeros and never stored, and one owner per output tile:
//   - grouped_gemm_pp_kernel: slots of more than 64 rows (not launched when no slot can hold
//     more than 512 rows: the streaming kernel then takes every slot).  256 x 256 tiles, 8 waves in two
//     groups that alternate between an MFMA phase and a memory phase; persistent grid, one
//     block per CU, XCD-grouped tile order (gemm_common.h).  fp8 weights with bf16
//     activations (the default for e4m3 weights) run here too: weight rows are staged as
//     fp8 (half the bytes) and a lane's 16 weight bytes are dequantised (exact e4m3 -> fp32,
//     times the block's fp32 scale, RNE to bf16) into the fragments of two MFMA steps.
//   - grouped_gemm_stream_kernel: bf16 weights, slots of 1-64 rows (every slot for batches of
//     at most 512 rows), which stream their weights: 64 x 128 tiles, 64-deep slices, five
//     stages, non-temporal weight loads.
//   - generic_gemm_kernel: any other shape, alignment or activation dtype, on the fp32
//     matrix cores.
// fp8 weights with per-1x128-group e4m3 activations (fp8 matrix cores, fp32 promotion per K
// group) live in expert_gemm_fp8.hip.
#include <hip/hip_runtime.h>

#include "gemm_common.h"
#include "moe_dev.h"

namespace moe {
namespace gemm {
int num_cus() { return device_cus(); }
int grid_blocks(hipStream_t stream) {
    const int n = stream_cus(stream) & ~7;  // whole XCD groups of 8 for the tile order
    return n >= 8 ? n : 8;
}
}  // namespace gemm

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256;
constexpr int BK = 64;      // K slice of the weight-streaming kernel: whole 128-byte lines per row
constexpr int UP_COLS = BN / 2;     // i-columns per up tile (gate and up each)
constexpr int kMaxKG8 = 128;        // fp8 weights: at most 128 K groups (K <= 16384)

struct GemmArgs {
    const uint16_t* A;       // [cap, K] bf16 rows in segment order
    const uint16_t* B;       // up: w13 [E_l, 2, I, H]; down: w2 [E_l, H, I] (bf16 weights)
    const uint8_t* B8;       // the same layouts in e4m3 (fp8 weights, dequantised in the kernel)
    const float* SB;         // fp8: 128x128 block scales, up [E_l, 2, I/128, H/128], down [E_l, H/128, I/128]
    uint16_t* C;             // up: h [cap, I]; down: y [cap, H]
    const int32_t* counts;   // [E_l]
    const int64_t* seg;      // [E_l + 1]
    int64_t cap;
    int64_t K;               // up: H; down: I
    int64_t N;               // up: I; down: H
    int32_t El;
    int32_t NT;              // column tiles per m-tile
    // gather form (amap != NULL): the permuted row r is row amap[r] / ak of A, which holds
    // arows rows (A = the [G, H] global buffer, amap = the plan's sorted_pair); a negative
    // entry reads as a zero row.  NULL: row r of A.
    const int32_t* amap;
    int32_t ak;
    int64_t arows;
    // the streaming kernel takes the slots of at most st_hi rows (ST_BM_SPLIT, or every slot
    // when no slot can outgrow a few of its tiles and the ping-pong kernel is not launched)
    int64_t st_hi;
};

// Offset past every buffer resource this file builds (each covers under 2^31 bytes): a DMA
// at it, plus its chunk and K offset, reads zeros.
constexpr uint32_t kAOut = 0x80000000u;

// Byte offsets of the A rows that tile-local rows r0 + p * rstep (permuted rows row0 + r)
// read, p < P: from the tile's first row in the copy form, from A itself in the gather form;
// kAOut past the tile's nrows rows or for an empty or out-of-range gather entry.  The P map
// entries are loaded at once (clamped to the tile's last row), then checked, so a tile start
// waits for one round trip, not P.
template <int P>
__device__ __forceinline__ void a_row_offsets(const GemmArgs& a, int64_t row0, uint32_t r0, uint32_t rstep,
                                              uint32_t nrows, uint32_t row_bytes, uint32_t (&off)[P]) {
    if (a.amap == nullptr || nrows == 0) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const uint32_t r = r0 + p * rstep;
            off[p] = r < nrows ? r * row_bytes : kAOut;
        }
        return;
    }
    int32_t f[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const uint32_t r = r0 + p * rstep;
        f[p] = a.amap[row0 + (r < nrows ? r : nrows - 1)];
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const uint32_t r = r0 + p * rstep;
        const int64_t g = f[p] >= 0 ? f[p] / a.ak : a.arows;
        off[p] = r < nrows && g < a.arows ? static_cast<uint32_t>(g) * row_bytes : kAOut;
    }
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

typedef float f32x2_t __attribute__((ext_vector_type(2)));
// 8 consecutive e4m3 weights times their fp32 block scale, rounded once more to bf16: the
// conversion to fp32 is exact, the product is rounded to fp32, then RNE to bf16
__device__ __forceinline__ bf16x8_t dequant8(uint2 u, float s) {
    const f32x2_t p0 = __builtin_amdgcn_cvt_pk_f32_fp8(u.x, false), p1 = __builtin_amdgcn_cvt_pk_f32_fp8(u.x, true);
    const f32x2_t p2 = __builtin_amdgcn_cvt_pk_f32_fp8(u.y, false), p3 = __builtin_amdgcn_cvt_pk_f32_fp8(u.y, true);
    const bf16x8_t r = {(__bf16)(p0[0] * s), (__bf16)(p0[1] * s), (__bf16)(p1[0] * s), (__bf16)(p1[1] * s),
                        (__bf16)(p2[0] * s), (__bf16)(p2[1] * s), (__bf16)(p3[0] * s), (__bf16)(p3[1] * s)};
    return r;
}

// LDS rows of BK bf16 (128 bytes), of CPR 16-byte chunks.  The LDS serves a 16-byte-per-lane
// read 16 lanes at a time from 64 banks (256 bytes); the fragment reads have 16 consecutive
// rows asking for the same logical chunk, so the chunk index is xor-ed with swz(row) =
// (row / 2) mod 8, which puts those 16 rows on 16 distinct 16-byte slots of the 256-byte
// bank window.
constexpr int CPR = BK / 8;            // 16-byte chunks per row
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// ------------------------------------------------------------------ bf16: 8-wave ping-pong
// bf16 weights.  The same 256 x 256 tiles, tile order and accumulation order as
// the earlier 4-wave form (so the same bits), with 8 waves, two per SIMD: waves w and w + 4
// share SIMD w % 4 and its 128 x 128 region, and each owns two of the region's four 32-column
// blocks (up: gate block g and its up block g + 2; down: blocks 2g, 2g + 1), i.e. 128 x 64
// outputs in 128 accumulators per lane, so two such waves fit in the register file.
//   - The two groups of four waves (g = w / 4) alternate: while one group runs the 16 MFMAs of
//     a 32-deep K slice, the other reads the fragments of its next slice and issues its DMAs,
//     and a barrier between phases swaps them.  A wave that streams MFMAs then issues no
//     vector-memory instruction (each costs such a wave tens of cycles of matrix-core time),
//     and every SIMD's matrix core is fed by one wave of the pair or the other.
//   - Operands come from L2 or HBM at a latency of thousands of cycles, so the LDS holds four
//     32-deep stages (128 KB) and three slices are in flight: group 0 DMAs the A rows, group 1
//     the weight rows, 4 instructions of 16 rows x 64 bytes per wave and slice.
// Phases p = 0, 1, ...: group 0 computes slice n in phase 2n and group 1 in phase 2n + 1; each
// wave reads slice n's fragments in the phase just before its own (group 0: 2n - 1, group 1:
// 2n).  Slice n sits in stage n % 4.  In its memory phase for slice n every wave issues the
// DMAs of slice n + 3 into stage (n + 3) % 4, whose last reads (slice n - 1, group 1, phase
// 2n - 2) are behind a barrier; past the last slice it reloads the last slice there, never
// read, so every phase issues the same number.  Before the barrier that ends phase 2n each
// wave waits until only its two newest DMA groups (slices n + 2, n + 3) are in flight, so
// slice n + 1 has landed when group 0 reads it in phase 2n + 1.  Group 1 starts one barrier
// late and group 0 ends one barrier late, so every wave passes the same barriers.
// fp8 weights (W8): a stage's weight rows are 32 fp8 bytes (8 KB for the tile, 2 DMAs of 32
// rows per group-1 wave and slice, so group 1 waits for vmcnt 4 where group 0 waits for 8);
// in its memory phase a wave reads 16 bytes per weight block, dequantises them with the
// block's scale (staged in LDS at tile start) into the fragments of both MFMA steps, and
// reads its activation fragments in the matching K order.  The MFMAs are the bf16 ones.
// fp8 weights take every slot (there is no streaming form for them).
// Where a tile's K loop starts, in 64-deep steps (it then wraps around K).  When every CU
// walks K from 0 in step, the rows of all tiles in flight are read at the same offset, and
// with weight rows 4 KB apart (K = 2048) those requests pile onto the same memory channels;
// starting each slot, and each group of eight 256-column tiles, elsewhere spreads them
// (measured cold: DP-gather gate+up 0.167 -> 0.145 ms, decode down 0.058 -> 0.048 ms).  The
// ping-pong kernel uses the same rule (its 32-deep slices in pairs), so an output column
// accumulates its K products in the same order in both kernels, whichever takes its slot;
// the eight tiles that one XCD sweeps together share a start, so they still share their
// activation panels through L2.
__device__ __forceinline__ int64_t k_start64(int e, int32_t tile256, int64_t steps64) {
    return (static_cast<int64_t>(e) * 5 + static_cast<int64_t>(tile256 >> 3) * 3) % steps64;
}

constexpr int ST_BM_SPLIT = 64;  // slots with more rows than this run here, the rest in the streaming kernel
// When no slot can hold more rows than this (G, or the fixed capacity), the streaming kernel
// takes every slot alone: at most 8 of its 64-row tiles per slot, whose repeated weight reads
// come from the caches, against a ping-pong launch that would find few tiles or none.
constexpr int64_t kStreamOnlyRows = 512;
constexpr int PP_THREADS = 512;
constexpr int PP_BK = 32;                        // K per slice
constexpr int PP_STAGES = 4;
constexpr int PP_CPR = PP_BK / 8;                // 16-byte chunks per LDS row
constexpr int PP_RPB = 64 / PP_CPR;              // rows per 1 KB DMA block
constexpr int PP_LPW = BM / PP_RPB / 4;          // DMAs per wave per slice
static_assert(PP_LPW == 4 && PP_RPB == 16, "the wait counts below assume 4 DMAs of 16 rows");
// the LDS serves a 16-byte-per-lane read 16 lanes at a time from 64 banks (256 bytes); a
// fragment read has 16 consecutive 64-byte rows asking for the same logical chunk, and the
// xor with (row / 4) mod 4 puts them on 16 distinct 16-byte slots of a 256-byte window
__device__ __forceinline__ int pp_swz(int row) { return (row >> 2) & 3; }
// fp8 weights: a stage's weight rows are 32 bytes; a fragment read has 16 consecutive rows
// asking for the same 16-byte half, and swapping the halves on every other group of 8 rows
// puts them on 16 distinct 16-byte slots of a 256-byte window
__device__ __forceinline__ int w8_swz(int row) { return (row >> 3) & 1; }
constexpr int PP_W8DMA = 2;                      // fp8 weight DMAs (32 rows x 32 bytes) per wave and slice

template <bool UP, bool W8>
__global__ __launch_bounds__(PP_THREADS, 1) void grouped_gemm_pp_kernel(GemmArgs a, gemm::TileOrder to) {
    __shared__ __attribute__((aligned(1024))) uint16_t As[PP_STAGES][BM * PP_BK];
    __shared__ __attribute__((aligned(1024))) uint16_t Bs[PP_STAGES][BN * PP_BK];
    __shared__ int32_t tile_prefix[gemm::kMaxSlots + 1];
    __shared__ int32_t part[PP_THREADS];
    // fp8 weights: the tile's weight block scales along K, [2][K/128] (up: gate, up half;
    // down: the two 128-column blocks of the tile), staged at tile start
    __shared__ float sbuf[W8 ? 2 : 1][W8 ? kMaxKG8 : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = wv >> 2;       // group
    const int sq = wv & 3;       // SIMD and 128 x 128 region
    const int wm = sq >> 1, wn = sq & 1;

    const int32_t total_mt =
        gemm::number_tiles<BM, PP_THREADS>(a.counts, a.seg, a.cap, a.El, tile_prefix, part,
                                           W8 ? 0 : ST_BM_SPLIT);  // fp8 weights: every slot
    const uint32_t row_bytes = static_cast<uint32_t>(a.K) * 2u;
    const int nsn = a.NT / to.SN;
    const int64_t total_super = static_cast<int64_t>((total_mt + to.SM - 1) / to.SM) * nsn;
    const int xcd = blockIdx.x & 7;
    const int q = blockIdx.x >> 3;
    const int dma_row = lane / PP_CPR;
    const int frow = lane & 31;
    // fragment of MFMA step ks (16 deep) of a slice: row frow of a 32-row block, logical
    // chunk 2 ks + lane / 32
    int fchunk[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) fchunk[ks] = ((2 * ks + (lane >> 5)) ^ pp_swz(frow)) * 8;
    // fp8 weights: a lane reads 16 weight bytes of its row at K 16 (lane / 32) of the slice and
    // feeds the first 8 to step 0, the last 8 to step 1; the activation fragments follow (step
    // ks of lane half h: K 16 h + 8 ks .. + 8), so every product still pairs equal K
    if constexpr (W8) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) fchunk[ks] = ((2 * (lane >> 5) + ks) ^ pp_swz(frow)) * 8;
    }
    const int64_t KG = a.K / 128, NB = a.N / 128;
    // LDS rows of the wave's two weight column blocks
    int brow[2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        const int j = UP ? g + 2 * jj : 2 * g + jj;
        brow[jj] = UP ? (j >> 1) * UP_COLS + wn * 64 + (j & 1) * 32 : wn * 128 + j * 32;
    }

    for (int64_t sup = xcd; sup < total_super; sup += 8) {
        const int32_t em = static_cast<int32_t>(sup / nsn) * to.SM + q / to.SN;
        const int32_t nt = static_cast<int32_t>(sup % nsn) * to.SN + q % to.SN;
        if (em >= total_mt) continue;
        const int e = gemm::slot_of_tile(tile_prefix, a.El, em);
        const int32_t mtile = __builtin_amdgcn_readfirstlane(em - tile_prefix[e]);
        const int64_t seg_start = a.seg[e];
        int64_t seg_end = seg_start + a.counts[e];
        seg_end = seg_end < a.cap ? seg_end : a.cap;
        const int64_t row0 = seg_start + static_cast<int64_t>(mtile) * BM;
        const int64_t nrows64 = seg_end - row0;
        const uint32_t nrows = static_cast<uint32_t>(nrows64 < BM ? nrows64 : BM);

        // group 0 streams A, group 1 streams B; wave sq of a group covers tile rows
        // 64 sq .. 64 sq + 63 in 4 DMA blocks of 16 rows
        const bool loads_a = g == 0;
        const uint16_t* dbase;
        uint32_t dbytes;
        if (loads_a) {
            // rows past the segment end fall outside the resource: they read as zeros
            dbase = a.amap ? a.A : a.A + row0 * a.K;
            dbytes = a.amap ? static_cast<uint32_t>(a.arows) * row_bytes : nrows * row_bytes;
        } else if (W8) {
            const int64_t rows = UP ? 2 * a.N : a.N;
            dbase = reinterpret_cast<const uint16_t*>(a.B8 + static_cast<int64_t>(e) * rows * a.K);
            dbytes = static_cast<uint32_t>(rows * a.K);
        } else if (UP) {
            dbase = a.B + static_cast<int64_t>(e) * 2 * a.N * a.K;
            dbytes = static_cast<uint32_t>(2 * a.N) * row_bytes;
        } else {
            dbase = a.B + static_cast<int64_t>(e) * a.N * a.K;
            dbytes = static_cast<uint32_t>(a.N) * row_bytes;
        }
        const __amdgpu_buffer_rsrc_t rsrc = gemm::make_rsrc_uniform(dbase, dbytes);
        // DMA p covers tile row r = 64 sq + 16 p + dma_row, global row that of p = 0 plus 16 p
        // (up: a wave's 64 rows lie all in the gate half or all in the up half); the swizzle
        // (r / 4) mod 4 is the same for every p
        const int r0 = 64 * sq + dma_row;
        uint32_t grow;
        if (loads_a) grow = static_cast<uint32_t>(r0);
        else if (UP) grow = static_cast<uint32_t>((r0 >= 128 ? a.N : 0) + nt * UP_COLS + (r0 & 127));
        else grow = static_cast<uint32_t>(nt * BN + r0);
        const uint32_t chunk = static_cast<uint32_t>(((lane % PP_CPR) ^ pp_swz(r0)) * 16);
        uint32_t vbase = grow * row_bytes + chunk;
        uint32_t rstep = static_cast<uint32_t>(PP_RPB) * row_bytes;
        // the lane's offset in DMA p: weight rows step by 16 rows, activation rows are looked
        // up (they are consecutive only in the copy form)
        uint32_t voff[PP_LPW];
        if (loads_a) {
            a_row_offsets<PP_LPW>(a, row0, static_cast<uint32_t>(r0), PP_RPB, nrows, row_bytes, voff);
#pragma unroll
            for (int p = 0; p < PP_LPW; ++p) voff[p] += chunk;
        } else {
#pragma unroll
            for (int p = 0; p < PP_LPW; ++p) voff[p] = vbase + static_cast<uint32_t>(p) * rstep;
        }
        if (W8 && !loads_a) {
            // fp8 weight rows are K bytes, 32 per slice: a DMA covers 32 rows x 32 bytes, lane
            // pair per row, wave sq tile rows 64 sq + 32 p + lane / 2; the 16-byte halves of a
            // row trade places on every other group of 8 rows (w8_swz), the same for both p
            const int rr = 64 * sq + lane / 2;
            const uint32_t g8 = UP ? static_cast<uint32_t>((rr >= 128 ? a.N : 0) + nt * UP_COLS + (rr & 127))
                                   : static_cast<uint32_t>(nt * BN + rr);
            vbase = g8 * static_cast<uint32_t>(a.K) + static_cast<uint32_t>(((lane & 1) ^ w8_swz(rr)) * 16);
            rstep = 32u * static_cast<uint32_t>(a.K);
        }
        auto issue = [&](int stage, int64_t kt) {
            if constexpr (W8) {
                if (!loads_a) {
                    uint8_t* b8 = reinterpret_cast<uint8_t*>(&Bs[0][0]) + stage * (BN * PP_BK * 2) + sq * PP_W8DMA * 1024;
                    uint32_t vb8 = vbase;
                    asm volatile("" : "+s"(b8), "+v"(vb8));
#pragma unroll
                    for (int p = 0; p < PP_W8DMA; ++p)
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (gemm::lds_void_t*)(b8 + p * 1024), 16,
                                                                vb8 + static_cast<uint32_t>(p) * rstep,
                                                                static_cast<int>(kt * PP_BK), 0, 0);
                    return;
                }
            }
            int off = stage * (BM * PP_BK) + sq * PP_LPW * 512;
            uint32_t v0 = voff[0], v1 = voff[1], v2 = voff[2], v3 = voff[3];
            asm volatile("" : "+s"(off), "+v"(v0), "+v"(v1), "+v"(v2), "+v"(v3));
            const uint32_t vo[PP_LPW] = {v0, v1, v2, v3};
            uint16_t* base = (loads_a ? &As[0][0] : &Bs[0][0]) + off;
            const int soff = static_cast<int>(kt * PP_BK * 2);
#pragma unroll
            for (int p = 0; p < PP_LPW; ++p)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (gemm::lds_void_t*)(base + p * 512), 16, vo[p],
                                                        soff, 0, 0);
        };

        floatx16_t acc[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][jj][v] = 0.f;
        const uint16_t* a_rd = &As[0][0] + (wm * 128 + frow) * PP_BK;
        const uint16_t* b_rd = &Bs[0][0] + frow * PP_BK;
        bf16x8_t fa[2][4], fb[2][2];
        // fragments of the slice in `stage`: two 16-deep MFMA steps
        // fp8 block scale of the wave's weight block jj in K group kg (up: gate half, up half;
        // down: the 128-column block wn)
        auto wscale = [&](int jj, int64_t kt) -> float {
            const int64_t kg = kt / (128 / PP_BK);
            return sbuf[UP ? jj : wn][kg];
        };
        auto read_slice = [&](int stage, int64_t kt) {
            if constexpr (W8) {
                const uint8_t* b8 = reinterpret_cast<const uint8_t*>(&Bs[0][0]) + stage * (BN * PP_BK * 2);
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        fa[ks][i] = *reinterpret_cast<const bf16x8_t*>(a_rd + stage * (BM * PP_BK) + i * 32 * PP_BK +
                                                                       fchunk[ks]);
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const int row = brow[jj] + frow;
                    const uint4 raw = *reinterpret_cast<const uint4*>(b8 + row * 32 + (((lane >> 5) ^ w8_swz(row)) * 16));
                    const float sc = wscale(jj, kt);
                    fb[0][jj] = dequant8(make_uint2(raw.x, raw.y), sc);
                    fb[1][jj] = dequant8(make_uint2(raw.z, raw.w), sc);
                }
                return;
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    fa[ks][i] = *reinterpret_cast<const bf16x8_t*>(a_rd + stage * (BM * PP_BK) + i * 32 * PP_BK +
                                                                   fchunk[ks]);
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
                    fb[ks][jj] = *reinterpret_cast<const bf16x8_t*>(b_rd + stage * (BN * PP_BK) + brow[jj] * PP_BK +
                                                                    fchunk[ks]);
            }
        };
        auto mfma_slice = [&]() {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj)
                        acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks][jj], fa[ks][i], acc[i][jj], 0,
                                                                              0, 0);
        };
        // a barrier that neither the compiler nor the scheduler moves work across
        auto phase_end = [&]() {
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        };

        const int64_t KT = a.K / PP_BK;
        // slice n of the loop is K slice rk(n): the loop starts at an even slice (k_start64)
        const int64_t rot = 2 * k_start64(e, nt, KT / 2);
        auto rk = [&](int64_t t) { t += rot; return t >= KT ? t - KT : t; };
        // the previous tile's output stores are done; every wave passed the previous tile's
        // last barrier, so no wave still reads a stage.  The intrinsic (all counters to zero)
        // rather than inline asm: the compiler's own wait tracking sees it, and no longer
        // carries the epilogue's stores into the K loop (where it would drain every DMA in
        // flight before reusing a register the stores read)
        __builtin_amdgcn_s_waitcnt(0);
        asm volatile("" ::: "memory");
        if constexpr (W8) {
            for (int t = tid; t < 2 * KG; t += PP_THREADS) {
                const int r = t / static_cast<int>(KG), kg = t % static_cast<int>(KG);
                sbuf[r][kg] = UP ? a.SB[((static_cast<int64_t>(e) * 2 + r) * NB + nt) * KG + kg]
                                 : a.SB[(static_cast<int64_t>(e) * NB + 2 * nt + r) * KG + kg];
            }
            // the prologue barrier below publishes sbuf; its loads end here, so the DMA
            // counts that follow start from zero
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        }
        issue(0, rk(0));
        issue(1, rk(KT > 1 ? 1 : KT - 1));
        issue(2, rk(KT > 2 ? 2 : KT - 1));
        // slice 0 landed: each wave's two newest groups may still be in flight
        if (W8 && g == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PP_W8DMA) : "memory");
        else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PP_LPW) : "memory");
        phase_end();
        if (g == 1) phase_end();
        for (int64_t n = 0; n < KT; ++n) {
            const int st = static_cast<int>(n & (PP_STAGES - 1));
            // memory phase: this slice's fragments, the DMAs of slice n + 3
            read_slice(st, rk(n));
            issue((st + 3) & (PP_STAGES - 1), rk(n + 3 < KT ? n + 3 : KT - 1));
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            // group 1: slice n + 1 landed before the barrier that ends phase 2n
            if (g == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * (W8 ? PP_W8DMA : PP_LPW)) : "memory");
            phase_end();
            // compute phase
            mfma_slice();
            if (g == 0) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PP_LPW) : "memory");
            phase_end();
        }
        if (g == 0) phase_end();

        // ---- epilogue over the wave's two column blocks
        const int rloc = wm * 128 + (lane & 31);
        const int64_t colbase = UP ? static_cast<int64_t>(nt) * UP_COLS + wn * 64 + (lane >> 5) * 4
                                   : static_cast<int64_t>(nt) * BN + wn * 128 + (lane >> 5) * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (rloc + i * 32 >= static_cast<int>(nrows)) continue;
            uint16_t* cp = a.C + (row0 + rloc + i * 32) * a.N + colbase;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                if (UP) {
                    float h[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) h[t] = silu_mul(acc[i][0][4 * qq + t], acc[i][1][4 * qq + t]);
                    *reinterpret_cast<uint2*>(cp + g * 32 + qq * 8) =
                        make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
                } else {
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj) {
                        const floatx16_t& c = acc[i][jj];
                        *reinterpret_cast<uint2*>(cp + (2 * g + jj) * 32 + qq * 8) =
                            make_uint2(pack_bf16x2(c[4 * qq], c[4 * qq + 1]), pack_bf16x2(c[4 * qq + 2], c[4 * qq + 3]));
                    }
                }
            }
        }
    }
    // no DMA into LDS may outlive the workgroup
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ------------------------------------------------------------------ bf16: weight streaming
// Slots with at most 64 rows (decode, and the many small slots of a DP-gathered batch) are
// bound by streaming their weights, not by the matrix cores: a 256-row tile of the ping-pong
// kernel spends its MFMAs on padding, and its 32-deep slices fetch half a 128-byte line per
// row and request, while a CU keeps only a bounded number of L1 -> L2 requests in flight, so
// its rate is set by the bytes per request.  Here a tile is 64 rows x 128 weight rows (up: 64
// gate + the same 64 up columns; down: 128 columns), so a decode batch whose routed rows sit
// in a few slots still has a tile for every CU, in 64-deep slices (whole lines, with the
// swizzle swz below): five 24 KB stages, four slices in flight.  Four
// waves, one per SIMD: wave w owns rows 32 (w mod 2) .. + 31 and column group w / 2 (up:
// gate block and up block of 32 columns; down: two 32-column blocks).  Per slice each wave
// DMAs two activation blocks and four weight blocks of 8 rows (all gate or all up), one
// barrier per slice.  The MFMAs see the K values in the same order as in the ping-pong kernel
// (four 16-deep steps per slice) and the epilogue is its epilogue, so the bits are the same.
// The ping-pong kernel takes the slots with more than 64 rows, except in batches of at most
// 512 rows, where this kernel takes every slot; the two kernels number their own tiles on the
// device, so the host never reads the counts.
constexpr int ST_THREADS = 256;
// cache-policy operand of the weight DMAs: non-temporal (each weight line is read once).
// Measured on the decode shape, cold: gate+up 0.148 -> 0.082 ms against plain loads.
constexpr int kNonTemporal = 2;
constexpr int ST_BM = ST_BM_SPLIT;               // rows per tile (the largest slot taken, unless st_hi says more)
constexpr int ST_BN = 128;                       // weight rows per tile
constexpr int ST_UPC = ST_BN / 2;                // up: i-columns per tile
constexpr int ST_STAGES = 5;
constexpr int ST_RPB = 64 / CPR;                 // rows per 1 KB DMA block (8)
constexpr int ST_ADMA = ST_BM / ST_RPB / 4;      // activation DMAs per wave and slice (2)
constexpr int ST_BDMA = ST_BN / ST_RPB / 4;      // weight DMAs per wave and slice (4)
constexpr int ST_VPS = ST_ADMA + ST_BDMA;        // DMAs per wave and slice
static_assert(BK == 64 && CPR == 8 && ST_ADMA == 2, "whole 128-byte lines per row and slice");

template <bool UP>
__global__ __launch_bounds__(ST_THREADS, 1) void grouped_gemm_stream_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(1024))) uint16_t As[ST_STAGES][ST_BM * BK];
    __shared__ __attribute__((aligned(1024))) uint16_t Bs[ST_STAGES][ST_BN * BK];
    __shared__ int32_t tile_prefix[gemm::kMaxSlots + 1];
    __shared__ int32_t part[ST_THREADS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rbk = w & 1, cg = w >> 1;  // row block, column group
    const int32_t total_mt =
        gemm::number_tiles<ST_BM, ST_THREADS>(a.counts, a.seg, a.cap, a.El, tile_prefix, part, 0, a.st_hi);
    const uint32_t row_bytes = static_cast<uint32_t>(a.K) * 2u;
    const int32_t NT = static_cast<int32_t>((UP ? 2 : 1) * a.N / ST_BN);
    const int64_t tiles = static_cast<int64_t>(total_mt) * NT;
    const int dma_row = lane / CPR;  // 0..7
    const int frow = lane & 31;
    // fragment of MFMA step ks (16 deep) of a slice: row frow of a 32-row block, logical
    // chunk 2 ks + lane / 32
    int fchunk[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) fchunk[ks] = ((2 * ks + (lane >> 5)) ^ swz(frow)) * 8;
    // B-tile rows of the wave's two 32-row weight blocks
    int brow[2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) brow[jj] = UP ? jj * ST_UPC + cg * 32 : cg * 64 + jj * 32;
    // activation DMA p: tile rows 16 w + 8 p + dma_row; weight DMA p: tile rows 32 w + 8 p +
    // dma_row.  The swizzle (row / 2) mod 8 of DMA p is that of p = 0 xor 4 (p mod 2).
    const int ra = 16 * w + dma_row, rb = 32 * w + dma_row;
    uint32_t achunk[2], bchunk[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        achunk[par] = static_cast<uint32_t>(((lane % CPR) ^ swz(ra + 8 * par)) * 16);
        bchunk[par] = static_cast<uint32_t>(((lane % CPR) ^ swz(rb + 8 * par)) * 16);
    }
    const uint32_t rstep = static_cast<uint32_t>(ST_RPB) * row_bytes;

    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        const int32_t em = static_cast<int32_t>(t / NT);
        const int32_t nt = static_cast<int32_t>(t % NT);
        const int e = gemm::slot_of_tile(tile_prefix, a.El, em);
        const int32_t mtile = __builtin_amdgcn_readfirstlane(em - tile_prefix[e]);
        const int64_t seg_start = a.seg[e];
        int64_t seg_end = seg_start + a.counts[e];
        seg_end = seg_end < a.cap ? seg_end : a.cap;
        const int64_t row0 = seg_start + static_cast<int64_t>(mtile) * ST_BM;
        const int64_t nrows64 = seg_end - row0;
        const uint32_t nrows = static_cast<uint32_t>(nrows64 < ST_BM ? nrows64 : ST_BM);

        // rows past the segment end fall outside the resource: they read as zeros
        const __amdgpu_buffer_rsrc_t arsrc =
            a.amap ? gemm::make_rsrc_uniform(a.A, static_cast<uint32_t>(a.arows) * row_bytes)
                   : gemm::make_rsrc_uniform(a.A + row0 * a.K, nrows * row_bytes);
        const uint16_t* bbase = a.B + static_cast<int64_t>(e) * (UP ? 2 : 1) * a.N * a.K;
        const __amdgpu_buffer_rsrc_t brsrc =
            gemm::make_rsrc_uniform(bbase, static_cast<uint32_t>((UP ? 2 : 1) * a.N) * row_bytes);
        // up: waves 0, 1 stream gate rows, waves 2, 3 up rows (N further on)
        const uint32_t grow = UP ? static_cast<uint32_t>((rb >= ST_UPC ? a.N : 0) + nt * ST_UPC + (rb & (ST_UPC - 1)))
                                 : static_cast<uint32_t>(nt * ST_BN + rb);
        const uint32_t bvb = grow * row_bytes;
        // activation DMA p reads tile row ra + 8 p (looked up in the gather form)
        uint32_t aoff[ST_ADMA];
        a_row_offsets<ST_ADMA>(a, row0, static_cast<uint32_t>(ra), ST_RPB, nrows, row_bytes, aoff);
#pragma unroll
        for (int p = 0; p < ST_ADMA; ++p) aoff[p] += achunk[p & 1];
        auto issue = [&](int stage, int64_t kt) {
            gemm::lds_void_t* adst = (gemm::lds_void_t*)(&As[0][0] + stage * (ST_BM * BK) + w * ST_ADMA * 512);
            gemm::lds_void_t* bdst = (gemm::lds_void_t*)(&Bs[0][0] + stage * (ST_BN * BK) + w * ST_BDMA * 512);
            uint32_t va0 = aoff[0], va1 = aoff[1], vb0 = bvb + bchunk[0], vb1 = bvb + bchunk[1];
            asm volatile("" : "+s"(adst), "+s"(bdst), "+v"(va0), "+v"(va1), "+v"(vb0), "+v"(vb1));
            const int soff = static_cast<int>(kt * BK * 2);
#pragma unroll
            for (int p = 0; p < ST_ADMA; ++p)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    arsrc, (gemm::lds_void_t*)((char __attribute__((address_space(3)))*)adst + p * 1024), 16,
                    (p & 1) ? va1 : va0, soff, 0, 0);
#pragma unroll
            for (int p = 0; p < ST_BDMA; ++p)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    brsrc, (gemm::lds_void_t*)((char __attribute__((address_space(3)))*)bdst + p * 1024), 16,
                    ((p & 1) ? vb1 : vb0) + static_cast<uint32_t>(p) * rstep, soff, 0, kNonTemporal);
        };

        floatx16_t acc[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[jj][v] = 0.f;

        const int64_t KT = a.K / BK;
        // step n of the loop is K step rk(n) (k_start64; this tile's 256-column tile is nt / 2)
        const int64_t rot = k_start64(e, nt >> 1, KT);
        auto rk = [&](int64_t t) { t += rot; return t >= KT ? t - KT : t; };
        // the previous tile's output stores are done (its reads ended at the barrier below)
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        // slices 0 .. S-2 (a short K reloads its last slice into the spare stages, never read)
#pragma unroll
        for (int s = 0; s < ST_STAGES - 1; ++s) issue(s, rk(s < KT ? s : KT - 1));
        int st = 0;
        for (int64_t n = 0; n < KT; ++n) {
            // slice n landed for this wave (its newest S - 2 slices may be in flight); after
            // the barrier, for every wave, and no wave still reads stage (n - 1) mod S
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"((ST_STAGES - 2) * ST_VPS) : "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            bf16x8_t fa[4], fb[4][2];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                fa[ks] = *reinterpret_cast<const bf16x8_t*>(&As[0][0] + st * (ST_BM * BK) +
                                                            (rbk * 32 + frow) * BK + fchunk[ks]);
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
                    fb[ks][jj] = *reinterpret_cast<const bf16x8_t*>(&Bs[0][0] + st * (ST_BN * BK) +
                                                                    (brow[jj] + frow) * BK + fchunk[ks]);
            }
            const int refill = st == 0 ? ST_STAGES - 1 : st - 1;
            issue(refill, rk(n + ST_STAGES - 1 < KT ? n + ST_STAGES - 1 : KT - 1));
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
                    acc[jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks][jj], fa[ks], acc[jj], 0, 0, 0);
            st = st == ST_STAGES - 1 ? 0 : st + 1;
        }
        // every wave's reads of every stage are done before the next tile refills them
        __syncthreads();

        // ---- epilogue, as in grouped_gemm_pp_kernel
        const int rloc = rbk * 32 + (lane & 31);
        if (rloc < static_cast<int>(nrows)) {
            const int64_t colbase = UP ? static_cast<int64_t>(nt) * ST_UPC + cg * 32 + (lane >> 5) * 4
                                       : static_cast<int64_t>(nt) * ST_BN + cg * 64 + (lane >> 5) * 4;
            uint16_t* cp = a.C + (row0 + rloc) * a.N + colbase;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                if (UP) {
                    float h[4];
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) h[tt] = silu_mul(acc[0][4 * qq + tt], acc[1][4 * qq + tt]);
                    *reinterpret_cast<uint2*>(cp + qq * 8) = make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
                } else {
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj) {
                        const floatx16_t& c = acc[jj];
                        *reinterpret_cast<uint2*>(cp + jj * 32 + qq * 8) =
                            make_uint2(pack_bf16x2(c[4 * qq], c[4 * qq + 1]), pack_bf16x2(c[4 * qq + 2], c[4 * qq + 3]));
                    }
                }
            }
        }
    }
    // no DMA into LDS may outlive the workgroup
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ------------------------------------------------------------------ generic path
// Any shape, alignment or activation dtype (fp32 activations, bf16 buffers off 16 bytes, H
// not a multiple of 256, I not a multiple of 128): 64-row x 64-column tiles on the fp32
// matrix cores (v_mfma_f32_32x32x2f32), operands widened exactly to fp32 and staged through
// LDS in 32-deep K slices by element loads (zeros past a segment's rows, past K or past N).
// A block of 4 waves owns one tile at a time (wave (wm, wn): 32 rows x 32 columns; up: the
// gate and the up accumulators of the same 32 i-columns) and walks the tiles grid-stride.
// The fp32 matrix-core peak is a sixteenth of bf16's, so these shapes run well below the
// bf16 tile kernels; moe_expert_gemm_fast_path tells a caller which path a call takes.
constexpr int GN_BM = 64, GN_BN = 64, GN_BK = 32;
constexpr int GN_LD = GN_BK + 1;  // odd stride: a column of reads falls on distinct banks

template <typename T>
__device__ __forceinline__ float gn_ld(const T* p, int64_t i) {
    if constexpr (sizeof(T) == 2) return bf16_to_f32(p[i]);
    else return p[i];
}

template <typename T, bool UP>
__global__ __launch_bounds__(256) void generic_gemm_kernel(GemmArgs a, const void* Av, const void* Bv, void* Cv) {
    __shared__ float As[GN_BM * GN_LD];
    __shared__ float Bs[(UP ? 2 : 1) * GN_BN * GN_LD];
    __shared__ int32_t tile_prefix[gemm::kMaxSlots + 1];
    __shared__ int32_t part[gemm::kThreads];
    const T* A = static_cast<const T*>(Av);
    const T* B = static_cast<const T*>(Bv);
    T* C = static_cast<T*>(Cv);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wm = wv >> 1, wn = wv & 1;
    const int32_t total_mt = gemm::number_tiles<GN_BM>(a.counts, a.seg, a.cap, a.El, tile_prefix, part);
    const int64_t NT = ceil_div(a.N, GN_BN);
    const int64_t tiles = static_cast<int64_t>(total_mt) * NT;
    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        const int32_t em = static_cast<int32_t>(t / NT);
        const int64_t n0 = (t % NT) * GN_BN;
        const int e = gemm::slot_of_tile(tile_prefix, a.El, em);
        const int64_t seg_start = a.seg[e];
        int64_t seg_end = seg_start + a.counts[e];
        seg_end = seg_end < a.cap ? seg_end : a.cap;
        const int64_t row0 = seg_start + static_cast<int64_t>(em - tile_prefix[e]) * GN_BM;
        const int64_t nrows = seg_end - row0 < GN_BM ? seg_end - row0 : GN_BM;
        // weight rows of slot e: up -> gate rows [0, N) then up rows [N, 2N); down -> [0, N)
        const T* Bw = B + static_cast<int64_t>(e) * (UP ? 2 : 1) * a.N * a.K;
        floatx16_t acc[2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[u][v] = 0.f;
        for (int64_t k0 = 0; k0 < a.K; k0 += GN_BK) {
            __syncthreads();  // the previous slice's reads are done
            for (int idx = tid; idx < GN_BM * GN_BK; idx += 256) {
                const int r = idx / GN_BK, c = idx % GN_BK;
                int64_t src = row0 + r;  // the gather form looks the row up
                if (a.amap != nullptr && r < nrows) {
                    const int32_t f = a.amap[row0 + r];
                    src = f < 0 || f / a.ak >= a.arows ? -1 : f / a.ak;
                }
                As[r * GN_LD + c] = (r < nrows && src >= 0 && k0 + c < a.K) ? gn_ld(A, src * a.K + k0 + c) : 0.f;
            }
            for (int idx = tid; idx < (UP ? 2 : 1) * GN_BN * GN_BK; idx += 256) {
                const int r = idx / GN_BK, c = idx % GN_BK;
                const int half = r / GN_BN, col = r % GN_BN;
                const bool in = n0 + col < a.N && k0 + c < a.K;
                Bs[r * GN_LD + c] = in ? gn_ld(Bw, (half * a.N + n0 + col) * a.K + k0 + c) : 0.f;
            }
            __syncthreads();
            const float* ar = As + (wm * 32 + (lane & 31)) * GN_LD + (lane >> 5);
            const float* br = Bs + (wn * 32 + (lane & 31)) * GN_LD + (lane >> 5);
#pragma unroll
            for (int kk = 0; kk < GN_BK; kk += 2) {
                const float av = ar[kk];
                acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, br[kk], acc[0], 0, 0, 0);
                if (UP) acc[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, br[GN_BN * GN_LD + kk], acc[1], 0, 0, 0);
            }
        }
        // lane l, register v: row 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32 of the wave's block
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t r = wm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            const int64_t c = n0 + wn * 32 + (lane & 31);
            if (r < nrows && c < a.N) {
                const float o = UP ? silu_mul(acc[0][v], acc[1][v]) : acc[0][v];
                if constexpr (sizeof(T) == 2) C[(row0 + r) * a.N + c] = f32_to_bf16(o);
                else C[(row0 + r) * a.N + c] = o;
            }
        }
    }
}

moe_status check_common(moe_dtype act_dt, const moe_plan* plan, const moe_expert_weights* w,
                        int64_t H, int64_t I) {
    MOE_CHECK_ARG(plan && w);
    MOE_CHECK_ARG(act_dt == MOE_F32 || act_dt == MOE_BF16);
    MOE_CHECK_ARG(H > 0 && I > 0);
    MOE_CHECK_ARG(plan->num_slots >= 1 && plan->num_slots <= gemm::kMaxSlots);
    MOE_CHECK_ARG(plan->counts && plan->seg_offsets && plan->num_rows && plan->cap >= 0);
    MOE_CHECK_ARG(w->w13 && w->w2);
    if (w->dtype == MOE_FP8_E4M3) {
        // block-scaled e4m3 weights take bf16 activations (kept bf16, or quantised per 1x128
        // group inside, by fp8_act)
        MOE_CHECK_ARG(w->fp8_act == MOE_FP8_ACT_BF16 || w->fp8_act == MOE_FP8_ACT_E4M3);
        if (act_dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
        MOE_CHECK_ARG(w->s13 && w->s2);
        return MOE_OK;
    }
    MOE_CHECK_ARG(w->dtype == act_dt);
    return MOE_OK;
}

// gather_rows > 0: the up GEMM gathers its rows from a [gather_rows, H] buffer
bool mfma_ok(moe_dtype act_dt, int64_t H, int64_t I, const void* A, const void* B, const void* C,
             int64_t gather_rows = 0) {
    // buffer resources cover one expert's weights and one 256-row A tile (< 4 GiB each), or
    // the whole gathered buffer (< 2 GiB, so that kAOut lies past it)
    const bool small = 2 * H * I * 2 < (int64_t(1) << 32) && int64_t(BM) * H * 2 < (int64_t(1) << 32) &&
                       int64_t(BM) * I * 2 < (int64_t(1) << 32) && gather_rows * H * 2 < (int64_t(1) << 31);
    return act_dt == MOE_BF16 && H % BN == 0 && I % UP_COLS == 0 && small && aligned(A, 16) &&
           aligned(B, 16) && aligned(C, 8);
}

// One GEMM half.  amap != NULL (up only): the gather form, A = the [arows, H] global buffer.
moe_status run_stage(bool up, const void* A, moe_dtype act_dt, const moe_plan* plan,
                     const moe_expert_weights* w, int64_t H, int64_t I, void* C, hipStream_t stream,
                     const int32_t* amap = nullptr, int32_t ak = 1, int64_t arows = 0) {
    if (plan->cap == 0) return MOE_OK;
    MOE_CHECK_ARG(A && C);
    const void* B = up ? w->w13 : w->w2;
    const int64_t K = up ? H : I;
    const int64_t N = up ? I : H;
    const bool w8 = w->dtype == MOE_FP8_E4M3;
    const bool tiles = mfma_ok(act_dt, H, I, A, B, C, amap ? arows : 0);
    // no fp8 fallback; the staged block scales hold up to kMaxKG8 K groups
    if (w8 && (!tiles || K / 128 > kMaxKG8)) return MOE_ERR_UNSUPPORTED;
    if (tiles) {
        GemmArgs g;
        g.A = static_cast<const uint16_t*>(A);
        g.B = static_cast<const uint16_t*>(B);
        g.B8 = static_cast<const uint8_t*>(B);
        g.SB = up ? w->s13 : w->s2;
        g.C = static_cast<uint16_t*>(C);
        g.counts = plan->counts;
        g.seg = plan->seg_offsets;
        g.cap = plan->cap;
        g.K = K;
        g.N = N;
        g.El = plan->num_slots;
        g.NT = static_cast<int32_t>(up ? I / UP_COLS : H / BN);
        g.amap = amap;
        g.ak = ak;
        g.arows = arows;
        g.st_hi = ST_BM_SPLIT;
        // one block per CU, 8 XCDs: a super-tile of SM x SN tiles per XCD per round
        const int blocks = gemm::grid_blocks(stream);
        gemm::TileOrder to;
        if (!gemm::pick_tile_order(g.NT, blocks, &to)) return MOE_ERR_UNSUPPORTED;
        const dim3 grid(static_cast<unsigned>(blocks));
        if (w8) {
            if (up) hipLaunchKernelGGL((grouped_gemm_pp_kernel<true, true>), grid, dim3(PP_THREADS), 0, stream, g, to);
            else hipLaunchKernelGGL((grouped_gemm_pp_kernel<false, true>), grid, dim3(PP_THREADS), 0, stream, g, to);
        } else {
            // slots of at most 64 rows stream their weights in 64-row tiles, the rest run the
            // ping-pong kernel; each kernel numbers its own slots' tiles on the device.  A slot
            // holds at most G rows (a token picks a slot once), at most seg_stride with fixed
            // capacity: when that bound is within kStreamOnlyRows the streaming kernel takes
            // every slot (a few 64-row tiles each) and the ping-pong launch, which would find
            // no tile or very few, is left out.  Both kernels give the same bits for a slot.
            const int64_t max_rows = plan->seg_stride > 0 && plan->seg_stride < plan->G ? plan->seg_stride : plan->G;
            const bool stream_only = max_rows <= kStreamOnlyRows;
            g.st_hi = stream_only ? INT64_MAX : ST_BM_SPLIT;
            if (up) hipLaunchKernelGGL((grouped_gemm_stream_kernel<true>), grid, dim3(ST_THREADS), 0, stream, g);
            else hipLaunchKernelGGL((grouped_gemm_stream_kernel<false>), grid, dim3(ST_THREADS), 0, stream, g);
            if (!stream_only) {
                MOE_LAUNCH_CHECK();
                if (up) hipLaunchKernelGGL((grouped_gemm_pp_kernel<true, false>), grid, dim3(PP_THREADS), 0, stream, g, to);
                else hipLaunchKernelGGL((grouped_gemm_pp_kernel<false, false>), grid, dim3(PP_THREADS), 0, stream, g, to);
            }
        }
        MOE_LAUNCH_CHECK();
        return MOE_OK;
    }
    GemmArgs g{};
    g.counts = plan->counts;
    g.seg = plan->seg_offsets;
    g.cap = plan->cap;
    g.K = K;
    g.N = N;
    g.El = plan->num_slots;
    g.amap = amap;
    g.ak = ak;
    g.arows = arows;
    const dim3 grid(static_cast<unsigned>(gemm::grid_blocks(stream) * 4));
    if (act_dt == MOE_BF16) {
        if (up) hipLaunchKernelGGL((generic_gemm_kernel<uint16_t, true>), grid, dim3(256), 0, stream, g, A, B, C);
        else hipLaunchKernelGGL((generic_gemm_kernel<uint16_t, false>), grid, dim3(256), 0, stream, g, A, B, C);
    } else {
        if (up) hipLaunchKernelGGL((generic_gemm_kernel<float, true>), grid, dim3(256), 0, stream, g, A, B, C);
        else hipLaunchKernelGGL((generic_gemm_kernel<float, false>), grid, dim3(256), 0, stream, g, A, B, C);
    }
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

size_t h_bytes(int64_t cap, int64_t I, moe_dtype act_dt) {
    return (static_cast<size_t>(cap * I) * dtype_size(act_dt) + 255) & ~static_cast<size_t>(255);
}

}  // namespace
}  // namespace moe

extern "C" size_t moe_expert_gemm_workspace_size(int64_t cap, int64_t H, int64_t I,
                                                 moe_dtype act_dt, moe_dtype w_dt) {
    if (cap < 0 || I <= 0 || H <= 0) return 0;
    size_t n = moe::h_bytes(cap, I, act_dt);
    if (w_dt == MOE_FP8_E4M3) {
        const size_t a = moe::gemm::fp8_stage_workspace(cap, H), b = moe::gemm::fp8_stage_workspace(cap, I);
        n += a > b ? a : b;
    }
    return n;
}

extern "C" int32_t moe_expert_gemm_fast_path(const void* x_perm, moe_dtype act_dt, const moe_expert_weights* w,
                                             int64_t H, int64_t I, const void* h, const void* y_perm) {
    if (!w || H <= 0 || I <= 0) return 0;
    return moe::mfma_ok(act_dt, H, I, x_perm, w->w13, h) && moe::mfma_ok(act_dt, H, I, h, w->w2, y_perm) ? 1 : 0;
}

extern "C" moe_status moe_expert_gemm_up(const void* x_perm, moe_dtype act_dt, const moe_plan* plan,
                                         const moe_expert_weights* w, int64_t H, int64_t I, void* h,
                                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
    moe_status st = moe::check_common(act_dt, plan, w, H, I);
    if (st != MOE_OK) return st;
    if (w->dtype == MOE_FP8_E4M3 && w->fp8_act == MOE_FP8_ACT_E4M3)
        return moe::gemm::run_fp8_stage(true, x_perm, plan, w, H, I, h, workspace, workspace_bytes, stream);
    return moe::run_stage(true, x_perm, act_dt, plan, w, H, I, h, stream);
}

extern "C" moe_status moe_expert_gemm_up_gather(const void* global_x, moe_dtype act_dt,
                                                const moe_plan* plan, const moe_expert_weights* w,
                                                int64_t H, int64_t I, void* h, void* workspace,
                                                size_t workspace_bytes, hipStream_t stream) {
    moe_status st = moe::check_common(act_dt, plan, w, H, I);
    if (st != MOE_OK) return st;
    if (plan->cap == 0) return MOE_OK;
    MOE_CHECK_ARG(plan->sorted_pair && plan->top_k >= 1 && plan->G >= 0);
    MOE_CHECK_ARG(plan->G == 0 || global_x);
    if (plan->G == 0) return MOE_OK;  // no pairs, so no rows
    if (w->dtype == MOE_FP8_E4M3 && w->fp8_act == MOE_FP8_ACT_E4M3)
        return moe::gemm::run_fp8_stage(true, global_x, plan, w, H, I, h, workspace, workspace_bytes, stream,
                                        plan->sorted_pair, plan->top_k, plan->G);
    return moe::run_stage(true, global_x, act_dt, plan, w, H, I, h, stream, plan->sorted_pair, plan->top_k,
                          plan->G);
}

extern "C" moe_status moe_expert_gemm_down(const void* h, moe_dtype act_dt, const moe_plan* plan,
                                           const moe_expert_weights* w, int64_t H, int64_t I,
                                           void* y_perm, void* workspace, size_t workspace_bytes,
                                           hipStream_t stream) {
    moe_status st = moe::check_common(act_dt, plan, w, H, I);
    if (st != MOE_OK) return st;
    if (w->dtype == MOE_FP8_E4M3 && w->fp8_act == MOE_FP8_ACT_E4M3)
        return moe::gemm::run_fp8_stage(false, h, plan, w, H, I, y_perm, workspace, workspace_bytes, stream);
    return moe::run_stage(false, h, act_dt, plan, w, H, I, y_perm, stream);
}

extern "C" moe_status moe_expert_gemm(const void* x_perm, moe_dtype act_dt, const moe_plan* plan,
                                      const moe_expert_weights* w, int64_t H, int64_t I,
                                      void* y_perm, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
    moe_status st = moe::check_common(act_dt, plan, w, H, I);
    if (st != MOE_OK) return st;
    if (plan->cap == 0) return MOE_OK;
    if (workspace_bytes < moe_expert_gemm_workspace_size(plan->cap, H, I, act_dt,
                                                         static_cast<moe_dtype>(w->dtype)))
        return MOE_ERR_CAPACITY;
    MOE_CHECK_ARG(workspace && moe::aligned(workspace, 256));
    const size_t hb = moe::h_bytes(plan->cap, I, act_dt);
    if (w->dtype == MOE_FP8_E4M3 && w->fp8_act == MOE_FP8_ACT_E4M3) {
        void* rest = static_cast<char*>(workspace) + hb;
        const size_t rest_bytes = workspace_bytes - hb;
        st = moe::gemm::run_fp8_stage(true, x_perm, plan, w, H, I, workspace, rest, rest_bytes, stream);
        if (st != MOE_OK) return st;
        return moe::gemm::run_fp8_stage(false, workspace, plan, w, H, I, y_perm, rest, rest_bytes, stream);
    }
    st = moe::run_stage(true, x_perm, act_dt, plan, w, H, I, workspace, stream);
    if (st != MOE_OK) return st;
    return moe::run_stage(false, workspace, act_dt, plan, w, H, I, y_perm, stream);
}
