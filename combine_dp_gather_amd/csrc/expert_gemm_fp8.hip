// fp8 expert GEMMs: OCP e4m3 weights with one fp32 scale per 128x128 block, bf16
// activations quantised on the fly to e4m3 with one fp32 scale per 1x128 group.
//
// The 128-wide per-token-group activation quantisation and its block-aligned companion,
// the 128x128 weight blocks, follow the SGLang walkthrough "SGLang 源码完全拆解(十七)", section
// "prefll 侧的一个必要步骤：per-token-group 量化" (group size hard-wired to 128, matching
// expert_alignment 128).  Values: weight = e4m3(q) * s_w[block], activation ~ e4m3(q) * s_a.
//
// quant kernel: a wave per row, four 128-column groups per step (16 lanes each): amax by reduction,
//   scale s = amax / 448 (1 for an all-zero group), codes = RNE(x / s) clamped to +-448 (the
//   hardware conversion turns larger magnitudes into NaN), both in fp32 with correctly
//   rounded divisions, so every code is decided exactly as the absmax reading of the page's
//   per-token-group step defines it.  Scales are stored transposed, [K/128][cap], so a
//   tile's 256 scales of one K group are contiguous.
// GEMM kernel (gfx950 v_mfma_f32_32x32x64_f8f6f4, e4m3 x e4m3, fp32 accumulate):
//   - block tile 256 rows x 256 columns (up: 128 gate + the same 128 up columns), 8 waves
//     in 2 x 4, each 128 x 64 = 4 x 2 MFMA blocks;
//   - one pipeline stage = one 128-deep K group = one scale block: each block's MFMAs of a
//     stage accumulate into a fresh partial sum, then acc += (s_a[row] * s_w) * partial;
//   - A, B and the stage's activation scales arrive in LDS by buffer DMA, 2 stages
//     (1 in flight); 128-byte rows with 16-byte chunks xor-swizzled by (row/2) mod 8 for the
//     64-bank LDS;
//   - same persistent XCD-grouped tile order and ragged-segment numbering as the bf16 path.
#include <hip/hip_runtime.h>

#include "gemm_common.h"
#include "moe_dev.h"

namespace moe {
namespace {

typedef int intx8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int QB = 128;              // quantisation group / scale block
constexpr float kE4M3Max = 448.0f;

// ------------------------------------------------------------------ activation quant
// A wave quantises four 128-wide groups of a row per step, 16 lanes per group, 8 values per
// lane (one 16-byte load, one 8-byte store): amax by a 16-lane reduction, then the same
// per-value arithmetic as the definition above.  A row's groups past the last whole step are
// masked off.
__global__ __launch_bounds__(256) void quant_fp8_kernel(const uint16_t* __restrict__ act,
                                                        const int64_t* __restrict__ num_rows,
                                                        int64_t cap, int64_t K,
                                                        uint8_t* __restrict__ q,
                                                        float* __restrict__ s_t,
                                                        const int32_t* __restrict__ amap,
                                                        int32_t ak, int64_t arows) {
    int64_t rows = *num_rows;
    rows = rows < cap ? rows : cap;
    const int lane = lane_id();
    const int sub = lane >> 4, sl = lane & 15;  // group of the step, lane within the group
    const int64_t nw = static_cast<int64_t>(gridDim.x) * 4;
    const int64_t groups = K / QB;
    for (int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave; r < rows; r += nw) {
        // the gather form reads row amap[r] / ak of the global buffer (no row: zeros)
        int64_t srow = r;
        if (amap != nullptr) {
            const int32_t f = amap[r];
            srow = f < 0 || f / ak >= arows ? -1 : f / ak;
        }
        const uint16_t* src = act + (srow >= 0 ? srow : 0) * K;
        uint8_t* dst = q + r * K;
        for (int64_t g0 = 0; g0 < groups; g0 += 4) {
            const int64_t g = g0 + sub;
            const bool valid = g < groups;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (valid && srow >= 0) v = *reinterpret_cast<const uint4*>(src + g * QB + sl * 8);
            const uint32_t u[4] = {v.x, v.y, v.z, v.w};
            float x[8];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                x[2 * t] = __uint_as_float(u[t] << 16);
                x[2 * t + 1] = __uint_as_float(u[t] & 0xffff0000u);
            }
            float m = 0.f;
#pragma unroll
            for (int t = 0; t < 8; ++t) m = fmaxf(m, fabsf(x[t]));
#pragma unroll
            for (int off = 8; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
            const float sc = m > 0.f ? __fdiv_rn(m, kE4M3Max) : 1.f;
            uint32_t packed[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float y[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) y[t] = fminf(fmaxf(__fdiv_rn(x[4 * h + t], sc), -kE4M3Max), kE4M3Max);
                int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
                w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
                packed[h] = static_cast<uint32_t>(w);
            }
            if (valid) {
                *reinterpret_cast<uint2*>(dst + g * QB + sl * 8) = make_uint2(packed[0], packed[1]);
                if (sl == 0) s_t[g * cap + r] = sc;
            }
        }
    }
}

// ------------------------------------------------------------------ fp8 grouped GEMM
constexpr int F_BM = 256, F_BN = 256;
constexpr int F_THREADS = 512;               // 8 waves, two per SIMD
constexpr int F_STAGES = 2;
constexpr int F_ROW = 128;                   // bytes per LDS row (one K group of fp8)
constexpr int F_A_BLKS = F_BM * F_ROW / 1024;  // 1 KB DMA blocks of A per stage (32)
constexpr int F_B_BLKS = F_BN * F_ROW / 1024;  // (32)
constexpr int F_DPW = (F_A_BLKS + F_B_BLKS) / 8;  // operand DMAs per wave per stage (8)
constexpr int F_UP_COLS = F_BN / 2;          // up: 128 gate + 128 up columns
constexpr int kMaxKG8 = 128;                 // K groups whose weight scales a tile stages (K <= 16384)

__device__ __forceinline__ int fswz(int row) { return (row >> 1) & 7; }

struct Fp8Args {
    const uint8_t* A;       // [cap, K] e4m3 activations
    const float* SA;        // [K/128, cap] activation scales
    const uint8_t* B;       // up: w13 [E_l, 2, I, H]; down: w2 [E_l, H, I]
    const float* SB;        // up: s13 [E_l, 2, I/128, H/128]; down: s2 [E_l, H/128, I/128]
    uint16_t* C;            // up: h [cap, I] bf16; down: y [cap, H] bf16
    const int32_t* counts;
    const int64_t* seg;
    int64_t cap, K, N;      // up: K=H, N=I; down: K=I, N=H
    int32_t El, NT;
};

__device__ __forceinline__ float silu_mul8(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// 8 waves in a 2 x 4 grid over the 256 x 256 tile: wave w owns rows 128 (w mod 2) .. + 127
// and column group w / 2 (up: gate block w / 2 of 32 columns and the same up block; down:
// 64 columns, blocks 2 (w / 2), + 1): 4 x 2 accumulator blocks of 32 x 32, 128 per lane.
// The weight fragment is the MFMAs' first operand, so a block's lane holds one token row
// (lane mod 32) and four consecutive output columns per register group: one activation scale
// per lane and row block, one weight scale per column block, and 8-byte output stores.  A
// stage is one 128-deep K group (A and B 32 KB each, plus the group's 256 activation
// scales); the group's two MFMAs per block accumulate into a fresh partial that is promoted
// at once (acc += partial * s_a * s_w), so no second set of accumulators is held.  The
// activation fragments are read one row block ahead of its MFMAs (32 registers), the weight
// fragments for the whole group (32).  Two stages: group kg + 1 is DMA'd while group kg is
// consumed; one barrier per group.
template <bool UP>
__global__ __launch_bounds__(F_THREADS, 1) void grouped_gemm_fp8_kernel(Fp8Args a, gemm::TileOrder to) {
    __shared__ __attribute__((aligned(1024))) uint8_t As[F_STAGES][F_BM * F_ROW];
    __shared__ __attribute__((aligned(1024))) uint8_t Bs[F_STAGES][F_BN * F_ROW];
    __shared__ __attribute__((aligned(16))) float Ss[F_STAGES][F_BM];
    __shared__ int32_t tile_prefix[gemm::kMaxSlots + 1];
    __shared__ int32_t part[F_THREADS];
    __shared__ float sw_lds[2][kMaxKG8];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv & 1, wn = wv >> 1;

    const int32_t total_mt = gemm::number_tiles<F_BM, F_THREADS>(a.counts, a.seg, a.cap, a.El, tile_prefix, part);
    const uint32_t row_bytes = static_cast<uint32_t>(a.K);
    const int64_t KG = a.K / QB;  // K groups = pipeline steps
    const int64_t SKG = a.N / QB;  // weight scale blocks along the output dimension
    const int nsn = a.NT / to.SN;
    const int64_t total_super = static_cast<int64_t>((total_mt + to.SM - 1) / to.SM) * nsn;
    const int xcd = blockIdx.x & 7;
    const int q = blockIdx.x >> 3;
    const int frow = lane & 31;
    // fragment bytes of MFMA step ks: 64 ks + 32 (lane / 32) .. + 32 = logical chunks c, c + 1
    int fch[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int h = 0; h < 2; ++h) fch[ks][h] = ((4 * ks + 2 * (lane >> 5) + h) ^ fswz(frow)) * 16;

    for (int64_t sup = xcd; sup < total_super; sup += 8) {
        const int32_t em = static_cast<int32_t>(sup / nsn) * to.SM + q / to.SN;
        const int32_t nt = static_cast<int32_t>(sup % nsn) * to.SN + q % to.SN;
        if (em >= total_mt) continue;
        const int e = gemm::slot_of_tile(tile_prefix, a.El, em);
        const int32_t mtile = __builtin_amdgcn_readfirstlane(em - tile_prefix[e]);
        const int64_t seg_start = a.seg[e];
        int64_t seg_end = seg_start + a.counts[e];
        seg_end = seg_end < a.cap ? seg_end : a.cap;
        const int64_t row0 = seg_start + static_cast<int64_t>(mtile) * F_BM;
        const int64_t nrows64 = seg_end - row0;
        const uint32_t nrows = static_cast<uint32_t>(nrows64 < F_BM ? nrows64 : F_BM);

        // descriptors: A rows of this tile (rows past the segment end read as zeros), this
        // slot's weights, and the activation scales from row0 to the end of the array
        const __amdgpu_buffer_rsrc_t ra = gemm::make_rsrc_uniform(a.A + row0 * a.K, nrows * row_bytes);
        const int64_t wslot = UP ? 2 * a.N * a.K : a.N * a.K;
        const __amdgpu_buffer_rsrc_t rb = gemm::make_rsrc_uniform(a.B + e * wslot, static_cast<uint32_t>(wslot));
        const __amdgpu_buffer_rsrc_t rs = gemm::make_rsrc_uniform(
            a.SA + row0, static_cast<uint32_t>((KG * a.cap - row0) * 4));
        // per-lane DMA offsets: A blocks 4w..4w+3 (rows 32 w ..), B blocks 4w..4w+3 (B tile rows
        // 32 w ..: up, waves 0-3 gate rows, 4-7 up rows); waves 0-3 also DMA 64 scales each
        uint32_t aoff[4], boff[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int r = (wv * 4 + p) * 8 + (lane >> 3);
            aoff[p] = static_cast<uint32_t>(r) * row_bytes + static_cast<uint32_t>(((lane & 7) ^ fswz(r)) * 16);
            uint32_t grow;
            if (UP) grow = static_cast<uint32_t>((r >> 7) * a.N + nt * F_UP_COLS + (r & (F_UP_COLS - 1)));
            else grow = static_cast<uint32_t>(nt * F_BN + r);
            boff[p] = grow * row_bytes + static_cast<uint32_t>(((lane & 7) ^ fswz(r)) * 16);
        }
        // the scale DMA carries its K-group offset in the per-lane offset, so the descriptor's
        // range check sees it (rows at or past cap in the last group read as zeros)
        const bool sdma = wv < 4;
        const uint32_t soff_lane = static_cast<uint32_t>((wv * 64 + lane) * 4);
        const uint32_t scap_bytes = static_cast<uint32_t>(a.cap * 4);
        // The LDS destinations are made opaque to the compiler: its wait tracking would
        // otherwise treat every later LDS read as dependent on every DMA in flight and drain
        // the next group's DMAs before this group's fragment reads.  The barrier protocol
        // below orders them instead.
        typedef __attribute__((address_space(3))) uint8_t lds_u8;
        auto issue = [&](int buf, int64_t kg) {
            lds_u8* ad = (lds_u8*)(&As[0][0] + buf * (F_BM * F_ROW) + wv * 4 * 1024);
            lds_u8* bd = (lds_u8*)(&Bs[0][0] + buf * (F_BN * F_ROW) + wv * 4 * 1024);
            lds_u8* sd = (lds_u8*)(&Ss[0][0] + buf * F_BM + wv * 64);
            asm volatile("" : "+s"(ad), "+s"(bd), "+s"(sd));
            const int koff = static_cast<int>(kg * QB);
#pragma unroll
            for (int p = 0; p < 4; ++p)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (gemm::lds_void_t*)(ad + p * 1024), 16, aoff[p], koff, 0, 0);
#pragma unroll
            for (int p = 0; p < 4; ++p)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (gemm::lds_void_t*)(bd + p * 1024), 16, boff[p], koff, 0, 0);
            if (sdma)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (gemm::lds_void_t*)sd, 4,
                                                        soff_lane + static_cast<uint32_t>(kg) * scap_bytes, 0, 0, 0);
        };
        // the tile's weight block scales along K, staged in LDS: up -> gate (0) and up (1)
        // halves of i-block nt; down -> the two 128-column blocks of the tile
        for (int t = tid; t < 2 * KG; t += F_THREADS) {
            const int r = t / static_cast<int>(KG), kgi = t % static_cast<int>(KG);
            sw_lds[r][kgi] = UP ? a.SB[((static_cast<int64_t>(e) * 2 + r) * SKG + nt) * KG + kgi]
                                : a.SB[(static_cast<int64_t>(e) * SKG + 2 * nt + r) * KG + kgi];
        }
        // weight block scale of the wave's column block j for K group kg
        auto wscale = [&](int j, int64_t kg) -> float { return sw_lds[UP ? j : (wn >> 1)][kg]; };

        floatx16_t acc[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
        const floatx16_t zero = {};

        const uint8_t* a_rd = &As[0][0] + (wm * 128 + frow) * F_ROW;
        // B rows of the wave's two column blocks
        const int brow0 = UP ? wn * 32 : wn * 64;
        const int brow1 = UP ? F_UP_COLS + wn * 32 : wn * 64 + 32;
        const uint8_t* b_rd0 = &Bs[0][0] + (brow0 + frow) * F_ROW;
        const uint8_t* b_rd1 = &Bs[0][0] + (brow1 + frow) * F_ROW;
        // the lane's token row in row block i: wm*128 + 32 i + lane mod 32
        const float* s_rd = &Ss[0][0] + wm * 128 + frow;
        auto read8 = [&](const uint8_t* p, int ks) -> intx8_t {
            const gemm::v4i_t lo = *reinterpret_cast<const gemm::v4i_t*>(p + fch[ks][0]);
            const gemm::v4i_t hi = *reinterpret_cast<const gemm::v4i_t*>(p + fch[ks][1]);
            return intx8_t{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        };

        // the previous tile's stores and reads, and this tile's scale staging, are done; the
        // intrinsic form keeps the compiler's wait tracking from carrying the epilogue's
        // stores into the K loop
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        issue(0, 0);
        for (int64_t kg = 0; kg < KG; ++kg) {
            const int cur = static_cast<int>(kg & 1);
            // group kg landed for this wave (nothing else is in flight); after the barrier for
            // every wave, and every wave is done with group kg - 1's stage, refilled next
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            issue(cur ^ 1, kg + 1 < KG ? kg + 1 : KG - 1);
            intx8_t fb[2][2], fa[2][2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                fb[0][ks] = read8(b_rd0 + cur * (F_BN * F_ROW), ks);
                fb[1][ks] = read8(b_rd1 + cur * (F_BN * F_ROW), ks);
                fa[0][ks] = read8(a_rd + cur * (F_BM * F_ROW), ks);
            }
            float sa[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) sa[i] = s_rd[cur * F_BM + 32 * i];
            const float sw0 = wscale(0, kg), sw1 = wscale(1, kg);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = i & 1;
                if (i + 1 < 4) {
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        fa[c ^ 1][ks] = read8(a_rd + cur * (F_BM * F_ROW) + (i + 1) * 32 * F_ROW, ks);
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    floatx16_t t = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j][0], fa[c][0], zero,
                                                                                   0, 0, 0, 0, 0, 0);
                    t = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j][1], fa[c][1], t, 0, 0, 0, 0, 0, 0);
                    const float sc = sa[i] * (j ? sw1 : sw0);
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[i][j][v] = __builtin_fmaf(sc, t[v], acc[i][j][v]);
                }
            }
        }
        // epilogue: in block (i, j) the lane holds token row wm*128 + 32 i + lane mod 32 and,
        // for g = 0..3, columns 8 g + 4 (lane / 32) + 0..3 of the block: one 8-byte store each
        const int rloc = wm * 128 + frow;
        const int64_t colbase = UP ? static_cast<int64_t>(nt) * F_UP_COLS + wn * 32 + (lane >> 5) * 4
                                   : static_cast<int64_t>(nt) * F_BN + wn * 64 + (lane >> 5) * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (rloc + i * 32 >= static_cast<int>(nrows)) continue;
            uint16_t* cp = a.C + (row0 + rloc + i * 32) * a.N + colbase;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                if (UP) {
                    float h[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) h[u] = silu_mul8(acc[i][0][4 * g + u], acc[i][1][4 * g + u]);
                    *reinterpret_cast<uint2*>(cp + g * 8) = make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
                } else {
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const floatx16_t& c = acc[i][j];
                        *reinterpret_cast<uint2*>(cp + j * 32 + g * 8) =
                            make_uint2(pack_bf16x2(c[4 * g], c[4 * g + 1]), pack_bf16x2(c[4 * g + 2], c[4 * g + 3]));
                    }
                }
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

moe_status launch_quant(const void* act, const int64_t* num_rows, int64_t cap, int64_t K, uint8_t* q,
                        float* s_t, hipStream_t stream, const int32_t* amap = nullptr, int32_t ak = 1,
                        int64_t arows = 0) {
    int64_t qblocks = ceil_div(cap, 4);
    if (qblocks > 4096) qblocks = 4096;
    hipLaunchKernelGGL(quant_fp8_kernel, dim3(static_cast<unsigned>(qblocks)), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(act), num_rows, cap, K, q, s_t, amap, ak, arows);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

}  // namespace

namespace gemm {

size_t fp8_stage_workspace(int64_t cap, int64_t K) {
    return align256(static_cast<size_t>(cap * K)) + align256(static_cast<size_t>(K / QB * cap) * 4);
}

moe_status run_fp8_stage(bool up, const void* act, const moe_plan* plan,
                         const moe_expert_weights* w, int64_t H, int64_t I, void* out,
                         void* workspace, size_t ws_bytes, hipStream_t stream,
                         const int32_t* amap, int32_t ak, int64_t arows) {
    if (plan->cap == 0) return MOE_OK;
    const int64_t K = up ? H : I, N = up ? I : H;
    if (H % F_BN != 0 || I % QB != 0) return MOE_ERR_UNSUPPORTED;  // whole 256-column down tiles
    if (K / QB > kMaxKG8) return MOE_ERR_UNSUPPORTED;              // the staged weight scales
    if (2 * H * I >= (int64_t(1) << 32) || int64_t(F_BM) * K >= (int64_t(1) << 32) ||
        plan->cap * (K / QB) * 4 >= (int64_t(1) << 32))
        return MOE_ERR_UNSUPPORTED;  // descriptor ranges are 32-bit
    MOE_CHECK_ARG(act && out && w->s13 && w->s2);
    MOE_CHECK_ARG(aligned(act, 16) && aligned(w->w13, 16) && aligned(w->w2, 16));
    if (ws_bytes < fp8_stage_workspace(plan->cap, K)) return MOE_ERR_CAPACITY;
    MOE_CHECK_ARG(workspace && aligned(workspace, 256));
    uint8_t* qa = static_cast<uint8_t*>(workspace);
    float* sa = reinterpret_cast<float*>(qa + align256(static_cast<size_t>(plan->cap * K)));
    const moe_status qs = launch_quant(act, plan->num_rows, plan->cap, K, qa, sa, stream, amap, ak, arows);
    if (qs != MOE_OK) return qs;
    Fp8Args g;
    g.A = qa;
    g.SA = sa;
    g.B = static_cast<const uint8_t*>(up ? w->w13 : w->w2);
    g.SB = up ? w->s13 : w->s2;
    g.C = static_cast<uint16_t*>(out);
    g.counts = plan->counts;
    g.seg = plan->seg_offsets;
    g.cap = plan->cap;
    g.K = K;
    g.N = N;
    g.El = plan->num_slots;
    g.NT = static_cast<int32_t>(up ? I / F_UP_COLS : H / F_BN);
    const int blocks = grid_blocks(stream);
    TileOrder to;
    if (!pick_tile_order(g.NT, blocks, &to)) return MOE_ERR_UNSUPPORTED;
    const dim3 grid(static_cast<unsigned>(blocks));
    if (up) hipLaunchKernelGGL(grouped_gemm_fp8_kernel<true>, grid, dim3(F_THREADS), 0, stream, g, to);
    else hipLaunchKernelGGL(grouped_gemm_fp8_kernel<false>, grid, dim3(F_THREADS), 0, stream, g, to);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
}

}  // namespace gemm
}  // namespace moe

extern "C" moe_status moe_quant_act_fp8(const void* act, const int64_t* num_rows, int64_t cap, int64_t K,
                                        uint8_t* q, float* s_t, hipStream_t stream) {
    MOE_CHECK_ARG(cap >= 0 && K > 0 && K % moe::QB == 0);
    if (cap == 0) return MOE_OK;
    MOE_CHECK_ARG(act && num_rows && q && s_t);
    MOE_CHECK_ARG(moe::aligned(act, 16) && moe::aligned(q, 8));
    return moe::launch_quant(act, num_rows, cap, K, q, s_t, stream);
}

