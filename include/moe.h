/*
 * moe.h -- C ABI of the single-rank MoE hot path under DP attention + expert parallelism,
 * for AMD Instinct MI355X (gfx950).
 *
 * One rank's MoE layer, as the SGLang walkthrough "SGLang 源码完全拆解(十七): DP Attention
 * 与专家并行" (below: "the SGLang page") lays it out:
 *   1. gather the DP replicas' token slices into one global buffer      moe_gather_layout, moe_gather
 *      (or, fused with the layer's residual add + RMSNorm entry step,       moe_entry_gather)
 *   2. route every global token to its top-k experts                     moe_route, moe_route_from_logits
 *   3. dispatch: counting-sort the (token, k) pairs into one contiguous
 *      segment per local expert slot                                     moe_dispatch
 *   4. run the SwiGLU experts as grouped GEMMs over those segments       moe_expert_gemm (_up, _down)
 *   5. combine: weighted un-permute back to token order                  moe_combine
 *   6. scatter the global rows back to each replica's slice              moe_scatter
 * and, beside the step, the expert-load statistics and placement of EPLB   moe_expert_load,
 *   moe_physical_to_logical_count, moe_eplb_balancedness, moe_eplb_rebalance,
 *   moe_eplb_logical_to_physical
 *
 * Conventions shared by every call
 *   - All tensors are dense, row-major, contiguous.  Device pointers are HIP device memory
 *     owned by the caller; the library allocates nothing and keeps no state between calls.
 *   - Host arrays and structs passed by pointer are read before the call returns.
 *   - Work is enqueued on the given stream; no call synchronises the host with the device,
 *     so every call can be captured in a HIP graph.  Device buffers must stay alive until
 *     the stream has run the work.
 *   - Argument errors are detected on the host and returned synchronously with nothing
 *     enqueued.  A failed launch returns MOE_ERR_HIP.  Conditions that only the device can
 *     see (dispatch capacity overflow) are reported through a device flag.
 *   - Calls are reentrant; calls on different streams may run concurrently as long as
 *     they do not share output or workspace buffers.
 *   - bf16 values are IEEE binary32 numbers with the low 16 bits dropped (2 bytes each);
 *     fp8 values are OCP e4m3fn bytes.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every enum of this interface is 32 bits wide.  C++ translation units give the enums that
 * width as a fixed base type, so every int32 a C caller passes is a value of the type and the
 * library's range checks on it are well defined. */
#ifdef __cplusplus
#define MOE_ENUM_BASE : int32_t
#else
#define MOE_ENUM_BASE
#endif

typedef enum MOE_ENUM_BASE {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,  /* a pointer, size or enum value is out of range; nothing enqueued */
    MOE_ERR_UNSUPPORTED = 2,  /* a valid combination this build does not implement, or a
                                 size whose launch would need 2^32 or more work-items in one
                                 grid dimension (moe_route: G >= 2^26 rows; moe_combine:
                                 G >= 2^24 rows on the 16-byte path) */
    MOE_ERR_CAPACITY = 3,     /* a caller buffer (workspace, table) is too small */
    MOE_ERR_HIP = 4,          /* the HIP runtime refused a launch */
    MOE_ERR_SCRATCH_LIMIT = 5 /* the problem needs more than a no-allocation entry point's
                                 fixed scratch holds; nothing enqueued */
} moe_status;

typedef enum MOE_ENUM_BASE { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

/* DpPaddingMode of the SGLang page, section "DpPaddingMode：补齐到最长还是补齐到总和":
 * MAX_LEN pads every replica to the longest one, SUM_LEN concatenates the replicas. */
typedef enum MOE_ENUM_BASE { MOE_PAD_AUTO = 0, MOE_PAD_MAX_LEN = 1, MOE_PAD_SUM_LEN = 2 } moe_pad_mode;

#define MOE_MAX_REPLICAS 256

/* Resolved layout of one gather (filled by moe_gather_layout, read by gather and scatter). */
typedef struct {
    int32_t mode;                              /* MOE_PAD_MAX_LEN or MOE_PAD_SUM_LEN */
    int32_t num_replicas;                      /* W */
    int64_t rows;                              /* G: rows of the global buffer */
    int64_t offsets[MOE_MAX_REPLICAS + 1];     /* first global row of each replica slot; [W] = G */
    int32_t sizes[MOE_MAX_REPLICAS];           /* rows each replica holds (n_i, or B) */
} moe_gather_layout_t;

/* Status as text (static storage). */
const char* moe_status_string(moe_status s);
/* Library version string, e.g. "0.1.0 gfx950". */
const char* moe_version(void);

/* ------------------------------------------------------------------------------------------
 * moe_gather_layout -- host only.
 * Offsets of each replica's slice in the global buffer: prefix sums of the replica token
 * counts (SGLang page, section "本 rank 的切片位置怎么算").  mode AUTO follows the heuristic
 * of section "DpPaddingMode": prefill (is_extend) with more than one replica -> SUM_LEN,
 * unless max_len_with_idle and some replica is idle -> MAX_LEN; otherwise MAX_LEN iff
 * 2*sum >= max*W.  MAX_LEN offsets are i*max(n).  static_bound B > 0 sizes every replica B
 * and places replica i at i*B (DP note, section "跳过同步：用约定代替通信"); a count above B is
 * an error.  All replicas idle gives rows = 0: every later call is then a no-op (SGLang page,
 * section "空闲副本也必须参与").
 *   num_tokens  host int32[W], each >= 0;  1 <= W <= MOE_MAX_REPLICAS
 *   out         host struct, filled on success
 * Errors: MOE_ERR_INVALID_ARG for NULL pointers, W out of range, negative counts, counts
 * above a static bound, or a bad mode.
 * ---------------------------------------------------------------------------------------- */
moe_status moe_gather_layout(const int32_t* num_tokens, int32_t W, moe_pad_mode mode,
                             int32_t is_extend, int32_t max_len_with_idle, int32_t static_bound,
                             moe_gather_layout_t* out);

/* ------------------------------------------------------------------------------------------
 * moe_gather -- the DP gather (SGLang page, section "两种 gather：all_reduce 与 all_gather"):
 * the global buffer is zero except for each replica's rows written at its offset.  On one
 * GPU every replica buffer is local, so the write replaces the collective.
 *   L          layout from moe_gather_layout
 *   replica_x  host array of W device pointers; replica i is [sizes[i], H] of dtype dt.
 *              The pointer of a replica with 0 rows may be NULL.
 *   H          hidden size (> 0);  dt: MOE_F32 or MOE_BF16
 *   global_x   device [rows, H] dt, written in full (pad rows = 0)
 *   row_valid  device int32[rows]: 1 for a real token row, 0 for a pad row
 * ---------------------------------------------------------------------------------------- */
moe_status moe_gather(const moe_gather_layout_t* L, const void* const* replica_x, int64_t H,
                      moe_dtype dt, void* global_x, int32_t* row_valid, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * moe_entry_gather -- the layer's entry step fused with the DP gather (SGLang page, section
 * "边界判定的融合" under "两层通信怎么省": with a plain residual add and a plain RMSNorm one
 * pass writes the sum into the residual, reads the normalised FFN input and gathers it).
 * For every real row r of replica i:
 *     residual_i[r] <- round(h_i[r] + residual_i[r])                  (in place, dtype dt)
 *     global_x[offsets[i] + r] = round(residual_i[r] * norm_weight
 *                                      / sqrt(mean over H of residual_i[r]^2 + eps))
 * The norm reads the residual as stored (after rounding); sums and the mean of squares are
 * fp32.  Pad rows of the global buffer are 0, and row_valid is written as by moe_gather, so
 * this call replaces moe_gather on the path.  The attention-TP all-reduce that precedes the
 * update on a multi-GPU rank is not part of it.
 *   L                 layout from moe_gather_layout
 *   replica_h         host array of W device pointers; replica i is [sizes[i], H] of dt
 *                     (the attention output).  NULL allowed for a replica with 0 rows.
 *   replica_residual  host array of W device pointers, [sizes[i], H] of dt, read and
 *                     overwritten.  It may be the same buffer as replica_h[i] (each element
 *                     is read before it is written) but must not overlap global_x.
 *   norm_weight       device [H] of dt
 *   eps               >= 0, added to the mean of squares inside the root
 *   H, dt             hidden size (> 0); MOE_F32 or MOE_BF16
 *   global_x          device [rows, H] dt, written in full;  row_valid: device int32[rows]
 * Errors: MOE_ERR_INVALID_ARG as moe_gather, plus a NULL norm_weight or residual pointer of a
 * non-idle replica, or a negative or non-finite eps.  Rows of 16-byte-aligned buffers with
 * H * sizeof(dt) a multiple of 16 and at most 16 KiB run from registers in one read of each
 * input; any other shape takes a slower two-pass path with the same results.
 * ---------------------------------------------------------------------------------------- */
moe_status moe_entry_gather(const moe_gather_layout_t* L, const void* const* replica_h,
                            void* const* replica_residual, const void* norm_weight, float eps,
                            int64_t H, moe_dtype dt, void* global_x, int32_t* row_valid,
                            hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * moe_scatter -- the inverse of moe_gather with the same layout: y_i[r] = out[offset_i + r]
 * for r < sizes[i] (SGLang page, section "scatter：把 MoE 的输出还回本副本": the counts that
 * placed the rows also cut them).  The cross-rank sum of reduce_scatterv needs other GPUs and
 * is not part of this call.
 *   out        device [rows, H] dt
 *   replica_y  host array of W device pointers to [sizes[i], H] dt (NULL allowed if 0 rows)
 * ---------------------------------------------------------------------------------------- */
moe_status moe_scatter(const moe_gather_layout_t* L, const void* out, int64_t H, moe_dtype dt,
                       void* const* replica_y, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Routing (op_gate + op_select_experts of the SGLang page, section "operations 与 yield";
 * TopKOutput of section "normal dispatch 的调用链").
 * ---------------------------------------------------------------------------------------- */
typedef enum MOE_ENUM_BASE { MOE_ROUTE_SOFTMAX = 0, MOE_ROUTE_GROUPED_SIGMOID = 1 } moe_route_kind;

/* Gate arithmetic.  EXACT: the defined summation order below, so logits and ids are the same
 * bits on every run, every rank and the reference.  FAST: bf16 matrix-core products with fp32
 * accumulation in tile order -- the same products, summed in another order, so logits differ
 * in the last bits and an id can differ only where two keys are that close (a near tie).
 * FAST reads x once from HBM and takes bf16 inputs only. */
typedef enum MOE_ENUM_BASE { MOE_GATE_EXACT = 0, MOE_GATE_FAST = 1 } moe_gate_mode;

typedef struct {
    int32_t kind;          /* moe_route_kind */
    int32_t num_experts;   /* E (logical), 1..1024 */
    int32_t top_k;         /* k, 1..32 and <= E */
    int32_t n_group;       /* grouped: groups of E/n_group contiguous experts (E % n_group == 0) */
    int32_t topk_group;    /* grouped: groups kept, 1..n_group; k <= topk_group*E/n_group */
    int32_t group_topn;    /* grouped: keys summed per group score, 1..E/n_group (DeepSeek-V3: 2) */
    int32_t renormalize;   /* weights divided by their sum over the k picks */
    int32_t gate_mode;     /* moe_gate_mode (moe_route only; ignored by moe_route_from_logits) */
} moe_route_cfg;

/* moe_route -- gate logits then top-k selection.
 *   global_x   device [G, H] dt (MOE_F32 or MOE_BF16); row_valid device int32[G] or NULL
 *   w_router   device [E, H] dt
 *   bias       device fp32[E] or NULL (grouped only: selection bias, never in the weights)
 *   logits     device fp32[G, E], written.  EXACT mode (cfg->gate_mode): the pages fix no
 *              summation order for the gate's matrix product; this library defines one so
 *              that the integer routing is reproducible: logits[g,e] is one fp32 fused
 *              multiply-add chain over h in ascending order from +0,
 *              acc = fmaf(x[g,h], w[e,h], acc).  FAST mode: bf16 MFMA products, fp32 sums in
 *              tile order (MOE_ERR_UNSUPPORTED for MOE_F32 inputs); a batch too small to
 *              fill the GPU with 128-row tiles runs the EXACT gate instead (faster at that
 *              size, exact logits).  0 for pad rows.
 *   topk_ids   device int32[G, k]: expert ids, slots in descending key order, ties to the
 *              lower id; -1 for pad rows
 *   topk_w     device fp32[G, k]: weights; 0 for pad rows
 * Selection: softmax -- the k largest logits, weight = softmax over all E (optionally
 * renormalised).  Grouped sigmoid -- key = sigmoid(l) + bias in fp64 with a Cody-Waite exp,
 * group score = sum of the group_topn largest keys of the group, the topk_group best groups
 * are kept, then the k largest keys inside them; weight = sigmoid(l) (bias excluded),
 * optionally renormalised.  Ties go to the lower group / expert index. */
moe_status moe_route(const void* global_x, const int32_t* row_valid, int64_t G, int64_t H,
                     moe_dtype dt, const void* w_router, const float* bias,
                     const moe_route_cfg* cfg, float* logits, int32_t* topk_ids, float* topk_w,
                     hipStream_t stream);

/* moe_route_from_logits -- the selection step alone, on caller logits fp32[G, E]. */
moe_status moe_route_from_logits(const float* logits, const int32_t* row_valid, int64_t G,
                                 const float* bias, const moe_route_cfg* cfg, int32_t* topk_ids,
                                 float* topk_w, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Dispatch (get_dispatch_layout's per-expert counts, expert_alignment and the dispatch
 * "handle" of the SGLang page, section "normal dispatch 的调用链"; physical replica choice of
 * section "推理时怎么“选副本”").
 * ---------------------------------------------------------------------------------------- */
typedef struct {
    int32_t num_logical;     /* E */
    int32_t max_rep;         /* columns of phys_of */
    const int32_t* phys_of;  /* device int32[E, max_rep]: physical slots of each logical expert */
    const int32_t* n_rep;    /* device int32[E]: valid columns of each row (>= 1) */
    int32_t first_slot;      /* p0: first physical slot owned by this rank */
    int32_t num_slots;       /* E_l: slots [p0, p0+E_l) are local, 1..1024 */
} moe_expert_map;
/* A pair (g, j) with logical id l goes to physical slot phys_of[l][g mod n_rep[l]]: the same
 * choice on every rank (rank_invariant).  With phys_of == NULL the map is the identity
 * (slot l holds logical l). */

/* Two segment layouts.  Packed (seg_stride == 0, the normal dispatch of the SGLang page,
 * section "normal dispatch 的调用链"): segments back to back, each counts[e] rounded up to
 * align rows, so addresses depend on the routing.  Fixed capacity (seg_stride > 0, the
 * low-latency path's pre-allocated per-expert buffers of section "normal 与 low-latency:一对
 * 互补的模式"): slot e always owns rows [e*seg_stride, (e+1)*seg_stride), the masked
 * [E_l, seg_stride, H] layout; only the counts depend on the routing, and pairs past a slot's
 * capacity are dropped with error_flag set (the page: exceeding the fixed maximum is a
 * runtime error).  seg_stride = G can never overflow (a token picks a slot at most once). */
typedef struct {
    int32_t* counts;        /* device int32[E_l]: pairs per local slot (fixed capacity: kept
                               pairs, <= seg_stride) */
    int64_t* seg_offsets;   /* device int64[E_l+1]: segment e is rows [seg[e], seg[e+1]);
                               packed: seg[e+1] - seg[e] = counts[e] rounded up to align;
                               fixed capacity: seg[e] = e*seg_stride */
    int32_t* sorted_pair;   /* device int32[cap]: flat pair index f = g*k + j of each row,
                               ascending f inside a segment; -1 on rows past a segment's pairs */
    int32_t* pair_row;      /* device int32[G*k]: row of pair f, -1 if not local (or dropped) */
    int64_t* num_rows;      /* device int64[1]: seg[E_l] */
    int32_t* error_flag;    /* device int32[1]: 1 if num_rows > cap (rows >= cap are dropped),
                               or, with fixed capacity, if some slot had more than seg_stride pairs */
    int64_t cap;            /* rows of sorted_pair / x_perm / y_perm (fixed capacity: >= E_l*seg_stride) */
    int64_t G;              /* global rows */
    int32_t top_k;          /* k */
    int32_t num_slots;      /* E_l */
    int32_t align;          /* packed segment alignment in rows (>= 1; 128 matches the grouped
                               GEMM tile); ignored with fixed capacity */
    int32_t seg_stride;     /* 0: packed segments; > 0: fixed capacity per slot, in rows */
} moe_plan;

/* Device workspace (bytes) moe_dispatch needs for G rows, k picks and E_l slots. */
size_t moe_dispatch_workspace_size(int64_t G, int32_t k, int32_t num_slots);

/* moe_dispatch -- counts, aligned exclusive scan, stable counting sort, permuted copy.
 *   global_x  device [G, H] dt;  topk_ids device int32[G, k] (ids outside [0, E) are skipped)
 *   map       expert map (see above); plan: caller buffers, filled here
 *   x_perm    device [cap, H] dt: row r = global_x[sorted_pair[r] / k]; alignment pad rows 0;
 *             rows >= num_rows are not written, nor (fixed capacity) the unused rows of a
 *             segment past its counts[e] pairs.  NULL: the plan alone, no copy (global_x is
 *             then not read and may be NULL); moe_expert_gemm_up_gather reads the rows in place
 *   workspace device, >= moe_dispatch_workspace_size(G, k, E_l) bytes, 16-byte aligned
 * Packed: cap >= G*min(k, E_l) + E_l*(align-1) can never overflow.  Fixed capacity: cap must
 * be >= E_l*seg_stride (else MOE_ERR_INVALID_ARG), and E_l*seg_stride < 2^31. */
moe_status moe_dispatch(const void* global_x, const int32_t* topk_ids, int64_t G, int32_t k,
                        int64_t H, moe_dtype dt, const moe_expert_map* map, const moe_plan* plan,
                        void* x_perm, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of device scratch the library keeps for moe_dispatch_noalloc, one copy per GPU. */
#define MOE_DISPATCH_NOALLOC_SCRATCH_BYTES (1u << 20)

/* moe_dispatch_noalloc -- moe_dispatch for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments and results as moe_dispatch, without the workspace: the per-block count tables
 * live in a fixed device array of MOE_DISPATCH_NOALLOC_SCRATCH_BYTES that the library holds
 * on every GPU it runs on until the process ends (its address is looked up on a device's
 * first call).  The call allocates nothing.  A problem whose
 * moe_dispatch_workspace_size(G, k, E_l) exceeds the array returns MOE_ERR_SCRATCH_LIMIT
 * with nothing enqueued (at E_l = 16 slots that is G*k above about 8.3 million pairs).
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU (two
 * streams, two threads) race and give undefined plans; serialise them.  The array keeps the
 * last call's contents, which no later call depends on. */
moe_status moe_dispatch_noalloc(const void* global_x, const int32_t* topk_ids, int64_t G, int32_t k,
                                int64_t H, moe_dtype dt, const moe_expert_map* map,
                                const moe_plan* plan, void* x_perm, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Experts: per local slot e, over the rows of its segment,
 *     h = silu(x Wg[e]^T) * (x Wu[e]^T),   y = h Wd[e]^T,   silu(z) = z / (1 + e^-z)
 * gate_proj / up_proj [I, H] and down_proj [H, I] as in the SGLang page, section "EP 下专家
 * 权重切不均匀的问题"; permute, MM1, activation, MM2 in the order of the vLLM walkthrough
 * "vLLM 源码完全拆解(二十七): Dual Batch Overlap" (figure of the modular-kernel blocks).
 * ---------------------------------------------------------------------------------------- */
/* How e4m3 weights meet the activations (fp8 weights only).
 *   MOE_FP8_ACT_BF16  activations stay bf16; each weight fragment is dequantised in the kernel
 *                     (e4m3 * block scale, rounded to bf16) and the bf16 matrix cores run.
 *                     Half the weight bytes of bf16, no activation rounding.  Default.
 *   MOE_FP8_ACT_E4M3  activations are quantised per 1x128 group to e4m3 (scale = amax/448,
 *                     the per-token-group quantisation of the SGLang page, section "prefll 侧的
 *                     一个必要步骤：per-token-group 量化"), fp8 matrix cores, and each 128-deep K
 *                     group's partial sum is promoted by (activation scale * weight scale). */
typedef enum MOE_ENUM_BASE { MOE_FP8_ACT_BF16 = 0, MOE_FP8_ACT_E4M3 = 1 } moe_fp8_act;

typedef struct {
    int32_t dtype;          /* MOE_F32, MOE_BF16 (same as activations) or MOE_FP8_E4M3 */
    int32_t fp8_act;        /* fp8 weights: moe_fp8_act; ignored otherwise */
    const void* w13;        /* device [E_l, 2, I, H]: [e][0] = gate_proj, [e][1] = up_proj */
    const void* w2;         /* device [E_l, H, I]: down_proj */
    const float* s13;       /* fp8 only: device fp32[E_l, 2, I/128, H/128] block scales */
    const float* s2;        /* fp8 only: device fp32[E_l, H/128, I/128] block scales */
} moe_expert_weights;
/* fp8 weights: value = e4m3(q) * scale of its 128x128 block. */

/* moe_quant_act_fp8 -- the per-token-group activation quantisation (the SGLang page,
 * section "prefll 侧的一个必要步骤：per-token-group 量化") that moe_expert_gemm runs before each
 * product when fp8_act is MOE_FP8_ACT_E4M3, exposed on its own.  Rows [0, min(*num_rows,
 * cap)) of act are cut into groups of 128 consecutive values; per group, in fp32 with
 * correctly rounded divisions,
 *     s = amax / 448 (1 for an all-zero group),   code = e4m3 RNE of clamp(x / s, +-448)
 * (OCP e4m3fn).  The pages fix the group, not the scale rule; absmax scaling is the reading.
 *   act       device bf16 [cap, K], K a multiple of 128, 16-byte aligned
 *   num_rows  device int64[1] (read on the device; rows past it are left untouched)
 *   q         device uint8 [cap, K], 8-byte aligned: the codes
 *   s_t       device fp32 [K / 128, cap]: the scales, transposed so that one group's scales
 *             of consecutive rows are contiguous
 * Returns MOE_ERR_INVALID_ARG for K not a multiple of 128 or a null or misaligned buffer. */
moe_status moe_quant_act_fp8(const void* act, const int64_t* num_rows, int64_t cap, int64_t K,
                             uint8_t* q, float* s_t, hipStream_t stream);

/* Device workspace (bytes) moe_expert_gemm needs (the intermediate h and, for fp8 weights,
 * the quantised activations). */
size_t moe_expert_gemm_workspace_size(int64_t cap, int64_t H, int64_t I, moe_dtype act_dt,
                                      moe_dtype w_dt);

/* moe_expert_gemm -- both grouped GEMMs.
 *   x_perm    device [cap, H] act_dt (MOE_F32 or MOE_BF16), from moe_dispatch
 *   plan      the plan moe_dispatch filled (counts, seg_offsets and cap are read on the device)
 *   y_perm    device [cap, H] act_dt: rows of each segment's pairs; alignment pad rows and
 *             rows >= num_rows are not written
 *   workspace device, >= moe_expert_gemm_workspace_size(...) bytes, 256-byte aligned
 * Accumulation is fp32; h and y are rounded to act_dt (nearest even).
 * The bf16 tile kernels (bf16 matrix cores) need bf16 activations, H % 256 == 0,
 * I % 128 == 0, x_perm, h and the weights 16-byte aligned and each GEMM's output (h, y_perm)
 * 8-byte aligned.  Anything else with bf16 or fp32 weights runs a generic tiled kernel on the
 * fp32 matrix cores (any shape and alignment, at the fp32 matrix-core rate);
 * moe_expert_gemm_fast_path tells which one a call takes.  fp8 weights have no generic form:
 * they need bf16 activations, H % 256 == 0 and I % 128 == 0 in both modes (and K / 128 <= 128
 * K groups), else MOE_ERR_UNSUPPORTED; with e4m3 activations a misaligned input or weight
 * buffer is MOE_ERR_INVALID_ARG, with bf16 activations MOE_ERR_UNSUPPORTED. */
moe_status moe_expert_gemm(const void* x_perm, moe_dtype act_dt, const moe_plan* plan,
                           const moe_expert_weights* w, int64_t H, int64_t I, void* y_perm,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* moe_expert_gemm_fast_path -- 1 if moe_expert_gemm on these buffers runs the tile kernels
 * in both halves, 0 if either half runs the generic kernel (see moe_expert_gemm).  h is the
 * buffer between the halves: the caller's for moe_expert_gemm_up / _down, the workspace for
 * moe_expert_gemm.  Reads no device memory. */
int32_t moe_expert_gemm_fast_path(const void* x_perm, moe_dtype act_dt, const moe_expert_weights* w,
                                  int64_t H, int64_t I, const void* h, const void* y_perm);

/* The two halves of moe_expert_gemm, for callers that time or overlap them separately.
 *   _up:   x_perm -> h      (h: device [cap, I] act_dt, caller memory)
 *   _down: h      -> y_perm
 * With fp8 weights in MOE_FP8_ACT_E4M3 mode each half quantises its activations into the
 * workspace first. */
moe_status moe_expert_gemm_up(const void* x_perm, moe_dtype act_dt, const moe_plan* plan,
                              const moe_expert_weights* w, int64_t H, int64_t I, void* h,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);
moe_status moe_expert_gemm_down(const void* h, moe_dtype act_dt, const moe_plan* plan,
                                const moe_expert_weights* w, int64_t H, int64_t I, void* y_perm,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* moe_expert_gemm_up_gather -- moe_expert_gemm_up with the permute folded into its loads:
 * permuted row r is read straight from global_x[sorted_pair[r] / top_k] (the rows the copy of
 * moe_dispatch would have put there), so moe_dispatch can run with x_perm = NULL and the
 * copy's read and write of every routed row are saved.  The vLLM walkthrough "vLLM 源码完全拆
 * 解(二十七): Dual Batch Overlap" (figure of the modular-kernel blocks) draws permute as its
 * own block before MM1; the products are the same either way.
 *   global_x  device [plan->G, H] act_dt, the buffer moe_dispatch was given
 *   plan      as for moe_expert_gemm_up; sorted_pair, top_k and G are read as well
 *   h         device [cap, I] act_dt: bit-identical to moe_expert_gemm_up on the copied x_perm
 * Kernels, alignment rules and errors as moe_expert_gemm_up with global_x in place of x_perm
 * (moe_expert_gemm_fast_path with global_x tells the kernel), except that the bf16 tile
 * kernels here also need plan->G * H * 2 < 2^31 bytes (they address global_x through one
 * buffer resource); beyond that the generic kernel runs (fp8 weights: MOE_ERR_UNSUPPORTED). */
moe_status moe_expert_gemm_up_gather(const void* global_x, moe_dtype act_dt, const moe_plan* plan,
                                     const moe_expert_weights* w, int64_t H, int64_t I, void* h,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * moe_combine -- out[g] = routed_scale * sum_{j = 0..k-1, pair_row[g*k+j] >= 0}
 *                          topk_w[g, j] * y_perm[pair_row[g*k+j]]
 * accumulated in fp32 in ascending j and rounded once to dt; rows with no local pair are 0.
 * The top-k weights are applied after the un-permute (vLLM walkthrough, figure of the
 * modular-kernel blocks: finalize applies them; combine itself takes no weights).  A gather
 * form: each output row is written by one owner, with no atomics, so results are
 * deterministic.
 *   y_perm device [cap, H] dt; topk_w device fp32[G, k]; out device [G, H] dt
 * Rows move as 16-byte vectors (one block per row) when H is a whole number of 16-byte
 * vectors and y_perm and out are 16-byte aligned.  Otherwise the same sums run element by
 * element (one wave per row, each wave's accesses still contiguous), with 2- or 4-byte
 * accesses instead of 16-byte ones; the result is the same either way.
 * ---------------------------------------------------------------------------------------- */
moe_status moe_combine(const void* y_perm, moe_dtype dt, const moe_plan* plan,
                       const float* topk_w, float routed_scale, int64_t H, void* out,
                       hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * moe_combine_scatter -- the fused exit: moe_combine followed by moe_scatter in one pass,
 * y_i[r] = (combine row offset_i + r) for r < sizes[i], written straight into the replica's
 * buffer; the [G, H] output buffer is neither written nor read.  The same bits as the two
 * calls.  It is the exit-side counterpart of moe_entry_gather: the SGLang page's section
 * "边界判定的融合" folds the work at the layer boundary into the gather pass, and here the
 * scatter's copy is folded into the combine that produces its rows.  Pad rows of MAX_LEN
 * slots are computed nowhere (the scatter does not copy them).
 *   y_perm, dt, plan, topk_w, routed_scale, H: as for moe_combine (plan->G must equal L->rows)
 *   L          layout from moe_gather_layout (the one the gather used)
 *   replica_y  host array of W device pointers to [sizes[i], H] dt (NULL allowed if 0 rows)
 * Errors: MOE_ERR_INVALID_ARG as moe_combine and moe_scatter; MOE_ERR_UNSUPPORTED when H is
 * not a whole number of 16-byte vectors or y_perm or a replica buffer is not 16-byte aligned
 * (then use moe_combine and moe_scatter).
 * ---------------------------------------------------------------------------------------- */
moe_status moe_combine_scatter(const void* y_perm, moe_dtype dt, const moe_plan* plan,
                               const float* topk_w, float routed_scale, int64_t H,
                               const moe_gather_layout_t* L, void* const* replica_y,
                               hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Expert-load statistics and expert placement (EPLB; SGLang page, section "EPLB:专家分布不均
 * 怎么办").
 * ---------------------------------------------------------------------------------------- */

/* moe_expert_load -- token count of every physical expert slot in one step, ADDED to
 * phys_count (the caller zeroes it at the start of a statistics window).  Each valid pair
 * (row g, pick j) counts for the rank-invariant replica phys_of[id, g mod n_rep[id]], the
 * same pick moe_dispatch makes (section "推理时怎么“选副本”").  Every rank routes every token
 * when there is no all-to-all back end, so this counts the whole physical picture from one
 * rank's ids.  Ids outside [0, E) and slots outside [0, num_physical) count nowhere.
 *   topk_ids      device int32[G, k];  map: as for moe_dispatch (first_slot/num_slots unused)
 *   num_physical  P, 1..8192
 *   phys_count    device int64[P], accumulated with atomic adds (integer: order-free)
 * Errors: MOE_ERR_INVALID_ARG for NULL pointers with G > 0, k outside 1..64, P outside range. */
moe_status moe_expert_load(const int32_t* topk_ids, int64_t G, int32_t k, const moe_expert_map* map,
                           int32_t num_physical, int64_t* phys_count, hipStream_t stream);

/* moe_physical_to_logical_count -- logical_count[l, e] = sum of phys_count[l, p] over the
 * slots p with phy2log[l, p] = e (section "统计:把物理计数还原成逻辑计数"); written in full.
 *   phys_count device int64[L, P];  phy2log device int32[L, P] (entries outside [0, E) skipped)
 *   logical_count device int64[L, E], E in 1..4096 */
moe_status moe_physical_to_logical_count(const int64_t* phys_count, const int32_t* phy2log,
                                         int32_t num_layers, int32_t num_physical,
                                         int32_t num_logical, int64_t* logical_count,
                                         hipStream_t stream);

/* moe_eplb_balancedness -- host only.  Per layer, (mean + 1e-5) / (max + 1e-5) of the per-GPU
 * token counts, GPU r holding the contiguous slots [r P/M, (r+1) P/M) (section "不均衡的代价
 * 与冗余专家的思路"); 1 is perfect balance.
 *   phys_count host int64[L, P];  out host double[L].  P must be a multiple of num_gpus. */
moe_status moe_eplb_balancedness(const int64_t* phys_count, int32_t num_layers, int32_t num_physical,
                                 int32_t num_gpus, double* out);

/* moe_eplb_rebalance -- host only.  Hierarchical placement of E logical experts on P physical
 * slots (section "三步算法:分组、复制、再打包"), per layer:
 *   1. groups of E/num_groups consecutive experts are packed onto nodes by their summed load
 *      (sums in ascending expert order), num_groups/num_nodes groups per node;
 *   2. inside a node its experts get the node's P/num_nodes slots: one each, then each extra
 *      slot to the expert with the largest load per replica (ties: lower position);
 *   3. inside a node the slots are packed onto its GPUs by per-replica load (load / replica
 *      count), P/num_gpus slots per GPU.
 * Packing is greedy (the page describes it in words only): items heaviest first (ties: lower
 * index), each to the lightest pack with room (ties: lower pack).  Slot numbering: node-major,
 * then GPU, then the order the GPU received the slot.
 *   weight     host double[L, E] loads (finite, >= 0; integer counts give results independent
 *              of summation order)
 *   phy2log    host int32[L, P] out: logical expert of each slot
 *   phy_rank   host int32[L, P] out: replica index of the slot among its expert's slots
 *   log_count  host int32[L, E] out: replicas per expert (>= 1)
 * Errors: MOE_ERR_INVALID_ARG unless E % num_groups == 0, num_groups % num_nodes == 0,
 * num_gpus % num_nodes == 0, P % num_gpus == 0, P/num_nodes >= E/num_nodes, and every weight
 * is finite and >= 0. */
moe_status moe_eplb_rebalance(const double* weight, int32_t num_layers, int32_t num_logical,
                              int32_t num_physical, int32_t num_groups, int32_t num_nodes,
                              int32_t num_gpus, int32_t* phy2log, int32_t* phy_rank,
                              int32_t* log_count);

/* moe_eplb_logical_to_physical -- host only.  Dispatch table of one layer's placement
 * (section "逻辑与物理的两套映射"): phys_of[e, r] = slot of replica r of expert e, -1 past its
 * count; n_rep[e] = its replica count.  The result is the phys_of / n_rep pair of
 * moe_expert_map once copied to the device.
 *   phy2log, phy_rank  host int32[P] (one layer of moe_eplb_rebalance's output)
 *   phys_of            host int32[E, max_rep] out;  n_rep host int32[E] out
 * Errors: MOE_ERR_CAPACITY if some replica index >= max_rep; MOE_ERR_INVALID_ARG for an entry
 * outside [0, E), a repeated (expert, replica) pair, a gap in an expert's replica indices, or
 * an expert with no slot.  Outputs are unspecified after an error. */
moe_status moe_eplb_logical_to_physical(const int32_t* phy2log, const int32_t* phy_rank,
                                        int32_t num_physical, int32_t num_logical, int32_t max_rep,
                                        int32_t* phys_of, int32_t* n_rep);

/* ------------------------------------------------------------------------------------------
 * CU-partitioned streams, for running two micro-batches side by side on one GPU (the vLLM
 * walkthrough's two-micro-batch schedule gives the communication kernels a fixed share of the
 * streaming multiprocessors and the GEMMs the rest: section "第八步：SM 的分配").
 *
 * moe_stream_create_cu_masked -- a new stream, at the default priority, whose kernels run only
 * on the compute units whose bits are set in cu_mask (bit i of word i / 32 = CU i, in the
 * runtime's CU numbering).  The library's persistent kernels (the grouped GEMMs, the gate)
 * size their grids to the CUs of the stream they are launched on, so they can run on such a
 * stream.  The caller owns the stream and releases it with moe_stream_destroy.
 *   cu_mask  host uint32[words], at least one bit set;  1 <= words <= 32
 *   out      host, the new stream on success
 * Errors: MOE_ERR_INVALID_ARG for NULL pointers, words out of range or an empty mask;
 * MOE_ERR_HIP if the runtime refuses the stream.
 * ---------------------------------------------------------------------------------------- */
moe_status moe_stream_create_cu_masked(const uint32_t* cu_mask, uint32_t words, hipStream_t* out);
/* moe_stream_destroy -- releases a stream from moe_stream_create_cu_masked (after its work;
 * the runtime waits for it).  MOE_ERR_INVALID_ARG for a NULL stream. */
moe_status moe_stream_destroy(hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
