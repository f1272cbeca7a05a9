"""CPU oracle of the single-rank MoE hot path -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (``combine_dp_gather_amd``)
never does, and this package imports nothing from it.

Every step is a plain definition: integer work in C (``moe_oracle.c``: exact gate
logits, top-k selection, the dispatch counting sort) and floating-point expert
maths in numpy float64.  Pages followed:

* the SGLang walkthrough "SGLang 源码完全拆解(十七): DP Attention 与专家并行"
  (below: "the SGLang page"),
* the vLLM walkthrough "vLLM 源码完全拆解(二十七): Dual Batch Overlap" ("the vLLM page"),
* the DP note at zdszero.github.io ("DP"), section "跳过同步：用约定代替通信".

Pinned by ``tests/test_oracle_*.py`` against brute force, closed forms, library
routines (stable sort, float64 matmul) and invariants; see each function.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

MAX_LEN, SUM_LEN = "max", "sum"


def build(force: bool = False) -> str:
    """Compile moe_oracle.c with gcc (no fast-math, no contraction, OpenMP)."""
    stale = (not os.path.exists(_LIB_PATH)) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    if force or stale:
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                               "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64, i32, d = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        lib.oracle_gate_logits.argtypes = [P, P, P, i64, i64, i64, P]
        lib.oracle_exp.argtypes = [d]
        lib.oracle_exp.restype = d
        lib.oracle_sigmoid.argtypes = [d]
        lib.oracle_sigmoid.restype = d
        lib.oracle_select_softmax.argtypes = [P, P, i64, i32, i32, i32, P, P]
        lib.oracle_select_grouped.argtypes = [P, P, P, i64, i32, i32, i32, i32, i32, i32, P, P]
        lib.oracle_dispatch.argtypes = [P, i64, i32, P, P, i32, i32, i32, i32, i32, i64,
                                        P, P, P, P, P, P]
        lib.oracle_e4m3_decode.argtypes = [P, i64, P]
        _lib = lib
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ============================================================================ O1 gather layout

def gather_layout(num_tokens: Sequence[int], mode: str = "auto", is_extend: bool = False,
                  max_len_with_idle: bool = False, static_bound: int = 0):
    """Global-buffer layout of one DP gather.  Returns (mode, G, offsets[W+1], sizes[W]).

    * offsets: prefix sums of the replica token counts (SGLang page, section
      "本 rank 的切片位置怎么算": replica i starts at the sum of the counts before it).
    * MAX_LEN pads every replica to max(n); SUM_LEN concatenates (section
      "DpPaddingMode：补齐到最长还是补齐到总和").  MAX_LEN offsets are i*max(n).
    * auto: prefill with more than one replica -> SUM_LEN, unless max_len_with_idle and
      some replica is idle -> MAX_LEN; otherwise MAX_LEN iff 2*sum >= max*width
      (the cost rule of the same section; back-end specific branches dropped).
    * static_bound B > 0: every replica counts as B tokens and the offset of
      replica i is i*B (DP note, section "跳过同步：用约定代替通信").
    * all replicas idle: G = 0, nothing runs (SGLang page, section "空闲副本也必须参与").
    """
    n = [int(v) for v in num_tokens]
    W = len(n)
    if W == 0 or any(v < 0 for v in n):
        raise ValueError("bad num_tokens")
    if static_bound > 0:
        if any(v > static_bound for v in n):
            raise ValueError("replica exceeds the static bound")
        n = [static_bound] * W
    mx, sm = max(n), sum(n)
    if mode == "auto":
        if is_extend and W > 1:
            mode = MAX_LEN if (max_len_with_idle and min(n) == 0) else SUM_LEN
        else:
            mode = MAX_LEN if sm * 2 >= mx * W else SUM_LEN
    if mode not in (MAX_LEN, SUM_LEN):
        raise ValueError(mode)
    if sm == 0:
        return mode, 0, [0] * (W + 1), n
    if mode == SUM_LEN:
        offs = [0]
        for v in n:
            offs.append(offs[-1] + v)
        return mode, sm, offs, n
    return mode, W * mx, [i * mx for i in range(W + 1)], n


def gather(layout, replicas: Sequence[np.ndarray], H: int, dtype) -> tuple:
    """global[off_i + r] = x_i[r] for r < n_i; every other row 0 with row_valid 0
    (SGLang page, section "两种 gather": zero the buffer, then write each slice at its
    offset)."""
    mode, G, offs, sizes = layout
    glob = np.zeros((G, H), dtype=dtype)
    valid = np.zeros(G, dtype=np.int32)
    for i, x in enumerate(replicas):
        ni = sizes[i]
        if ni == 0:
            continue
        glob[offs[i]:offs[i] + ni] = x[:ni]
        valid[offs[i]:offs[i] + ni] = 1
    return glob, valid


def scatter(layout, out: np.ndarray) -> List[np.ndarray]:
    """y_i[r] = out[off_i + r] for r < n_i: the inverse of gather with the same counts
    (SGLang page, section "scatter：把 MoE 的输出还回本副本").  One GPU holds the whole
    expert set of this rank, so no cross-rank sum takes place."""
    mode, G, offs, sizes = layout
    return [out[offs[i]:offs[i] + sizes[i]].copy() for i in range(len(sizes))]


# ============================================================================ O0 fused entry step

def bf16_rne(a: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns, round to nearest with ties to even, taken straight from
    the float64 value (no float32 step, so no double rounding).  Non-zero inputs must lie in
    bf16's normal range; the step never produces anything else on these workloads."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    mag = np.abs(a)
    if not np.all(np.isfinite(a)) or np.any((mag != 0) & ((mag < 2.0 ** -126) | (mag >= 2.0 ** 128))):
        raise ValueError("bf16_rne: value outside bf16's normal range")
    u = a.view(np.uint64)
    # keep the top 7 of float64's 52 stored fraction bits: add just under half of the
    # dropped range, plus the kept lowest bit (ties to even), then clear the dropped bits
    drop = np.uint64(45)
    keep_lsb = (u >> drop) & np.uint64(1)
    r = (u + np.uint64((1 << 44) - 1) + keep_lsb) & ~np.uint64((1 << 45) - 1)
    v = r.view(np.float64)
    if np.any(np.abs(v) >= 2.0 ** 128):
        raise ValueError("bf16_rne: rounds past bf16's largest value")
    # v has at most 8 significant bits and a float32 exponent: float32 holds it exactly
    return (v.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def entry_gather(layout, hidden: Sequence[Optional[np.ndarray]], residual: Sequence[Optional[np.ndarray]],
                 gamma: np.ndarray, eps: float, H: int):
    """The layer's entry step fused with the DP gather, on one replica set.

    SGLang page, section "边界判定的融合" (under "两层通信怎么省"): when the residual update
    is a plain add and the norm a plain RMSNorm, one pass writes the sum into the residual,
    reads the normalised FFN input from it, and gathers that input; the attention-TP sum owed
    before it has no counterpart on one rank.  Per replica row (plain readings):

        residual <- round(hidden + residual)          (the stored dtype; the sum is exact in float64)
        x        =  residual * gamma / sqrt(mean_h(residual^2) + eps)

    RMSNorm is the plain definition (root mean square over the hidden dimension, eps inside
    the root, an elementwise weight); it reads the residual as stored, i.e. after rounding.

    Returns (x_global float64 [G, H], row_valid int32 [G], new residuals in the input dtype,
    one per replica; None for idle replicas).  Pad rows of x_global are 0."""
    mode, G, offs, sizes = layout
    g = as_f32(gamma).astype(np.float64)
    new_res, normed = [], []
    for i in range(len(sizes)):
        n = sizes[i]
        if n == 0:
            new_res.append(None)
            normed.append(None)
            continue
        h, r = hidden[i][:n], residual[i][:n]
        bf = np.asarray(r).dtype == np.uint16
        s = as_f32(h).astype(np.float64) + as_f32(r).astype(np.float64)
        rq = bf16_rne(s) if bf else s.astype(np.float32)
        rv = as_f32(rq).astype(np.float64)
        ms = np.mean(rv * rv, axis=1, keepdims=True)
        normed.append(rv / np.sqrt(ms + float(eps)) * g)
        new_res.append(rq.reshape(n, H))
    gx, valid = gather(layout, [np.zeros((0, H)) if y is None else y for y in normed], H, np.float64)
    return gx, valid, new_res


# ============================================================================ O2 routing

def as_f32(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) or fp32 -> fp32 (exact)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return np.ascontiguousarray(a, dtype=np.float32)


def gate_logits(x: np.ndarray, w: np.ndarray, row_valid: Optional[np.ndarray] = None) -> np.ndarray:
    """fp32 router logits: one fmaf chain per (g, e) in ascending h from +0 (see
    moe_oracle.c); 0 for rows with row_valid == 0."""
    lib = _load()
    xf, wf = as_f32(x), as_f32(w)
    G, H = xf.shape
    E = wf.shape[0]
    out = np.empty((G, E), dtype=np.float32)
    rv = None if row_valid is None else np.ascontiguousarray(row_valid, dtype=np.int32)
    if G:
        lib.oracle_gate_logits(_p(xf), _p(wf), _p(rv), G, E, H, _p(out))
    return out


def exp_defined(x: float) -> float:
    return _load().oracle_exp(float(x))


def sigmoid_defined(x: float) -> float:
    return _load().oracle_sigmoid(float(x))


def select_softmax(logits: np.ndarray, k: int, renormalize: bool = False,
                   row_valid: Optional[np.ndarray] = None):
    lib = _load()
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    G, E = lg.shape
    ids = np.empty((G, k), dtype=np.int32)
    w = np.empty((G, k), dtype=np.float32)
    rv = None if row_valid is None else np.ascontiguousarray(row_valid, dtype=np.int32)
    if G:
        lib.oracle_select_softmax(_p(lg), _p(rv), G, E, k, int(renormalize), _p(ids), _p(w))
    return ids, w


def select_grouped(logits: np.ndarray, bias: Optional[np.ndarray], n_group: int, topk_group: int,
                   k: int, renormalize: bool = True, group_topn: int = 2,
                   row_valid: Optional[np.ndarray] = None):
    lib = _load()
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    G, E = lg.shape
    assert E % n_group == 0
    ids = np.empty((G, k), dtype=np.int32)
    w = np.empty((G, k), dtype=np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    rv = None if row_valid is None else np.ascontiguousarray(row_valid, dtype=np.int32)
    if G:
        lib.oracle_select_grouped(_p(lg), _p(b), _p(rv), G, E, n_group, topk_group, group_topn,
                                  k, int(renormalize), _p(ids), _p(w))
    return ids, w


def route(cfg, x: np.ndarray, row_valid: np.ndarray, router_w: np.ndarray, bias):
    """Gate logits then the config's selection rule."""
    logits = gate_logits(x, router_w, row_valid)
    if cfg.route == "softmax":
        ids, w = select_softmax(logits, cfg.top_k, cfg.renormalize, row_valid)
    else:
        ids, w = select_grouped(logits, bias, cfg.n_group, cfg.topk_group, cfg.top_k,
                                cfg.renormalize, cfg.group_topn, row_valid)
    return logits, ids, w


# ============================================================================ O3 dispatch

def dispatch(ids: np.ndarray, phys_of: np.ndarray, n_rep: np.ndarray, p0: int, El: int,
             align: int = 1, cap: Optional[int] = None) -> dict:
    """Counting-sort plan for the rank's slots (see oracle_dispatch in moe_oracle.c)."""
    lib = _load()
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    G, k = ids.shape
    P = G * k
    if cap is None:
        cap = G * min(k, El) + El * (align - 1)
    phys = np.ascontiguousarray(phys_of, dtype=np.int32)
    nrep = np.ascontiguousarray(n_rep, dtype=np.int32)
    E, max_rep = phys.shape
    counts = np.zeros(El, dtype=np.int32)
    seg = np.zeros(El + 1, dtype=np.int64)
    sorted_pair = np.full(max(cap, 1), -2, dtype=np.int32)
    pair_row = np.full(max(P, 1), -2, dtype=np.int32)
    num_rows = np.zeros(1, dtype=np.int64)
    err = np.zeros(1, dtype=np.int32)
    lib.oracle_dispatch(_p(ids), G, k, _p(phys), _p(nrep), max_rep, E, p0, El, align, cap,
                        _p(counts), _p(seg), _p(sorted_pair), _p(pair_row), _p(num_rows), _p(err))
    rows = int(min(num_rows[0], cap))
    return dict(counts=counts, seg_offsets=seg, sorted_pair=sorted_pair[:rows],
                pair_row=pair_row[:P], num_rows=int(num_rows[0]), error_flag=int(err[0]),
                cap=int(cap), k=k)


def dispatch_masked(ids: np.ndarray, phys_of: np.ndarray, n_rep: np.ndarray, p0: int, El: int,
                    stride: int) -> dict:
    """Fixed-capacity ("masked") plan: slot e owns rows [e * stride, (e + 1) * stride) whatever
    the routing, as the low-latency path's pre-allocated per-expert buffers do (SGLang page,
    section "normal 与 low-latency:一对互补的模式": a fixed maximum per expert, exceeding it is a
    runtime error).  The slot's pairs fill its rows in ascending flat index; pairs past the
    stride are dropped (pair_row -1) and raise error_flag; counts are the rows filled; the
    rest of each segment is -1 in sorted_pair.  num_rows = El * stride."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    G, k = ids.shape
    P = G * k
    E = phys_of.shape[0]
    sorted_pair = np.full(El * stride, -1, dtype=np.int32)
    pair_row = np.full(P, -1, dtype=np.int32)
    counts = np.zeros(El, dtype=np.int32)
    err = 0
    for f in range(P):
        l = int(ids.flat[f])
        if l < 0 or l >= E:
            continue
        p = int(phys_of[l, (f // k) % int(n_rep[l])]) - p0
        if p < 0 or p >= El:
            continue
        if counts[p] < stride:
            row = p * stride + int(counts[p])
            sorted_pair[row] = f
            pair_row[f] = row
            counts[p] += 1
        else:
            err = 1
    seg = np.arange(El + 1, dtype=np.int64) * stride
    return dict(counts=counts, seg_offsets=seg, sorted_pair=sorted_pair, pair_row=pair_row,
                num_rows=El * stride, error_flag=err, cap=El * stride, k=k)


def permute_rows(global_x: np.ndarray, plan: dict) -> np.ndarray:
    """x_perm[row] = global_x[sorted_pair[row] // k]; alignment pad rows are 0."""
    sp = plan["sorted_pair"]
    xp = np.zeros((len(sp),) + global_x.shape[1:], dtype=global_x.dtype)
    m = sp >= 0
    xp[m] = global_x[sp[m] // plan["k"]]
    return xp


# ============================================================================ O4 SwiGLU experts

def e4m3_decode(q: np.ndarray) -> np.ndarray:
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.uint8)
    out = np.empty(q.shape, dtype=np.float64)
    lib.oracle_e4m3_decode(_p(q), q.size, _p(out))
    return out


def dequant_block(q: np.ndarray, s: np.ndarray, block: int = 128) -> np.ndarray:
    """value = e4m3(q) * scale[r // 128, c // 128], exact in float64."""
    v = e4m3_decode(q)
    return v * np.repeat(np.repeat(s.astype(np.float64), block, axis=-2), block, axis=-1)


E4M3_MAX = 448.0
ACT_GROUP = 128


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """OCP e4m3fn code of each value (|v| <= 448), rounded to nearest, ties to even.  A
    binade [2^e, 2^(e+1)) with e >= -6 holds 8 codes 2^(e-3) apart; below 2^-6 the codes are
    the multiples of 2^-9 (subnormals).  The sign bit is kept, so -0 encodes as 0x80."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(a > E4M3_MAX) or np.any(np.isnan(v)):
        raise ValueError("e4m3_encode takes finite values within +-448")
    _, ex = np.frexp(a)                         # a = m 2^ex, m in [0.5, 1)
    e = np.maximum(ex - 1, -6)                  # binade of a (subnormals share e = -6)
    step = np.ldexp(1.0, e - 3)
    n = np.rint(a / step)                       # a / step is exact; rint rounds ties to even
    mag = n * step                              # rounded magnitude (may carry to 2^(e+1))
    _, ex2 = np.frexp(mag)
    e2 = ex2 - 1
    normal = mag >= 2.0 ** -6
    mant = np.where(normal, np.rint(mag / np.ldexp(1.0, np.where(normal, e2, 0) - 3)) - 8, 0)
    field = np.where(normal, ((e2 + 7) << 3) + mant, np.rint(mag / 2.0 ** -9))
    return (field.astype(np.uint8) | (np.signbit(v).astype(np.uint8) << 7)).astype(np.uint8)


def quant_group_e4m3(a: np.ndarray, group: int = ACT_GROUP):
    """Per-token-group activation quantisation (SGLang page, section "prefll 侧的一个必要步
    骤：per-token-group 量化": fp8 activations with one scale per 128 consecutive values of a
    token).  The pages fix the group, not the scale rule; the reading is absmax scaling, in
    fp32 as the activations are stored:
        s = amax(|x| over the group) / 448   (1 for an all-zero group)
        q = e4m3_rne(clamp(x / s, -448, 448))
    so that the group's largest value maps onto the largest e4m3 code.  `a` is fp32 (or bf16
    bits) [R, K] with K a multiple of the group; returns codes uint8 [R, K] and scales fp32
    [R, K / group]."""
    x = as_f32(a)
    R, K = x.shape
    g = x.reshape(R, K // group, group)
    amax = np.max(np.abs(g), axis=2)
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = np.clip(g / s[:, :, None], np.float32(-E4M3_MAX), np.float32(E4M3_MAX)).astype(np.float32)
    return e4m3_encode(y).reshape(R, K), s


def dequant_group(q: np.ndarray, s: np.ndarray, group: int = ACT_GROUP) -> np.ndarray:
    """value = e4m3(q) * s[r, c // group], exact in float64."""
    return e4m3_decode(q) * np.repeat(s.astype(np.float64), group, axis=1)


def expert_weights_f64(inp, slot: int):
    """(Wg [I,H], Wu [I,H], Wd [H,I]) of one local slot in float64."""
    if inp.w13 is not None:
        return (as_f32(inp.w13[slot, 0]).astype(np.float64),
                as_f32(inp.w13[slot, 1]).astype(np.float64),
                as_f32(inp.w2[slot]).astype(np.float64))
    return (dequant_block(inp.w13_q[slot, 0], inp.w13_s[slot, 0]),
            dequant_block(inp.w13_q[slot, 1], inp.w13_s[slot, 1]),
            dequant_block(inp.w2_q[slot], inp.w2_s[slot]))


def swiglu(x: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """y = (silu(x Wg^T) * (x Wu^T)) Wd^T in float64, silu(z) = z / (1 + e^-z).
    gate_proj/up_proj are [I, H] and down_proj [H, I] (SGLang page, section "EP 下专家
    权重切不均匀的问题"); MM1, activation, MM2 in that order (vLLM page, modular-kernel
    block figure caption)."""
    gt = x @ wg.T
    u = x @ wu.T
    h = gt / (1.0 + np.exp(-gt)) * u
    return h @ wd.T


def swiglu_e4m3_act(x: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """The expert with fp8 activations, as the pages' DeepGEMM path feeds it: the input rows
    are quantised per 1x128 group (quant_group_e4m3) before the gate/up product, and the
    intermediate h, stored as bf16, is quantised the same way before the down product.  The
    products of the exactly dequantised operands are float64."""
    xd = dequant_group(*quant_group_e4m3(x))
    gt = xd @ wg.T
    u = xd @ wu.T
    h = bf16_rne(gt / (1.0 + np.exp(-gt)) * u)
    return dequant_group(*quant_group_e4m3(h)) @ wd.T


def expert_ffn(x_perm: np.ndarray, plan: dict, inp, fp8_act: str = "bf16") -> np.ndarray:
    """y_perm rows of every segment; alignment pad rows stay 0.  float64.  fp8_act = "e4m3"
    quantises the activations per 1x128 group before each product (swiglu_e4m3_act)."""
    ffn = swiglu_e4m3_act if fp8_act == "e4m3" else swiglu
    rows = len(plan["sorted_pair"])
    H = inp.cfg.hidden
    y = np.zeros((rows, H), dtype=np.float64)
    seg, counts = plan["seg_offsets"], plan["counts"]
    xf = as_f32(x_perm).astype(np.float64)
    for e in range(len(counts)):
        a = int(seg[e])
        b = min(int(seg[e]) + int(counts[e]), rows)
        if b <= a:
            continue
        wg, wu, wd = expert_weights_f64(inp, e)
        y[a:b] = ffn(xf[a:b], wg, wu, wd)
    return y


# ============================================================================ O5 combine

def combine(y_perm: np.ndarray, plan: dict, weights: np.ndarray, G: int,
            routed_scale: float = 1.0) -> np.ndarray:
    """out[g] = scale * sum_{j ascending, pair_row >= 0} w[g,j] * y[pair_row[g*k+j]] (float64);
    rows with no local pair are 0.  The finalize step applies the top-k weights after the
    un-permute (vLLM page, modular-kernel figure caption), and the combine call itself is
    given no weights (vLLM page, section "第 3 段：combine 前再交一次棒")."""
    k = plan["k"]
    yf = as_f32(y_perm).astype(np.float64) if y_perm.dtype != np.float64 else y_perm
    H = yf.shape[1] if yf.ndim == 2 else 0
    out = np.zeros((G, H), dtype=np.float64)
    pr = plan["pair_row"].reshape(G, k)
    w = weights.astype(np.float64)
    for j in range(k):
        m = pr[:, j] >= 0
        out[m] += w[m, j:j + 1] * yf[pr[m, j]]
    return out * routed_scale


# ============================================================================ per-token form

def token_output(inp, g: int, x_row: np.ndarray, ids_row: np.ndarray, w_row: np.ndarray,
                 weights_cache: Optional[dict] = None) -> np.ndarray:
    """Output of one global row computed directly:  scale * sum_j w_j * FFN_{slot(g,j)}(x_g)
    over the pairs that land on a local slot.  Equal to dispatch -> experts -> combine for
    that row; used to sample full-size outputs one row at a time."""
    cfg = inp.cfg
    x = as_f32(x_row).astype(np.float64)[None, :]
    out = np.zeros(cfg.hidden, dtype=np.float64)
    for j in range(len(ids_row)):
        l = int(ids_row[j])
        if l < 0:
            continue
        p = int(inp.phys_of[l, g % int(inp.n_rep[l])])
        e = p - cfg.first_local
        if not (0 <= e < cfg.num_local):
            continue
        if weights_cache is not None and e in weights_cache:
            wts = weights_cache[e]
        else:
            wts = expert_weights_f64(inp, e)
            if weights_cache is not None:
                weights_cache[e] = wts
        out += float(w_row[j]) * swiglu(x, *wts)[0]
    return out * cfg.routed_scale


# ============================================================================ whole layer

def run_layer(inp, mode: str = "sum", align: int = 1, cap: Optional[int] = None,
              seg_stride: int = 0, fp8_act: str = "bf16") -> dict:
    """All six steps on the inputs of one workload; returns every intermediate.  seg_stride > 0
    dispatches into the fixed-capacity layout (dispatch_masked) instead of packed segments;
    fp8_act = "e4m3" runs the experts on per-group quantised activations."""
    cfg = inp.cfg
    dt = np.float32 if cfg.dtype == "f32" else np.uint16
    layout = gather_layout(cfg.num_tokens, mode, static_bound=cfg.static_bound)
    G = layout[1]
    gx, valid = gather(layout, inp.replicas, cfg.hidden, dt)
    logits, ids, w = route(cfg, gx, valid, inp.router_w, inp.bias)
    if seg_stride > 0:
        plan = dispatch_masked(ids, inp.phys_of, inp.n_rep, cfg.first_local, cfg.num_local, seg_stride)
    else:
        plan = dispatch(ids, inp.phys_of, inp.n_rep, cfg.first_local, cfg.num_local, align, cap)
    xp = permute_rows(gx, plan)
    y = expert_ffn(xp, plan, inp, fp8_act)
    out = combine(y, plan, w, G, cfg.routed_scale)
    return dict(layout=layout, global_x=gx, row_valid=valid, logits=logits, ids=ids, weights=w,
                plan=plan, x_perm=xp, y_perm=y, out=out, replicas_out=scatter(layout, out))


# ============================================================================ O7 EPLB statistics

def physical_counts(ids: np.ndarray, phys_of: np.ndarray, n_rep: np.ndarray, num_physical: int) -> np.ndarray:
    """Tokens per physical expert slot in one step: every valid (row g, pick j) goes to the
    rank-invariant replica phys_of[id, g mod n_rep[id]] (SGLang page, section "推理时怎么“选副本”":
    without an all-to-all back end every rank must pick the same replica).  Ids outside
    [0, E) (pad rows) and slots outside [0, num_physical) count nowhere.  int64[num_physical]."""
    G, k = ids.shape
    E = phys_of.shape[0]
    out = np.zeros(num_physical, dtype=np.int64)
    g = np.repeat(np.arange(G, dtype=np.int64), k)
    e = ids.reshape(-1).astype(np.int64)
    ok = (e >= 0) & (e < E)
    g, e = g[ok], e[ok]
    p = phys_of[e, g % n_rep[e]].astype(np.int64)
    p = p[(p >= 0) & (p < num_physical)]
    np.add.at(out, p, 1)
    return out


def physical_to_logical_count(phys_count: np.ndarray, phy2log: np.ndarray, num_logical: int) -> np.ndarray:
    """Each physical slot's count added to the logical expert it holds (section "统计:把物理计数
    还原成逻辑计数": the scatter-add that turns per-slot counts into per-expert load).
    phys_count and phy2log are [L, P]; returns int64 [L, E]."""
    L, P = phys_count.shape
    out = np.zeros((L, num_logical), dtype=np.int64)
    for l in range(L):
        for p in range(P):
            out[l, phy2log[l, p]] += phys_count[l, p]
    return out


def gpu_counts(phys_count: np.ndarray, num_gpus: int) -> np.ndarray:
    """[..., P] per-slot counts -> [..., num_gpus] per-GPU sums; GPU r holds the contiguous
    slots [r P/M, (r+1) P/M) (section "三步算法", step 3: phy2pphy = pack * slots-per-GPU + rank)."""
    P = phys_count.shape[-1]
    assert P % num_gpus == 0
    return phys_count.reshape(*phys_count.shape[:-1], num_gpus, P // num_gpus).sum(axis=-1)


def utilization_rate(gpu_count: np.ndarray) -> np.ndarray:
    """Balancedness over the last axis (section "不均衡的代价与冗余专家的思路"):
    (mean + 1e-5) / (max + 1e-5) of the per-GPU token counts; 1 is perfect balance."""
    c = np.asarray(gpu_count, dtype=np.float64)
    return (c.mean(axis=-1) + 1e-5) / (c.max(axis=-1) + 1e-5)


def balanced_packing(weight: Sequence[float], num_packs: int):
    """Spread n items over num_packs packs of n / num_packs items each, balancing pack loads.

    The page describes it only in words (section "三步算法", step 1: balance the packs' total
    load).  Reading (greedy, heaviest first): items in descending weight, ties in ascending
    index; each goes to the lightest pack that still has room, ties to the lower pack index.
    Returns (pack of each item, its position inside the pack in assignment order)."""
    n = len(weight)
    assert n % num_packs == 0
    per = n // num_packs
    order = sorted(range(n), key=lambda i: (-weight[i], i))
    load = [0.0] * num_packs
    size = [0] * num_packs
    pack = [0] * n
    rank = [0] * n
    for i in order:
        best = -1
        for q in range(num_packs):
            if size[q] < per and (best < 0 or load[q] < load[best]):
                best = q
        pack[i] = best
        rank[i] = size[best]
        load[best] += weight[i]
        size[best] += 1
    return pack, rank


def replicate_experts(weight: Sequence[float], num_phy: int):
    """Give num_phy slots to n logical experts, heavy experts several (section "三步算法", step 2:
    loaded experts get more slots, light ones one).  Reading (greedy): every expert first gets
    one slot in index order; each further slot goes to the expert with the largest load per
    replica weight / count, ties to the lower index.  This greedy minimises the largest
    per-replica load.  Returns (logical expert of each slot, replica rank of the slot,
    replica count of each expert)."""
    n = len(weight)
    assert num_phy >= n
    phy2log = list(range(n))
    rank = [0] * n
    cnt = [1] * n
    for _ in range(n, num_phy):
        best = 0
        for e in range(1, n):
            if weight[e] / cnt[e] > weight[best] / cnt[best]:
                best = e
        phy2log.append(best)
        rank.append(cnt[best])
        cnt[best] += 1
    return phy2log, rank, cnt


def rebalance_hierarchical(weight: np.ndarray, num_physical: int, num_groups: int, num_nodes: int,
                           num_gpus: int):
    """Expert placement from per-layer logical loads (section "三步算法:分组、复制、再打包").

    1. Whole expert groups are packed onto nodes by group load (balanced_packing).
    2. Inside each node, its logical experts get the node's P / nodes slots
       (replicate_experts); replicas never leave their node.
    3. Inside each node, the slots are packed onto the node's GPUs by per-replica load (the
       expert's load divided by its replica count), P / gpus slots per GPU; a slot's global
       index is node * (P / nodes) + gpu-in-node * (P / gpus) + position on the GPU.

    Sums run in ascending index order.  weight: [L, E] float64.  Returns (phy2log [L, P],
    phy_rank [L, P], log_count [L, E]) as int32."""
    weight = np.asarray(weight, dtype=np.float64)
    L, E = weight.shape
    P = num_physical
    if E % num_groups or num_groups % num_nodes or num_gpus % num_nodes or P % num_gpus:
        raise ValueError("shapes do not divide")
    group_size = E // num_groups
    groups_per_node = num_groups // num_nodes
    e_node, p_node = E // num_nodes, P // num_nodes
    gpus_per_node, per_gpu = num_gpus // num_nodes, P // num_gpus
    if p_node < e_node:
        raise ValueError("fewer slots than experts on a node")
    phy2log = np.empty((L, P), dtype=np.int32)
    phy_rank = np.empty((L, P), dtype=np.int32)
    log_count = np.empty((L, E), dtype=np.int32)
    for l in range(L):
        w = [float(v) for v in weight[l]]
        group_load = []
        for q in range(num_groups):
            acc = 0.0
            for e in range(q * group_size, (q + 1) * group_size):
                acc += w[e]
            group_load.append(acc)
        gnode, gpos = balanced_packing(group_load, num_nodes)
        # logical experts of node n in node order: its groups by position, each group's
        # experts in ascending id
        node_experts = [[0] * e_node for _ in range(num_nodes)]
        for q in range(num_groups):
            for t in range(group_size):
                node_experts[gnode[q]][gpos[q] * group_size + t] = q * group_size + t
        for nd in range(num_nodes):
            ex = node_experts[nd]
            wl = [w[e] for e in ex]
            s2m, srank, mcnt = replicate_experts(wl, p_node)
            share = [wl[s2m[i]] / mcnt[s2m[i]] for i in range(p_node)]
            gpu, pos = balanced_packing(share, gpus_per_node)
            for i in range(p_node):
                slot = nd * p_node + gpu[i] * per_gpu + pos[i]
                phy2log[l, slot] = ex[s2m[i]]
                phy_rank[l, slot] = srank[i]
            for m_ in range(e_node):
                log_count[l, ex[m_]] = mcnt[m_]
    return phy2log, phy_rank, log_count


def logical_to_physical(phy2log: np.ndarray, phy_rank: np.ndarray, num_logical: int, max_rep: int):
    """Dispatch table of one layer from a placement: phys_of[e, r] = the slot holding replica r
    of expert e (-1 past its count), n_rep[e] = its replica count (ExpertLocationMetadata's
    logical_to_all_physical_map and its num_valid, section "逻辑与物理的两套映射")."""
    P = phy2log.shape[0]
    phys_of = np.full((num_logical, max_rep), -1, dtype=np.int32)
    n_rep = np.zeros(num_logical, dtype=np.int32)
    for p in range(P):
        e, r = int(phy2log[p]), int(phy_rank[p])
        if r >= max_rep:
            raise ValueError("more replicas than max_rep")
        phys_of[e, r] = p
        n_rep[e] += 1
    return phys_of, n_rep


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max|got - ref| / max|ref| (infinity-norm relative error)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    den = float(np.max(np.abs(ref)))
    num = float(np.max(np.abs(got - ref)))
    return num / den if den > 0 else num


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """Largest per-row error: max over rows r of max|got_r - ref_r| / max|ref_r|.  A row whose
    reference is all zero contributes max|got_r|.  Unlike rel_err, one row with a small
    magnitude cannot hide behind the largest value of the whole tensor."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    got = got.reshape(ref.shape[0], -1)
    ref = ref.reshape(ref.shape[0], -1)
    num = np.max(np.abs(got - ref), axis=1)
    den = np.max(np.abs(ref), axis=1)
    per_row = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    return float(per_row.max())


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |v| (float64): 2^(e - 7) for |v| in [2^e, 2^(e+1)) with
    e >= -126, and the subnormal spacing 2^-133 below 2^-126 (and at 0)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    _, ex = np.frexp(a)                   # a = m * 2^ex, m in [0.5, 1): floor(log2 a) = ex - 1
    e = np.where(a > 0, np.maximum(ex - 1, -126), -126)
    return np.ldexp(1.0, e - 7)

