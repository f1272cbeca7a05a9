"""Python binding of libmoe_hip.so: one rank's MoE layer under DP attention + expert
parallelism on an MI355X (gfx950).

Each function carries the name of the C entry point it calls (include/moe.h) and only
marshals arguments: device tensors become pointers, the stream is torch's current stream.
Every step runs in the HIP kernels of ``csrc/``; if the library is missing the calls raise.
"""
from __future__ import annotations

import ctypes
from typing import List, Optional, Sequence

import numpy as np
import torch

from . import _lib
from ._lib import (MOE_BF16, MOE_F32, MOE_FP8_E4M3, MOE_PAD_AUTO, MOE_PAD_MAX_LEN, MOE_PAD_SUM_LEN,
                   MOE_ROUTE_GROUPED_SIGMOID, MOE_ROUTE_SOFTMAX, ExpertMap, ExpertWeights,
                   GatherLayout, MoEError, Plan, RouteCfg, check)

__all__ = [
    "moe_gather_layout", "moe_gather", "moe_entry_gather", "moe_scatter", "moe_expert_load",
    "moe_physical_to_logical_count", "moe_eplb_balancedness", "moe_eplb_rebalance",
    "moe_eplb_logical_to_physical", "moe_route", "moe_route_from_logits",
    "moe_dispatch", "moe_dispatch_noalloc", "moe_dispatch_workspace_size", "moe_quant_act_fp8", "moe_expert_gemm_fast_path", "moe_expert_gemm", "moe_expert_gemm_up", "moe_expert_gemm_up_gather",
    "moe_expert_gemm_down", "moe_expert_gemm_workspace_size", "moe_combine", "moe_version",
    "PlanBuffers", "make_route_cfg", "make_expert_map", "make_expert_weights", "MoEError",
    "GatherLayout", "RouteCfg", "ExpertMap", "ExpertWeights", "Plan",
    "moe_stream_create_cu_masked", "moe_stream_destroy",
]

_MODES = {"auto": MOE_PAD_AUTO, "max": MOE_PAD_MAX_LEN, "sum": MOE_PAD_SUM_LEN}
_MODE_NAMES = {MOE_PAD_MAX_LEN: "max", MOE_PAD_SUM_LEN: "sum"}


def lib():
    return _lib.load()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.uint8:
        return MOE_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the HIP library must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def moe_version() -> str:
    return lib().moe_version().decode()


# ------------------------------------------------------------------ gather / scatter

def moe_gather_layout(num_tokens: Sequence[int], mode: str = "auto", is_extend: bool = False,
                      max_len_with_idle: bool = False, static_bound: int = 0) -> GatherLayout:
    n = (ctypes.c_int32 * len(num_tokens))(*[int(v) for v in num_tokens])
    out = GatherLayout()
    check("moe_gather_layout", lib().moe_gather_layout(
        ctypes.cast(n, ctypes.c_void_p), len(num_tokens), _MODES[mode], int(is_extend),
        int(max_len_with_idle), int(static_bound), ctypes.byref(out)))
    return out


def layout_mode(L: GatherLayout) -> str:
    return _MODE_NAMES[L.mode]


def layout_offsets(L: GatherLayout) -> List[int]:
    return [int(L.offsets[i]) for i in range(L.num_replicas + 1)]


def layout_sizes(L: GatherLayout) -> List[int]:
    return [int(L.sizes[i]) for i in range(L.num_replicas)]


def _ptr_array(ts: Sequence[Optional[torch.Tensor]]):
    arr = (ctypes.c_void_p * len(ts))(*[(_ptr(t) if (t is not None and t.numel() > 0) else None)
                                         for t in ts])
    return arr


def moe_gather(L: GatherLayout, replicas: Sequence[torch.Tensor], global_x: torch.Tensor,
               row_valid: torch.Tensor, stream=None) -> None:
    H = global_x.shape[1]
    arr = _ptr_array(replicas)
    check("moe_gather", lib().moe_gather(ctypes.byref(L), ctypes.cast(arr, ctypes.c_void_p), H,
                                         _dtype_code(global_x), _ptr(global_x), _ptr(row_valid),
                                         _stream(stream)))


def moe_entry_gather(L: GatherLayout, hidden: Sequence[torch.Tensor], residual: Sequence[torch.Tensor],
                     norm_weight: torch.Tensor, eps: float, global_x: torch.Tensor,
                     row_valid: torch.Tensor, stream=None) -> None:
    """Residual add + RMSNorm + DP gather in one pass; ``residual`` tensors are updated in place."""
    H = global_x.shape[1]
    ha, ra = _ptr_array(hidden), _ptr_array(residual)
    check("moe_entry_gather", lib().moe_entry_gather(
        ctypes.byref(L), ctypes.cast(ha, ctypes.c_void_p), ctypes.cast(ra, ctypes.c_void_p),
        _ptr(norm_weight), float(eps), H, _dtype_code(global_x), _ptr(global_x), _ptr(row_valid),
        _stream(stream)))


def moe_scatter(L: GatherLayout, out: torch.Tensor, replicas_out: Sequence[torch.Tensor],
                stream=None) -> None:
    H = out.shape[1]
    arr = _ptr_array(replicas_out)
    check("moe_scatter", lib().moe_scatter(ctypes.byref(L), _ptr(out), H, _dtype_code(out),
                                           ctypes.cast(arr, ctypes.c_void_p), _stream(stream)))


# ------------------------------------------------------------------ routing

def make_route_cfg(kind: str, num_experts: int, top_k: int, n_group: int = 1, topk_group: int = 1,
                   group_topn: int = 2, renormalize: bool = False, gate: str = "exact") -> RouteCfg:
    k = MOE_ROUTE_SOFTMAX if kind == "softmax" else MOE_ROUTE_GROUPED_SIGMOID
    mode = {"exact": _lib.MOE_GATE_EXACT, "fast": _lib.MOE_GATE_FAST}[gate]
    return RouteCfg(k, num_experts, top_k, n_group, topk_group, group_topn, int(renormalize), mode)


def moe_route(global_x: torch.Tensor, row_valid: torch.Tensor, w_router: torch.Tensor,
              bias: Optional[torch.Tensor], cfg: RouteCfg, logits: torch.Tensor,
              topk_ids: torch.Tensor, topk_w: torch.Tensor, stream=None) -> None:
    G, H = global_x.shape
    check("moe_route", lib().moe_route(_ptr(global_x), _ptr(row_valid), G, H, _dtype_code(global_x),
                                       _ptr(w_router), _ptr(bias), ctypes.byref(cfg), _ptr(logits),
                                       _ptr(topk_ids), _ptr(topk_w), _stream(stream)))


def moe_route_from_logits(logits: torch.Tensor, row_valid: Optional[torch.Tensor],
                          bias: Optional[torch.Tensor], cfg: RouteCfg, topk_ids: torch.Tensor,
                          topk_w: torch.Tensor, stream=None) -> None:
    check("moe_route_from_logits", lib().moe_route_from_logits(
        _ptr(logits), _ptr(row_valid), logits.shape[0], _ptr(bias), ctypes.byref(cfg),
        _ptr(topk_ids), _ptr(topk_w), _stream(stream)))


# ------------------------------------------------------------------ dispatch

def make_expert_map(num_logical: int, first_slot: int, num_slots: int,
                    phys_of: Optional[torch.Tensor] = None, n_rep: Optional[torch.Tensor] = None):
    """Keeps the device tables referenced on the returned struct."""
    m = ExpertMap(num_logical, phys_of.shape[1] if phys_of is not None else 1, _ptr(phys_of),
                  _ptr(n_rep), first_slot, num_slots)
    m._keep = (phys_of, n_rep)
    return m


# ------------------------------------------------------------------ expert-load statistics (EPLB)

def moe_expert_load(topk_ids: torch.Tensor, emap, num_physical: int, phys_count: torch.Tensor,
                    stream=None) -> None:
    """Adds this step's token count of every physical slot to ``phys_count`` (int64 [P])."""
    G, k = topk_ids.shape
    check("moe_expert_load", lib().moe_expert_load(_ptr(topk_ids), G, k, ctypes.byref(emap), num_physical,
                                                   _ptr(phys_count), _stream(stream)))


def moe_physical_to_logical_count(phys_count: torch.Tensor, phy2log: torch.Tensor,
                                  logical_count: torch.Tensor, stream=None) -> None:
    """logical_count[l, e] = sum of phys_count[l, p] over the slots holding e (device, int64)."""
    L, P = phys_count.shape
    check("moe_physical_to_logical_count",
          lib().moe_physical_to_logical_count(_ptr(phys_count), _ptr(phy2log), L, P, logical_count.shape[1],
                                              _ptr(logical_count), _stream(stream)))


def _host(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def moe_eplb_balancedness(phys_count, num_gpus: int) -> np.ndarray:
    """Host: per-layer (mean + 1e-5) / (max + 1e-5) of per-GPU counts from int64 [L, P]."""
    pc, pp = _host(np.atleast_2d(phys_count), np.int64)
    out = np.empty(pc.shape[0], dtype=np.float64)
    check("moe_eplb_balancedness", lib().moe_eplb_balancedness(pp, pc.shape[0], pc.shape[1], num_gpus,
                                                               out.ctypes.data_as(ctypes.c_void_p)))
    return out


def moe_eplb_rebalance(weight, num_physical: int, num_groups: int, num_nodes: int, num_gpus: int):
    """Host: hierarchical expert placement from loads [L, E] -> (phy2log, phy_rank, log_count)."""
    w, wp = _host(np.atleast_2d(weight), np.float64)
    L, E = w.shape
    phy2log = np.empty((L, num_physical), dtype=np.int32)
    rank = np.empty((L, num_physical), dtype=np.int32)
    cnt = np.empty((L, E), dtype=np.int32)
    check("moe_eplb_rebalance", lib().moe_eplb_rebalance(
        wp, L, E, num_physical, num_groups, num_nodes, num_gpus, phy2log.ctypes.data_as(ctypes.c_void_p),
        rank.ctypes.data_as(ctypes.c_void_p), cnt.ctypes.data_as(ctypes.c_void_p)))
    return phy2log, rank, cnt


def moe_eplb_logical_to_physical(phy2log, phy_rank, num_logical: int, max_rep: int):
    """Host: one layer's dispatch table (phys_of int32 [E, max_rep], n_rep int32 [E])."""
    a, ap = _host(phy2log, np.int32)
    r, rp = _host(phy_rank, np.int32)
    phys_of = np.empty((num_logical, max_rep), dtype=np.int32)
    n_rep = np.empty(num_logical, dtype=np.int32)
    check("moe_eplb_logical_to_physical", lib().moe_eplb_logical_to_physical(
        ap, rp, a.shape[0], num_logical, max_rep, phys_of.ctypes.data_as(ctypes.c_void_p),
        n_rep.ctypes.data_as(ctypes.c_void_p)))
    return phys_of, n_rep


class PlanBuffers:
    """Device buffers of one dispatch plan (torch-allocated) and the C struct over them."""

    def __init__(self, G: int, k: int, num_slots: int, align: int = 1, cap: Optional[int] = None,
                 device="cuda", seg_stride: int = 0):
        """seg_stride > 0 selects the fixed-capacity layout (slot e at rows e * seg_stride)."""
        if cap is None:
            cap = num_slots * seg_stride if seg_stride > 0 else G * min(k, num_slots) + num_slots * (align - 1)
        i32, i64 = torch.int32, torch.int64
        self.counts = torch.zeros(num_slots, dtype=i32, device=device)
        self.seg_offsets = torch.zeros(num_slots + 1, dtype=i64, device=device)
        self.sorted_pair = torch.zeros(max(cap, 1), dtype=i32, device=device)
        self.pair_row = torch.zeros(max(G * k, 1), dtype=i32, device=device)
        self.num_rows = torch.zeros(1, dtype=i64, device=device)
        self.error_flag = torch.zeros(1, dtype=i32, device=device)
        self.cap, self.G, self.k, self.num_slots, self.align = cap, G, k, num_slots, align
        self.seg_stride = seg_stride
        self.struct = Plan(_ptr(self.counts), _ptr(self.seg_offsets), _ptr(self.sorted_pair),
                           _ptr(self.pair_row), _ptr(self.num_rows), _ptr(self.error_flag),
                           cap, G, k, num_slots, align, seg_stride)


def moe_dispatch_workspace_size(G: int, k: int, num_slots: int) -> int:
    return int(lib().moe_dispatch_workspace_size(G, k, num_slots))


def moe_dispatch(global_x: torch.Tensor, topk_ids: torch.Tensor, emap: ExpertMap,
                 plan: PlanBuffers, x_perm: Optional[torch.Tensor], workspace: torch.Tensor,
                 stream=None) -> None:
    """x_perm=None: the plan only (no permuted copy), for moe_expert_gemm_up_gather."""
    G, H = global_x.shape
    k = plan.k
    check("moe_dispatch", lib().moe_dispatch(
        _ptr(global_x), _ptr(topk_ids), G, k, H, _dtype_code(global_x), ctypes.byref(emap),
        ctypes.byref(plan.struct), _ptr(x_perm), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_dispatch_noalloc(global_x: torch.Tensor, topk_ids: torch.Tensor, emap: ExpertMap,
                         plan: PlanBuffers, x_perm: Optional[torch.Tensor], stream=None) -> None:
    """moe_dispatch with the library's fixed per-GPU scratch instead of a workspace
    (x_perm=None: the plan only)."""
    G, H = global_x.shape
    check("moe_dispatch_noalloc", lib().moe_dispatch_noalloc(
        _ptr(global_x), _ptr(topk_ids), G, plan.k, H, _dtype_code(global_x), ctypes.byref(emap),
        ctypes.byref(plan.struct), _ptr(x_perm), _stream(stream)))


# ------------------------------------------------------------------ experts

def moe_expert_gemm_fast_path(x_perm: torch.Tensor, w: ExpertWeights, H: int, I: int, h: torch.Tensor,
                              y_perm: torch.Tensor) -> bool:
    """True when both GEMM halves run the bf16 tile kernels on these buffers."""
    return bool(lib().moe_expert_gemm_fast_path(_ptr(x_perm), _dtype_code(x_perm), ctypes.byref(w), H, I,
                                                 _ptr(h), _ptr(y_perm)))


def moe_quant_act_fp8(act: torch.Tensor, num_rows: torch.Tensor, q: torch.Tensor, s_t: torch.Tensor,
                      stream=None) -> None:
    """Per-1x128-group e4m3 codes q [cap, K] (uint8) and transposed scales s_t [K/128, cap]
    (fp32) of the first num_rows rows of act (bf16 [cap, K])."""
    cap, K = act.shape
    check("moe_quant_act_fp8", lib().moe_quant_act_fp8(_ptr(act), _ptr(num_rows), cap, K, _ptr(q),
                                                       _ptr(s_t), _stream(stream)))

def make_expert_weights(w13: torch.Tensor, w2: torch.Tensor, s13: Optional[torch.Tensor] = None,
                        s2: Optional[torch.Tensor] = None, fp8_act: str = "bf16") -> ExpertWeights:
    """fp8_act (e4m3 weights only): "bf16" keeps activations bf16 and dequantises weight
    fragments in the kernel; "e4m3" quantises activations per 1x128 group for fp8 MFMA."""
    mode = {"bf16": _lib.MOE_FP8_ACT_BF16, "e4m3": _lib.MOE_FP8_ACT_E4M3}[fp8_act]
    w = ExpertWeights(_dtype_code(w13), mode, _ptr(w13), _ptr(w2), _ptr(s13), _ptr(s2))
    w._keep = (w13, w2, s13, s2)
    return w


def moe_expert_gemm_workspace_size(cap: int, H: int, I: int, act_dtype: torch.dtype,
                                   w_dtype: torch.dtype) -> int:
    a = MOE_BF16 if act_dtype == torch.bfloat16 else MOE_F32
    w = {torch.bfloat16: MOE_BF16, torch.float32: MOE_F32, torch.uint8: MOE_FP8_E4M3}[w_dtype]
    return int(lib().moe_expert_gemm_workspace_size(cap, H, I, a, w))


def moe_expert_gemm(x_perm: torch.Tensor, plan: PlanBuffers, w: ExpertWeights, H: int, I: int,
                    y_perm: torch.Tensor, workspace: torch.Tensor, stream=None) -> None:
    check("moe_expert_gemm", lib().moe_expert_gemm(
        _ptr(x_perm), _dtype_code(x_perm), ctypes.byref(plan.struct), ctypes.byref(w), H, I,
        _ptr(y_perm), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def moe_expert_gemm_up(x_perm: torch.Tensor, plan: PlanBuffers, w: ExpertWeights, H: int, I: int,
                       h: torch.Tensor, workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check("moe_expert_gemm_up", lib().moe_expert_gemm_up(
        _ptr(x_perm), _dtype_code(x_perm), ctypes.byref(plan.struct), ctypes.byref(w), H, I,
        _ptr(h), _ptr(workspace), ws, _stream(stream)))


def moe_expert_gemm_up_gather(global_x: torch.Tensor, plan: PlanBuffers, w: ExpertWeights, H: int,
                              I: int, h: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                              stream=None) -> None:
    """The up GEMM reading each permuted row from global_x through the plan's sorted_pair
    (after moe_dispatch with x_perm=None): the same h as moe_expert_gemm_up on the copy."""
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check("moe_expert_gemm_up_gather", lib().moe_expert_gemm_up_gather(
        _ptr(global_x), _dtype_code(global_x), ctypes.byref(plan.struct), ctypes.byref(w), H, I,
        _ptr(h), _ptr(workspace), ws, _stream(stream)))


def moe_expert_gemm_down(h: torch.Tensor, plan: PlanBuffers, w: ExpertWeights, H: int, I: int,
                         y_perm: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                         stream=None) -> None:
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check("moe_expert_gemm_down", lib().moe_expert_gemm_down(
        _ptr(h), _dtype_code(h), ctypes.byref(plan.struct), ctypes.byref(w), H, I, _ptr(y_perm),
        _ptr(workspace), ws, _stream(stream)))


# ------------------------------------------------------------------ combine

def moe_combine(y_perm: torch.Tensor, plan: PlanBuffers, topk_w: torch.Tensor, routed_scale: float,
                out: torch.Tensor, stream=None) -> None:
    H = out.shape[1]
    check("moe_combine", lib().moe_combine(_ptr(y_perm), _dtype_code(out), ctypes.byref(plan.struct),
                                           _ptr(topk_w), float(routed_scale), H, _ptr(out),
                                           _stream(stream)))


def moe_combine_scatter(y_perm: torch.Tensor, plan: PlanBuffers, topk_w: torch.Tensor,
                        routed_scale: float, L: GatherLayout, replicas_out: Sequence[torch.Tensor],
                        stream=None) -> None:
    """The fused exit: combine written straight into the replicas' buffers (combine + scatter)."""
    H = y_perm.shape[1]
    arr = _ptr_array(replicas_out)
    check("moe_combine_scatter", lib().moe_combine_scatter(
        _ptr(y_perm), _dtype_code(y_perm), ctypes.byref(plan.struct), _ptr(topk_w),
        float(routed_scale), H, ctypes.byref(L), ctypes.cast(arr, ctypes.c_void_p), _stream(stream)))


# ------------------------------------------------------------------ CU-partitioned streams

def moe_stream_create_cu_masked(cu_mask) -> int:
    """A new stream (default priority) confined to the CUs whose bits are set in cu_mask, a
    sequence of 32-bit words (bit i of word i // 32 = CU i); returns the raw stream handle,
    which torch.cuda.ExternalStream can wrap.  Release it with moe_stream_destroy."""
    words = [int(x) & 0xFFFFFFFF for x in cu_mask]
    arr = (ctypes.c_uint32 * max(len(words), 1))(*words)
    out = ctypes.c_void_p()
    check("moe_stream_create_cu_masked", lib().moe_stream_create_cu_masked(arr, len(words), ctypes.byref(out)))
    return int(out.value)


def moe_stream_destroy(handle: int) -> None:
    check("moe_stream_destroy", lib().moe_stream_destroy(ctypes.c_void_p(handle)))
