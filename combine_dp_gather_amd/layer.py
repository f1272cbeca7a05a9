"""One rank's MoE layer as the six C-ABI calls in order, with torch-allocated buffers.

gather -> route -> dispatch -> expert GEMMs -> combine -> scatter: the step order of the
SGLang walkthrough "SGLang 源码完全拆解(十七): DP Attention 与专家并行" (DP gather before the
MoE, section "两种 gather"; op_gate, op_select_experts, dispatch, experts, combine in the
operations list of section "operations 与 yield"; scatter back, section "scatter：把 MoE 的
输出还回本副本").  Python only allocates and passes pointers; every step runs in HIP.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np
import torch

from . import (PlanBuffers, layout_offsets, layout_sizes, make_expert_map, make_expert_weights,
               make_route_cfg, moe_combine, moe_dispatch, moe_dispatch_workspace_size,
               moe_expert_gemm, moe_expert_gemm_down, moe_expert_gemm_up, moe_expert_gemm_up_gather,
               moe_entry_gather, moe_expert_gemm_workspace_size, moe_gather, moe_gather_layout, moe_route,
               moe_scatter, moe_combine_scatter)


def _to_dev(a: Optional[np.ndarray], device, bf16: bool = False) -> Optional[torch.Tensor]:
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if bf16:
        assert a.dtype == np.uint16
        t = t.view(torch.bfloat16)
    return t.to(device)


@dataclass
class LayerSpec:
    hidden: int
    inter: int
    num_experts: int
    top_k: int
    route: str                  # "softmax" | "grouped"
    num_local: int
    first_local: int = 0
    n_group: int = 1
    topk_group: int = 1
    group_topn: int = 2
    renormalize: bool = False
    routed_scale: float = 1.0
    gate: str = "exact"         # "exact" (defined summation order) | "fast" (bf16 matrix cores)


class DeviceWeights:
    """Router and expert weights resident in HBM."""

    def __init__(self, inp, device="cuda", fp8_act: str = "bf16"):
        cfg = inp.cfg
        bf = cfg.dtype == "bf16"
        self.router = _to_dev(inp.router_w, device, bf)
        self.bias = _to_dev(inp.bias, device)
        if inp.w13 is not None:
            self.w13 = _to_dev(inp.w13, device, bf)
            self.w2 = _to_dev(inp.w2, device, bf)
            self.s13 = self.s2 = None
        else:
            self.w13 = _to_dev(inp.w13_q, device)
            self.w2 = _to_dev(inp.w2_q, device)
            self.s13 = _to_dev(inp.w13_s, device)
            self.s2 = _to_dev(inp.w2_s, device)
        trivial = cfg.slot_logical is None
        self.phys_of = None if trivial else _to_dev(inp.phys_of, device)
        self.n_rep = None if trivial else _to_dev(inp.n_rep, device)
        self.ew = make_expert_weights(self.w13, self.w2, self.s13, self.s2, fp8_act)


def spec_of(cfg) -> LayerSpec:
    return LayerSpec(hidden=cfg.hidden, inter=cfg.inter, num_experts=cfg.num_experts,
                     top_k=cfg.top_k, route=cfg.route, num_local=cfg.num_local,
                     first_local=cfg.first_local, n_group=cfg.n_group, topk_group=cfg.topk_group,
                     group_topn=cfg.group_topn, renormalize=cfg.renormalize,
                     routed_scale=cfg.routed_scale)


class MoELayer:
    """Buffers for one step shape (replica counts, gather mode) and the six calls.

    ``fuse_permute`` (default): dispatch builds the plan only and the up GEMM reads its rows
    from ``global_x`` through ``sorted_pair`` (moe_expert_gemm_up_gather), so no ``x_perm``
    copy is made or allocated; False runs the permuted copy and the plain up GEMM.  The
    results are the same bits."""

    def __init__(self, spec: LayerSpec, weights: DeviceWeights, num_tokens: Sequence[int],
                 act_dtype: torch.dtype, mode: str = "auto", static_bound: int = 0,
                 is_extend: bool = False, align: int = 1, cap: Optional[int] = None,
                 device="cuda", seg_stride: int = 0, fuse_permute: bool = True):
        self.spec, self.w, self.device, self.dt = spec, weights, device, act_dtype
        self.fuse_permute = fuse_permute
        self.layout = moe_gather_layout(num_tokens, mode, is_extend=is_extend,
                                        static_bound=static_bound)
        G = int(self.layout.rows)
        self.G = G
        H, I, k = spec.hidden, spec.inter, spec.top_k
        self.sizes = layout_sizes(self.layout)
        self.offsets = layout_offsets(self.layout)
        self.global_x = torch.empty((G, H), dtype=act_dtype, device=device)
        self.row_valid = torch.empty(max(G, 1), dtype=torch.int32, device=device)
        self.route_cfg = make_route_cfg(spec.route, spec.num_experts, k, spec.n_group,
                                        spec.topk_group, spec.group_topn, spec.renormalize, spec.gate)
        self.logits = torch.empty((max(G, 1), spec.num_experts), dtype=torch.float32, device=device)
        self.topk_ids = torch.empty((max(G, 1), k), dtype=torch.int32, device=device)
        self.topk_w = torch.empty((max(G, 1), k), dtype=torch.float32, device=device)
        self.emap = make_expert_map(spec.num_experts, spec.first_local, spec.num_local,
                                    weights.phys_of, weights.n_rep)
        # seg_stride > 0: fixed-capacity layout, every slot's rows at a fixed address
        self.plan = PlanBuffers(G, k, spec.num_local, align, cap, device, seg_stride)
        cap = self.plan.cap
        self.dispatch_ws = torch.empty(max(moe_dispatch_workspace_size(G, k, spec.num_local), 16),
                                       dtype=torch.uint8, device=device)
        self.x_perm = None if fuse_permute else torch.empty((max(cap, 1), H), dtype=act_dtype,
                                                            device=device)
        self.h = torch.empty((max(cap, 1), I), dtype=act_dtype, device=device)
        self.y_perm = torch.empty((max(cap, 1), H), dtype=act_dtype, device=device)
        self.gemm_ws = torch.empty(max(moe_expert_gemm_workspace_size(cap, H, I, act_dtype,
                                                                      weights.w13.dtype), 256),
                                   dtype=torch.uint8, device=device)
        self.out = torch.empty((G, H), dtype=act_dtype, device=device)
        self.replicas_out = [torch.empty((n, H), dtype=act_dtype, device=device) for n in self.sizes]

    # the six steps, individually callable
    def gather(self, replicas):
        moe_gather(self.layout, replicas, self.global_x, self.row_valid)

    def entry(self, hidden, residual, norm_weight, eps: float):
        """The fused entry step in place of the gather: residual add, RMSNorm, gather."""
        moe_entry_gather(self.layout, hidden, residual, norm_weight, eps, self.global_x, self.row_valid)

    def route(self):
        if self.G:
            moe_route(self.global_x, self.row_valid, self.w.router, self.w.bias, self.route_cfg,
                      self.logits, self.topk_ids, self.topk_w)

    def dispatch(self):
        if self.G:
            moe_dispatch(self.global_x, self.topk_ids[:self.G], self.emap, self.plan, self.x_perm,
                         self.dispatch_ws)

    def experts(self, split: bool = True):
        if not self.G:
            return
        s = self.spec
        if split or self.fuse_permute:
            self.experts_up()
            self.experts_down()
        else:
            moe_expert_gemm(self.x_perm, self.plan, self.w.ew, s.hidden, s.inter, self.y_perm,
                            self.gemm_ws)

    def experts_up(self):
        if not self.G:
            return
        if self.fuse_permute:
            moe_expert_gemm_up_gather(self.global_x, self.plan, self.w.ew, self.spec.hidden,
                                      self.spec.inter, self.h, self.gemm_ws)
        else:
            moe_expert_gemm_up(self.x_perm, self.plan, self.w.ew, self.spec.hidden, self.spec.inter,
                               self.h, self.gemm_ws)

    def experts_down(self):
        if self.G:
            moe_expert_gemm_down(self.h, self.plan, self.w.ew, self.spec.hidden, self.spec.inter,
                                 self.y_perm, self.gemm_ws)

    def combine(self):
        if self.G:
            moe_combine(self.y_perm, self.plan, self.topk_w, self.spec.routed_scale, self.out)

    def scatter(self, replicas_out=None):
        moe_scatter(self.layout, self.out, self.replicas_out if replicas_out is None else replicas_out)

    def combine_scatter(self, replicas_out=None):
        """The fused exit in place of combine + scatter (same bits; ``out`` is not written)."""
        dst = self.replicas_out if replicas_out is None else replicas_out
        if self.G:
            moe_combine_scatter(self.y_perm, self.plan, self.topk_w, self.spec.routed_scale,
                                self.layout, dst)

    def forward(self, replicas, entry=None, fused_exit: bool = False) -> List[torch.Tensor]:
        """One step.  ``entry = (residual, norm_weight, eps)`` runs the fused entry step on
        ``replicas`` (the attention outputs) instead of the plain gather; ``fused_exit`` runs
        the fused combine + scatter."""
        if entry is None:
            self.gather(replicas)
        else:
            self.entry(replicas, *entry)
        self.route()
        self.dispatch()
        self.experts()
        if fused_exit:
            self.combine_scatter()
        else:
            self.combine()
            self.scatter()
        return self.replicas_out


def split_micro_batches(num_tokens: Sequence[int]) -> List[List[tuple]]:
    """Two micro-batches of one step: each replica's tokens cut at half their count.

    The two-batch-overlap split of the SGLang page (section "Two-batch Overlap:把通信藏进另一个
    micro-batch 的计算里", compute_split_seq_index): decode batches split at half the token
    count (one token per sequence), and a prefill batch whose boundary split is unbalanced
    falls back to cutting a sequence at half the tokens.  The replicas here carry no sequence
    structure, so every replica is cut at n // 2: micro-batch 0 takes rows [0, n // 2) of
    each replica, micro-batch 1 the rest (the vLLM page's UBatchSlice token slices).
    Returns [[(start, stop) per replica] for each micro-batch]."""
    return [[(0, n // 2) for n in num_tokens], [(n // 2, n) for n in num_tokens]]


class TwoBatchOverlap:
    """One step as two micro-batches on two streams, software-pipelined by stages.

    Each micro-batch runs the six calls on its own buffers (a MoELayer of its shape; weights
    shared) and on its own stream (both at the default priority).  The calls are grouped in
    stages, split where the pages put their yield points (after dispatch, after the experts):
        stage 0: gather, route, dispatch      stage 1: expert GEMMs      stage 2: combine, scatter
    Micro-batch 1's stage s waits for micro-batch 0's stage s (an event), so on the GPU
    micro-batch 1's memory-bound stage 0 runs beside micro-batch 0's GEMMs, and its GEMMs
    beside micro-batch 0's combine and scatter (the delayed start of the pages' decode
    schedule, one stage deep).  The host only issues work; nothing synchronises it.

    Every per-token result of the path is independent of which tokens share the batch (the
    gate's order is defined per row, expert rows do not interact, combine sums per token), so
    the replica outputs equal the single-batch step's bit for bit."""

    STAGES = (("gather", "route", "dispatch"), ("experts",), ("combine", "scatter"))

    def __init__(self, spec: LayerSpec, weights: DeviceWeights, num_tokens: Sequence[int],
                 act_dtype: torch.dtype, mode: str = "sum", device="cuda", seg_stride: int = 0,
                 cu_split: int = 0, fuse_permute: bool = True):
        """cu_split = n > 0 partitions the CUs (the vLLM page's SM allocation, section
        "第八步：SM 的分配"): both micro-batches' memory stages (0 and 2) run on a stream
        confined to CUs 0 .. n - 1, both micro-batches' expert GEMMs on a stream confined to the
        others.  The runtime numbers CU i on XCD i mod 8 and refuses a mask that leaves an XCD
        without CUs, so n is a multiple of 8 and each XCD gives n / 8 CUs to the small side."""
        self.num_tokens = [int(n) for n in num_tokens]
        self.slices = split_micro_batches(self.num_tokens)
        self.layers = [MoELayer(spec, weights, [b - a for a, b in sl], act_dtype, mode=mode, device=device,
                                seg_stride=seg_stride, fuse_permute=fuse_permute) for sl in self.slices]
        H = spec.hidden
        self.replicas_out = [torch.empty((n, H), dtype=act_dtype, device=device) for n in self.num_tokens]
        self.events = [[torch.cuda.Event() for _ in self.STAGES] for _ in range(2)]
        self.cu_split = int(cu_split)
        self._owned = []
        if self.cu_split > 0:
            from . import moe_stream_create_cu_masked
            cus = torch.cuda.get_device_properties(device).multi_processor_count
            if not 0 < self.cu_split < cus or self.cu_split % 8:
                raise ValueError(f"cu_split must be a multiple of 8 in 8..{cus - 8}")
            small = set(range(self.cu_split))
            words = (cus + 31) // 32
            masks = []
            for member in (lambda i: i in small, lambda i: i not in small):
                m = [0] * words
                for i in range(cus):
                    if member(i):
                        m[i // 32] |= 1 << (i % 32)
                masks.append(m)
            self._owned = [moe_stream_create_cu_masked(m) for m in masks]
            self.mem_stream, self.gemm_stream = (torch.cuda.ExternalStream(h, device=device) for h in self._owned)
        else:
            self.side = torch.cuda.Stream(device=device)

    def __del__(self):
        if getattr(self, "_owned", None):
            from . import moe_stream_destroy
            torch.cuda.synchronize()
            for h in self._owned:
                moe_stream_destroy(h)
            self._owned = []

    def _stage(self, mb: int, s: int, ins, outs):
        layer = self.layers[mb]
        for op in self.STAGES[s]:
            if op == "gather":
                layer.gather(ins)
            elif op == "scatter":
                layer.scatter(outs)
            else:
                getattr(layer, op)()

    def forward(self, replicas) -> List[torch.Tensor]:
        main = torch.cuda.current_stream()
        ins = [[r[a:b] for r, (a, b) in zip(replicas, sl)] for sl in self.slices]
        outs = [[y[a:b] for y, (a, b) in zip(self.replicas_out, sl)] for sl in self.slices]
        if self.cu_split > 0:
            return self._forward_partitioned(main, ins, outs)
        streams = (main, self.side)
        self.side.wait_stream(main)            # inputs written before the step are visible
        for s in range(len(self.STAGES)):
            with torch.cuda.stream(streams[0]):
                self._stage(0, s, ins[0], outs[0])
                self.events[0][s].record(streams[0])
            with torch.cuda.stream(streams[1]):
                streams[1].wait_event(self.events[0][s])
                self._stage(1, s, ins[1], outs[1])
                self.events[1][s].record(streams[1])
        main.wait_event(self.events[1][-1])    # the step ends when both micro-batches have
        return self.replicas_out

    def _forward_partitioned(self, main, ins, outs) -> List[torch.Tensor]:
        """Memory stages of both micro-batches in order on the small partition, GEMMs of both
        in order on the large one; each stage waits for its micro-batch's previous stage, so
        micro-batch 1's stage 0 runs beside micro-batch 0's GEMMs and micro-batch 0's stage 2
        beside micro-batch 1's GEMMs."""
        mem, gemm = self.mem_stream, self.gemm_stream
        mem.wait_stream(main)
        gemm.wait_stream(main)
        # host issue order (micro-batch, stage); on each stream the work runs in this order
        for mb, s in ((0, 0), (1, 0), (0, 1), (1, 1), (0, 2), (1, 2)):
            st = gemm if s == 1 else mem
            with torch.cuda.stream(st):
                if s > 0:
                    st.wait_event(self.events[mb][s - 1])
                self._stage(mb, s, ins[mb], outs[mb])
                self.events[mb][s].record(st)
        main.wait_event(self.events[0][-1])
        main.wait_event(self.events[1][-1])
        return self.replicas_out
