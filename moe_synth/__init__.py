"""Seeded synthetic workloads for the single-rank MoE hot path.

This module only draws random numbers and stores them in the formats the
path consumes (fp32, bf16 bit patterns, OCP e4m3 codes with block scales).
It holds none of the method's arithmetic: no gather offsets, no routing, no
permutation, no expert maths.  Both the CPU oracle (``oracle/``) and the HIP
path (``combine_dp_gather_amd``) read the arrays it returns.

Workload shapes follow the SGLang DP-attention / expert-parallel walkthrough
("SGLang 源码完全拆解(十七): DP Attention 与专家并行"): DeepSeek-V3 experts
with gate/up of [2048, 7168] and down of [7168, 2048] (section "EP 下专家权重
切不均匀的问题"), 256 experts split 16 per EP rank (same section), DP replica
token counts that differ between replicas and may be zero (sections
"DpPaddingMode" and "空闲副本也必须参与"), and the static sync bound B=24 of the
DP note (zdszero "DP", section "跳过同步：用约定代替通信").

Random streams: every tensor is split into chunks of ``CHUNK`` values and chunk
``c`` of tensor ``tid`` is drawn from ``PCG64(SeedSequence([seed, tid, c]))``.
The result does not depend on the number of threads used to draw it.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import List, Optional

import numpy as np

CHUNK = 1 << 20
_THREADS = 16

# tensor ids of the random streams
TID_X = 0            # replica i uses TID_X + i  (i < 1000)
TID_ROUTER = 1000
TID_BIAS = 1001
TID_EXPERT = 2000    # local expert e uses TID_EXPERT + 3e + {0 gate, 1 up, 2 down}
TID_RESIDUAL = 4000  # replica i's residual stream uses TID_RESIDUAL + i (i < 1000)
TID_NORM = 5000      # the RMSNorm weight of the layer's entry step


@dataclass(frozen=True)
class MoEConfig:
    name: str
    seed: int
    dtype: str                    # "f32" or "bf16" (activations, router, expert weights)
    num_tokens: tuple             # tokens per DP replica this step
    hidden: int                   # H
    num_experts: int              # E (logical)
    top_k: int                    # k
    route: str                    # "softmax" or "grouped"
    inter: int                    # I (SwiGLU intermediate)
    num_local: int                # E_l physical slots on this rank
    first_local: int = 0          # p0: first physical slot owned by this rank
    n_group: int = 1
    topk_group: int = 1
    group_topn: int = 2           # keys summed per group to score a group
    renormalize: bool = False
    bias: str = "none"            # "none", "uniform" (U(-0.1, 0.1)) or "zipf"
    zipf_s: float = 1.2
    zipf_beta: float = 0.0
    routed_scale: float = 1.0
    static_bound: int = 0         # B > 0: every replica is sized B
    pad_modes: tuple = ("sum",)   # gather modes the workload is run in
    weight_format: str = "dense"  # "dense" (same dtype as activations) or "fp8_block"
    slot_logical: Optional[tuple] = None  # logical expert held by each local slot (None: trivial)
    x_std: float = 1.0
    w_std: float = 0.02

    @property
    def W(self) -> int:
        return len(self.num_tokens)

    @property
    def T(self) -> int:
        return int(sum(self.num_tokens))

    def with_tokens(self, num_tokens, name=None):
        return replace(self, num_tokens=tuple(int(n) for n in num_tokens),
                       static_bound=0, name=name or self.name + "-resized")


def _cfg5_slots():
    # four hot logical experts (0..3) hold two slots each, logical 4..11 one each
    return tuple([0, 0, 1, 1, 2, 2, 3, 3] + list(range(4, 12)))


CONFIGS = {
    "cfg1": MoEConfig(name="tiny-fp32", seed=0, dtype="f32", num_tokens=(64,), hidden=256,
                      num_experts=8, top_k=2, route="softmax", inter=128, num_local=8),
    "cfg2": MoEConfig(name="dp4-gather-bf16", seed=1, dtype="bf16", num_tokens=(37, 0, 128, 5),
                      hidden=2048, num_experts=64, top_k=6, route="softmax", inter=1408,
                      num_local=64, pad_modes=("max", "sum")),
    "cfg3": MoEConfig(name="dsv3-decode-ep16-B24", seed=2, dtype="bf16", num_tokens=(24,) * 16,
                      hidden=7168, num_experts=256, top_k=8, route="grouped", inter=2048,
                      num_local=16, n_group=8, topk_group=4, renormalize=True, bias="uniform",
                      static_bound=24, pad_modes=("max", "sum")),
    "cfg4": MoEConfig(name="dsv3-prefill-ep16", seed=3, dtype="bf16", num_tokens=(4096,) * 8,
                      hidden=7168, num_experts=256, top_k=8, route="grouped", inter=2048,
                      num_local=16, n_group=8, topk_group=4, renormalize=True, bias="uniform"),
    "cfg5": MoEConfig(name="dsv3-zipf-redundant-fp8", seed=4, dtype="bf16", num_tokens=(2048,) * 8,
                      hidden=7168, num_experts=256, top_k=8, route="grouped", inter=2048,
                      num_local=16, n_group=8, topk_group=4, renormalize=True, bias="zipf",
                      zipf_s=1.2, zipf_beta=0.12, weight_format="fp8_block",
                      slot_logical=_cfg5_slots()),
}


# --------------------------------------------------------------------------- random streams

def _chunk_values(seed, tid, c, n, dist, a, b):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, c])))
    if dist == "normal":
        out = rng.standard_normal(n, dtype=np.float32)
        if a != 1.0:
            out *= np.float32(a)
        return out
    return (rng.random(n, dtype=np.float64) * (b - a) + a).astype(np.float32)


class _Req:
    """One tensor to draw: stream (seed, tid), distribution, storage format."""

    def __init__(self, seed, tid, shape, dist="normal", a=1.0, b=0.0, fmt="f32", out=None):
        self.seed, self.tid, self.shape = seed, tid, tuple(int(s) for s in shape)
        self.dist, self.a, self.b, self.fmt = dist, a, b, fmt
        n = int(np.prod(self.shape)) if self.shape else 1
        self.n = n
        dt = np.float32 if fmt == "f32" else np.uint16
        if out is None:
            out = np.empty(n, dtype=dt)
        assert out.dtype == dt and out.size == n and out.flags.c_contiguous
        self.out = out.reshape(n)

    def tasks(self):
        return [(self, c) for c in range(max(1, -(-self.n // CHUNK)))]

    def run(self, c):
        lo = c * CHUNK
        n = min(CHUNK, self.n - lo)
        if n <= 0:
            return
        v = _chunk_values(self.seed, self.tid, c, n, self.dist, self.a, self.b)
        self.out[lo:lo + n] = v if self.fmt == "f32" else to_bf16_bits(v)


def draw_all(reqs):
    """Fill every request; chunks of all tensors are drawn in parallel."""
    tasks = [t for r in reqs for t in r.tasks()]
    if len(tasks) == 1:
        tasks[0][0].run(tasks[0][1])
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(lambda t: t[0].run(t[1]), tasks))
    return [r.out.reshape(r.shape) for r in reqs]


def draw(seed: int, tid: int, shape, dist="normal", std=1.0, lo=0.0, hi=1.0) -> np.ndarray:
    """fp32 array of ``shape`` from the chunked stream (seed, tid)."""
    a, b = (std, 0.0) if dist == "normal" else (lo, hi)
    return draw_all([_Req(seed, tid, shape, dist, a, b, "f32")])[0]


# --------------------------------------------------------------------------- storage formats

def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _e4m3_positive_table():
    """Values of the OCP e4m3fn codes 0x00..0x7E (0x7F is NaN), in code order."""
    vals = np.zeros(0x7F, dtype=np.float64)
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        vals[c] = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3 = _e4m3_positive_table()


def to_e4m3_codes(a: np.ndarray) -> np.ndarray:
    """fp32 -> OCP e4m3fn codes (uint8): round to nearest, ties to even code, saturate at 448."""
    a = np.asarray(a, dtype=np.float64)
    mag = np.minimum(np.abs(a), _E4M3[-1])
    hi = np.clip(np.searchsorted(_E4M3, mag, side="left"), 0, len(_E4M3) - 1)
    lo = np.maximum(hi - 1, 0)
    d_hi = _E4M3[hi] - mag
    d_lo = mag - _E4M3[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((hi & 1) == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return code | np.where(np.signbit(a) & (code != 0), 0x80, 0).astype(np.uint8)


def block_quant_e4m3(w: np.ndarray, block=128):
    """[..., R, C] fp32 -> (e4m3 codes [..., R, C], fp32 scales [..., R/128, C/128]); scale = amax/448."""
    *lead, R, C = w.shape
    assert R % block == 0 and C % block == 0
    wb = w.reshape(*lead, R // block, block, C // block, block)
    amax = np.abs(wb).max(axis=(-3, -1))
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = to_e4m3_codes(wb / scale[..., :, None, :, None])
    return q.reshape(w.shape), scale


# --------------------------------------------------------------------------- workloads

@dataclass
class MoEInputs:
    cfg: MoEConfig
    replicas: List[np.ndarray]          # W arrays [n_i, H]: float32 or uint16 (bf16 bits)
    router_w: np.ndarray                # [E, H] float32 or uint16
    bias: Optional[np.ndarray]          # [E] float32 or None
    w13: Optional[np.ndarray]           # dense: [E_l, 2, I, H] (gate, up)
    w2: Optional[np.ndarray]            # dense: [E_l, H, I]
    w13_q: Optional[np.ndarray] = None  # fp8: uint8 [E_l, 2, I, H]
    w13_s: Optional[np.ndarray] = None  # fp8: float32 [E_l, 2, I/128, H/128]
    w2_q: Optional[np.ndarray] = None   # fp8: uint8 [E_l, H, I]
    w2_s: Optional[np.ndarray] = None   # fp8: float32 [E_l, H/128, I/128]
    phys_of: np.ndarray = None          # int32 [E, max_rep] physical slots of each logical expert
    n_rep: np.ndarray = None            # int32 [E]
    extras: dict = field(default_factory=dict)


def expert_map(cfg: MoEConfig):
    """Logical -> physical slot table.  Without redundancy slot i holds logical i.  With
    ``slot_logical`` the rank's slots [p0, p0+E_l) hold the listed logical experts and every
    other logical expert gets one slot after them."""
    E = cfg.num_experts
    if cfg.slot_logical is None:
        return np.arange(E, dtype=np.int32).reshape(E, 1), np.ones(E, dtype=np.int32)
    slots = {e: [] for e in range(E)}
    for s, lg in enumerate(cfg.slot_logical):
        slots[lg].append(cfg.first_local + s)
    nxt = cfg.first_local + len(cfg.slot_logical)
    for e in range(E):
        if not slots[e]:
            slots[e].append(nxt)
            nxt += 1
    max_rep = max(len(v) for v in slots.values())
    phys = np.full((E, max_rep), -1, dtype=np.int32)
    nrep = np.zeros(E, dtype=np.int32)
    for e, v in slots.items():
        phys[e, :len(v)] = v
        nrep[e] = len(v)
    return phys, nrep


def make_inputs(cfg: MoEConfig, with_experts=True) -> MoEInputs:
    H, E, I, El = cfg.hidden, cfg.num_experts, cfg.inter, cfg.num_local
    sizes = list(cfg.num_tokens)
    if cfg.static_bound > 0:
        sizes = [cfg.static_bound] * cfg.W
    fmt = "f32" if cfg.dtype == "f32" else "bf16"
    reqs = [_Req(cfg.seed, TID_X + i, (n, H), a=cfg.x_std, fmt=fmt) for i, n in enumerate(sizes)]
    reqs.append(_Req(cfg.seed, TID_ROUTER, (E, H), a=cfg.w_std, fmt=fmt))
    if cfg.bias == "uniform":
        reqs.append(_Req(cfg.seed, TID_BIAS, (E,), dist="uniform", a=-0.1, b=0.1))
    drawn = draw_all(reqs)
    replicas, router = drawn[:len(sizes)], drawn[len(sizes)]
    bias = drawn[-1] if cfg.bias == "uniform" else None
    if cfg.bias == "zipf":
        # popularity p_e ~ (e+1)^-s imposed as bias = beta * ln(p_e / p_0)
        e = np.arange(E, dtype=np.float64)
        bias = (cfg.zipf_beta * (-cfg.zipf_s) * np.log(e + 1.0)).astype(np.float32)
    phys, nrep = expert_map(cfg)
    inp = MoEInputs(cfg=cfg, replicas=replicas, router_w=router, bias=bias, w13=None, w2=None,
                    phys_of=phys, n_rep=nrep)
    if not with_experts:
        return inp
    # one weight set per distinct logical expert held locally, copied into each of its slots
    slot_src = list(range(El)) if cfg.slot_logical is None else list(cfg.slot_logical)
    distinct = sorted(set(slot_src), key=slot_src.index)
    first_slot = {lg: slot_src.index(lg) for lg in distinct}
    if cfg.weight_format == "dense":
        w13 = np.empty((El, 2, I, H), dtype=np.float32 if fmt == "f32" else np.uint16)
        w2 = np.empty((El, H, I), dtype=w13.dtype)
        reqs = []
        for j, lg in enumerate(distinct):
            s = first_slot[lg]
            base = TID_EXPERT + 3 * j
            reqs += [_Req(cfg.seed, base + 0, (I, H), a=cfg.w_std, fmt=fmt, out=w13[s, 0]),
                     _Req(cfg.seed, base + 1, (I, H), a=cfg.w_std, fmt=fmt, out=w13[s, 1]),
                     _Req(cfg.seed, base + 2, (H, I), a=cfg.w_std, fmt=fmt, out=w2[s])]
        draw_all(reqs)
        for s, lg in enumerate(slot_src):
            if s != first_slot[lg]:
                w13[s] = w13[first_slot[lg]]
                w2[s] = w2[first_slot[lg]]
        inp.w13, inp.w2 = w13, w2
    else:
        q13 = np.empty((El, 2, I, H), dtype=np.uint8)
        s13 = np.empty((El, 2, I // 128, H // 128), dtype=np.float32)
        q2 = np.empty((El, H, I), dtype=np.uint8)
        s2 = np.empty((El, H // 128, I // 128), dtype=np.float32)
        jobs = []
        for j, lg in enumerate(distinct):
            s = first_slot[lg]
            base = TID_EXPERT + 3 * j
            jobs += [(base + 0, (I, H), q13[s, 0], s13[s, 0]),
                     (base + 1, (I, H), q13[s, 1], s13[s, 1]),
                     (base + 2, (H, I), q2[s], s2[s])]

        def one(job):
            tid, shape, qdst, sdst = job
            w = _Req(cfg.seed, tid, shape, a=cfg.w_std)
            for c in range(max(1, -(-w.n // CHUNK))):
                w.run(c)
            q, sc = block_quant_e4m3(w.out.reshape(shape))
            qdst[...] = q
            sdst[...] = sc

        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(one, jobs))
        for s, lg in enumerate(slot_src):
            if s != first_slot[lg]:
                q13[s], s13[s] = q13[first_slot[lg]], s13[first_slot[lg]]
                q2[s], s2[s] = q2[first_slot[lg]], s2[first_slot[lg]]
        inp.w13_q, inp.w13_s, inp.w2_q, inp.w2_s = q13, s13, q2, s2
    return inp


@dataclass
class EntryInputs:
    """Inputs of the fused entry step: per replica the attention block's output (the
    replica's token rows, the same arrays make_inputs draws) and the residual stream, plus
    the RMSNorm weight.  Residual rows are drawn wider (std residual_std) than the attention
    output, as a residual stream that has accumulated many layers is."""
    hidden: List[np.ndarray]
    residual: List[np.ndarray]
    gamma: np.ndarray
    eps: float


def make_entry_inputs(cfg: MoEConfig, hidden: List[np.ndarray], residual_std: float = 4.0,
                      eps: float = 1e-6) -> EntryInputs:
    """Residual rows shaped like ``hidden`` (the replicas of make_inputs) and a weight drawn
    U(0.5, 1.5), stored in the workload's dtype."""
    fmt = "f32" if cfg.dtype == "f32" else "bf16"
    reqs = [_Req(cfg.seed, TID_RESIDUAL + i, x.shape, a=residual_std, fmt=fmt) for i, x in enumerate(hidden)]
    reqs.append(_Req(cfg.seed, TID_NORM, (cfg.hidden,), dist="uniform", a=0.5, b=1.5, fmt=fmt))
    drawn = draw_all(reqs)
    return EntryInputs(hidden=list(hidden), residual=drawn[:-1], gamma=drawn[-1], eps=eps)


def fake_uniform_logits(seed: int, G: int, E: int) -> np.ndarray:
    """Router logits drawn U(5, 10): the balanced-load device of the expert-location
    dispatch section (ep_dispatch_algorithm "fake") of the SGLang walkthrough."""
    return draw(seed, 3000, (G, E), dist="uniform", lo=5.0, hi=10.0)


def random_logits(seed: int, G: int, E: int, std=1.0) -> np.ndarray:
    return draw(seed, 3001, (G, E), std=std)
