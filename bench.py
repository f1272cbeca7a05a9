#!/usr/bin/env python3
"""Throughput of one rank's MoE layer (DP gather -> route -> dispatch -> SwiGLU grouped GEMM
-> combine -> scatter) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload cfg4]

A step is one pass of all six C-ABI calls over one batch whose inputs are already resident
in HBM (dispatch builds the plan and the up GEMM gathers its rows from the global buffer;
--copy-permute has dispatch write the permuted copy instead).  By default the six calls are
captured once in a HIP graph and each timed step is one replay (--eager launches them call by
call).  Before every timed step a kernel writes a
512 MiB scratch buffer (outside the step's event pair), so the Infinity Cache and the L2 hold
none of the step's data: the step figures are cold-cache ones, as median, p90 and mean over
the timed steps; the same steps back to back give the warm figures beside them.  Prints one
JSON line: tokens/s, the roofline of the dominant kernel (timed with HIP events on the stream
the kernels run on), a per-call breakdown (cold, one eager step per flush), and the CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA, TFLOP/s
FP32_MFMA_PEAK_TFLOPS = 157.3    # fp32 matrix cores (the exact-order gate runs there)
FP8_MFMA_PEAK_TFLOPS = 5000.0    # dense fp8 MFMA, TFLOP/s

WORKLOAD_TEXT = {
    "cfg1": "tiny-fp32: 1 replica x 64 tokens, H=256, E=8 top-2 softmax, I=128",
    "cfg2": "dp4-gather: replicas [37,0,128,5], H=2048, E=64 top-6 softmax, I=1408",
    "cfg3": "dsv3-decode-ep16-B24: 16 replicas x 24 (static bound), H=7168, E=256 grouped top-8, "
            "16 local experts, I=2048",
    "cfg4": "dsv3-prefill-ep16: 8 DP replicas x 4096 tokens, H=7168, E=256 grouped (8 groups, "
            "top-4 groups, top-8), 16 local experts of 256, I=2048",
    "cfg5": "dsv3-zipf-fp8: 8 x 2048 tokens, H=7168, E=256 grouped + Zipf bias, 16 slots / 12 "
            "logical, fp8 weights, I=2048",
}


# profile summaries are named for the kernel and the workload they cover
PROFILE_WORKLOAD = {"cfg4": "prefill_8x4096_bf16", "cfg5": "prefill_8x2048_fp8",
                    "cfg3": "decode_16x24_bf16", "cfg2": "dp4_gather_bf16", "cfg1": "tiny_fp32"}
GEMM_SOURCES = {
    "bf16": ["combine_dp_gather_amd/csrc/expert_gemm.hip", "combine_dp_gather_amd/csrc/gemm_common.h",
             "combine_dp_gather_amd/csrc/moe_dev.h"],
    "fp8": ["combine_dp_gather_amd/csrc/expert_gemm_fp8.hip", "combine_dp_gather_amd/csrc/gemm_common.h",
            "combine_dp_gather_amd/csrc/moe_dev.h"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# placement the --eplb cycle computes: DeepSeek-V3's 256 experts in 8 groups on 256 + 32
# redundant slots, 2 nodes of 9 GPUs, 16 slots per GPU
EPLB = {"P": 288, "groups": 8, "nodes": 2, "gpus": 18}


def eplb_cycle(cfg, inp, layer, reps, args, dev, act):
    """One statistics window (a step under the workload's own slot table), the placement, and
    the layer rebuilt under the new table.  Returns (cfg, inp, weights, layer, summary)."""
    import torch
    import moe_synth
    import combine_dp_gather_amd as m
    from dataclasses import replace
    from combine_dp_gather_amd.layer import DeviceWeights, MoELayer, spec_of
    E, k = cfg.num_experts, cfg.top_k
    phys_h, nrep_h = inp.phys_of, inp.n_rep
    Ph = int(phys_h.max()) + 1
    p2l_h = np.zeros(Ph, dtype=np.int32)
    for e in range(E):
        for r in range(int(nrep_h[e])):
            p2l_h[phys_h[e, r]] = e
    layer.gather(reps)
    layer.route()
    counts = torch.zeros(Ph, dtype=torch.int64, device=dev)
    m.moe_expert_load(layer.topk_ids[:layer.G], layer.emap, Ph, counts)
    logical = torch.empty((1, E), dtype=torch.int64, device=dev)
    m.moe_physical_to_logical_count(counts[None], torch.from_numpy(p2l_h[None]).to(dev), logical)
    loads = logical.cpu().numpy().astype(np.float64)
    p2l, rank, cnt = m.moe_eplb_rebalance(loads, EPLB["P"], EPLB["groups"], EPLB["nodes"], EPLB["gpus"])
    phys_of, n_rep = m.moe_eplb_logical_to_physical(p2l[0], rank[0], E, int(cnt.max()))
    # balancedness over the GPUs: the old table's slots padded to P, then the new table
    old = np.zeros(EPLB["P"], dtype=np.int64)
    old[:Ph] = counts.cpu().numpy()
    before = float(m.moe_eplb_balancedness(old[None], EPLB["gpus"])[0])
    cfg2 = replace(cfg, slot_logical=tuple(int(v) for v in p2l[0, :cfg.num_local]))
    inp2 = moe_synth.make_inputs(cfg2)
    inp2.phys_of, inp2.n_rep = phys_of, n_rep
    del layer
    torch.cuda.empty_cache()
    w2 = DeviceWeights(inp2, dev, fp8_act=args.fp8_act)
    layer2 = MoELayer(spec_of(cfg2), w2, cfg2.num_tokens, act, mode=args.mode,
                      static_bound=cfg2.static_bound, device=dev, seg_stride=args.seg_stride,
                      fuse_permute=not args.copy_permute)
    layer2.gather(reps)
    layer2.route()
    new = torch.zeros(EPLB["P"], dtype=torch.int64, device=dev)
    m.moe_expert_load(layer2.topk_ids[:layer2.G], layer2.emap, EPLB["P"], new)
    after = float(m.moe_eplb_balancedness(new.cpu().numpy()[None], EPLB["gpus"])[0])
    log(f"[bench] EPLB: balancedness over {EPLB['gpus']} GPUs {before:.3f} -> {after:.3f}; "
        f"this GPU holds logical {p2l[0, :cfg.num_local].tolist()}")
    summary = {"kind": "EPLB hierarchical", **EPLB, "this_gpu_slots": [0, cfg.num_local],
               "this_gpu_logical": [int(v) for v in p2l[0, :cfg.num_local]],
               "balancedness_before": round(before, 4), "balancedness_after": round(after, 4)}
    return cfg2, inp2, w2, layer2, summary


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, sample_per_replica: int):
    """The oracle as it stands on the first rows of every replica (a bounded sample): one
    untimed run, then the median of three timed runs."""
    import oracle
    from dataclasses import replace
    import moe_synth
    cfg = inp.cfg
    n = [min(sample_per_replica, v) for v in cfg.num_tokens]
    scfg = replace(cfg, num_tokens=tuple(n), static_bound=0)
    sinp = moe_synth.MoEInputs(cfg=scfg, replicas=[r[:k] for r, k in zip(inp.replicas, n)],
                               router_w=inp.router_w, bias=inp.bias, w13=inp.w13, w2=inp.w2,
                               w13_q=inp.w13_q, w13_s=inp.w13_s, w2_q=inp.w2_q, w2_s=inp.w2_s,
                               phys_of=inp.phys_of, n_rep=inp.n_rep)
    oracle.build()
    oracle.run_layer(sinp, "sum")
    runs = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.run_layer(sinp, "sum")
        runs.append(time.perf_counter() - t0)
    dt = float(np.median(runs))
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(sum(n) / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "logical_cpus": os.cpu_count(),
            "sample": f"first {sample_per_replica} tokens of each replica ({sum(n)} tokens), all six "
                      f"steps; one untimed run, median of 3 timed runs: {dt:.2f} s "
                      f"(runs {', '.join(f'{r:.2f}' for r in runs)} s)"}


def _time_ms(fn, iters=10):
    import torch
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / iters


def ceilings(cfg, R: int) -> dict:
    """Practical ceilings on this GPU, for context next to the spec peaks: a plain device
    copy, and the vendor library GEMM over the same per-slot shapes as the grouped GEMMs."""
    import torch
    out = {}
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    ms = _time_ms(lambda: dst.copy_(src))
    out["device_copy_GBps"] = round(2 * n / ms / 1e6, 1)
    # the same bytes through this library's streaming copy: a one-replica gather of 1 GiB of
    # bf16 rows (block-contiguous spans, non-temporal loads and stores)
    import combine_dp_gather_amd as m
    H = 8192
    rows = n // (2 * H)
    L = m.moe_gather_layout([rows], "sum")
    xs, xd = src.view(torch.bfloat16).view(rows, H), dst.view(torch.bfloat16).view(rows, H)
    rv = torch.empty(rows, dtype=torch.int32, device="cuda")
    ms = _time_ms(lambda: m.moe_gather(L, [xs], xd, rv))
    out["stream_copy_GBps"] = round((2 * n + 4 * rows) / ms / 1e6, 1)
    del src, dst, xs, xd, rv
    if cfg.dtype == "bf16":
        H, I, El = cfg.hidden, cfg.inter, cfg.num_local
        rows = max(R // El, 1)
        bf = torch.bfloat16
        x = torch.randn(El, rows, H, device="cuda", dtype=bf)
        w13 = torch.randn(El, 2 * I, H, device="cuda", dtype=bf)
        w2 = torch.randn(El, H, I, device="cuda", dtype=bf)
        h = torch.randn(El, rows, I, device="cuda", dtype=bf)
        o1 = torch.empty(El, rows, 2 * I, device="cuda", dtype=bf)
        o2 = torch.empty(El, rows, H, device="cuda", dtype=bf)

        def up():
            for e in range(El):
                torch.matmul(x[e], w13[e].t(), out=o1[e])

        def down():
            for e in range(El):
                torch.matmul(h[e], w2[e].t(), out=o2[e])
        for name, fn, fl in (("gemm_up", up, 4.0 * El * rows * H * I), ("gemm_down", down, 2.0 * El * rows * H * I)):
            ms = _time_ms(fn)
            out[f"vendor_{name}_ms"] = round(ms, 4)
            out[f"vendor_{name}_TFLOPs"] = round(fl / ms / 1e9, 1)
        out["vendor_gemm_shape"] = f"{El} slots x {rows} rows, H={H}, I={I}, bf16 (torch.matmul per slot)"
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="scratch written before every timed step (0: no flush)")
    ap.add_argument("--workload", default="cfg4")
    ap.add_argument("--mode", default="sum", choices=["sum", "max", "auto"])
    ap.add_argument("--cpu-sample", type=int, default=1024, help="tokens per replica for the oracle")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fp8-act", default="bf16", choices=["bf16", "e4m3"],
                    help="fp8-weight workloads: keep activations bf16 (weights dequantised in the "
                         "kernel) or quantise them per 1x128 group for the fp8 matrix cores")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step (all six calls) in a HIP graph and time its replays "
                         "(the default)")
    ap.add_argument("--eager", action="store_true",
                    help="launch the six calls one by one each step instead of replaying a graph")
    ap.add_argument("--ceilings", action="store_true",
                    help="also measure practical ceilings: a plain 1 GiB device copy and the vendor "
                         "GEMM (torch.matmul) on the same per-expert shapes")
    ap.add_argument("--entry", action="store_true",
                    help="run the fused entry step (residual add + RMSNorm + gather) in the step "
                         "in place of the plain gather; without it the fused step is timed apart")
    ap.add_argument("--exit", action="store_true",
                    help="run the fused exit (combine written straight into the replicas' buffers) "
                         "in place of combine + scatter")
    ap.add_argument("--seg-stride", type=int, default=0, metavar="ROWS",
                    help="dispatch into the fixed-capacity layout, ROWS rows per local slot (the "
                         "global row count never overflows); 0: packed segments")
    ap.add_argument("--tbo", action="store_true",
                    help="run each step as two micro-batches (each replica's tokens halved) on two "
                         "streams, pipelined by stages; the per-call breakdown comes from "
                         "single-batch steps run after the timed ones")
    ap.add_argument("--cu-split", type=int, default=0, metavar="N",
                    help="with --tbo: run both micro-batches' memory stages on a stream confined to "
                         "CUs 0..N-1 (N a multiple of 8: N/8 on every XCD) and their expert GEMMs on a "
                         "stream confined to the other CUs")
    ap.add_argument("--eplb", action="store_true",
                    help="skewed workload: count one step's expert load under the workload's own "
                         "slot table, place the experts with the library (288 slots, 8 groups, "
                         "2 nodes x 9 GPUs; this GPU holds slots 0-15), and time the step under "
                         "the new table with the per-step load count included")
    ap.add_argument("--copy-permute", action="store_true",
                    help="dispatch writes the permuted copy x_perm and the up GEMM reads it (without "
                         "this flag the up GEMM gathers its rows from the global buffer itself)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB (reference for HBM counters)")
    args = ap.parse_args()
    args.graph = not args.eager
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU: this path has no multi-GPU mode "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_synth
    from combine_dp_gather_amd.layer import DeviceWeights, MoELayer, spec_of

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: {n} bytes read and written per copy")
        del src, dst

    cfg = moe_synth.CONFIGS[args.workload]
    t0 = time.time()
    inp = moe_synth.make_inputs(cfg)
    log(f"[bench] inputs {cfg.name} generated in {time.time() - t0:.1f}s")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    act = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    w = DeviceWeights(inp, dev, fp8_act=args.fp8_act)
    layer = MoELayer(spec_of(cfg), w, cfg.num_tokens, act, mode=args.mode,
                     static_bound=cfg.static_bound, device=dev, seg_stride=args.seg_stride,
                     fuse_permute=not args.copy_permute)
    bf = cfg.dtype == "bf16"
    reps = []
    for r in inp.replicas:
        t = torch.from_numpy(np.ascontiguousarray(r))
        reps.append((t.view(torch.bfloat16) if bf else t).to(dev))
    # the entry step's residual stream and norm weight (the replicas are the attention output)
    ent = moe_synth.make_entry_inputs(cfg, inp.replicas)
    res_dev = []
    for r in ent.residual:
        t = torch.from_numpy(np.ascontiguousarray(r))
        res_dev.append((t.view(torch.bfloat16) if bf else t).to(dev))
    gamma_dev = torch.from_numpy(np.ascontiguousarray(ent.gamma))
    gamma_dev = (gamma_dev.view(torch.bfloat16) if bf else gamma_dev).to(dev)
    torch.cuda.synchronize()
    log(f"[bench] resident in HBM; G={layer.G}")
    eplb_info = None
    if args.eplb:
        cfg, inp, w, layer, eplb_info = eplb_cycle(cfg, inp, layer, reps, args, dev, act)

    stream = torch.cuda.current_stream()
    first = ("entry", lambda: layer.entry(reps, res_dev, gamma_dev, ent.eps)) if args.entry else \
        ("gather", lambda: layer.gather(reps))
    names = [first[0], "route", "dispatch", "gemm_up", "gemm_down"]
    calls = [first[1], layer.route, layer.dispatch, lambda: layer.experts_up(), lambda: layer.experts_down()]
    if args.exit:
        names.append("combine_scatter")
        calls.append(layer.combine_scatter)
    else:
        names += ["combine", "scatter"]
        calls += [layer.combine, layer.scatter]
    if eplb_info is not None:
        # the statistics recorder's per-step work: this step's load of every physical slot
        import combine_dp_gather_amd as m
        load_acc = torch.zeros(EPLB["P"], dtype=torch.int64, device=dev)
        names.append("expert_load")
        calls.append(lambda: m.moe_expert_load(layer.topk_ids[:layer.G], layer.emap, EPLB["P"], load_acc))

    def step(evs=None):
        for i, c in enumerate(calls):
            if evs is not None:
                evs[i][0].record(stream)
            c()
            if evs is not None:
                evs[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    R = int(layer.plan.counts.sum().item())
    # only the slots that received rows have their weights read; an empty slot's weights
    # are not part of the GEMMs' algorithmic bytes
    E_active = int((layer.plan.counts > 0).sum().item())
    overflow = int(layer.plan.error_flag.item())
    log(f"[bench] warmup done; routed local pairs R={R} overflow={overflow}")

    tbo = None
    if args.tbo:
        from combine_dp_gather_amd.layer import TwoBatchOverlap
        if args.entry or args.exit or eplb_info is not None:
            raise SystemExit("--tbo runs the plain six-call step only")
        tbo = TwoBatchOverlap(spec_of(cfg), w, layer.sizes, act, mode=args.mode, device=dev,
                              seg_stride=args.seg_stride, cu_split=args.cu_split,
                              fuse_permute=not args.copy_permute)
        for _ in range(args.warmup):
            tbo.forward(reps)
        torch.cuda.synchronize()

    def whole_step():
        if tbo is not None:
            tbo.forward(reps)
        else:
            step()

    graph = None
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            whole_step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            whole_step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()

    flush = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device=dev) if args.flush_mib else None

    def evict():
        # a kernel writes the scratch buffer, so no earlier data stays in the caches
        if flush is not None:
            flush.fill_(1)

    def new_events(n):
        return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]

    def run_step():
        if graph is not None:
            graph.replay()
        elif tbo is not None:
            tbo.forward(reps)
        else:
            step()

    # the timed steps: K whole steps, each after the cache flush, each bracketed by its events
    cold_ev = new_events(args.steps)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for s in range(args.steps):
        evict()
        cold_ev[s][0].record(stream)
        run_step()
        cold_ev[s][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    cold = np.array([a.elapsed_time(b) for a, b in cold_ev])
    total_ms = float(cold.sum())
    # warm: the same steps back to back, no flush
    warm_ev = new_events(args.steps)
    torch.cuda.synchronize()
    for s in range(args.steps):
        warm_ev[s][0].record(stream)
        run_step()
        warm_ev[s][1].record(stream)
    torch.cuda.synchronize()
    warm = np.array([a.elapsed_time(b) for a, b in warm_ev])
    # per call: K eager single-batch steps, each after the flush, with events around every call
    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
           for _ in names] for _ in range(args.steps)]
    for s in range(args.steps):
        evict()
        step(ev[s])
    torch.cuda.synchronize()
    per_all = {n: np.array([ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)])
               for i, n in enumerate(names)}
    per = {n: float(np.median(v)) for n, v in per_all.items()}

    def stats(v):
        return {"median_ms": round(float(np.median(v)), 4), "p90_ms": round(float(np.percentile(v, 90)), 4),
                "mean_ms": round(float(np.mean(v)), 4)}
    ms_per_step = total_ms / args.steps
    T = cfg.T
    H, I, E, k, G = cfg.hidden, cfg.inter, cfg.num_experts, cfg.top_k, layer.G
    E_slots = cfg.num_local
    es = 2 if bf else 4
    fp8w = cfg.weight_format == "fp8_block"
    # the arithmetic type of the matrix cores: fp8 only when the activations are quantised too
    mm = "mfma8" if fp8w and args.fp8_act == "e4m3" else "mfma"
    wb = 1 if fp8w else es   # weight bytes per element

    def gemm_work(kind, flops, bytes_):
        # below the ridge point (peak flop/s over HBM bytes/s) the GEMM streams its weights
        # and HBM bounds it: report bytes against HBM; above it, flops against the MFMA peak
        ridge = (FP8_MFMA_PEAK_TFLOPS if kind == "mfma8" else BF16_MFMA_PEAK_TFLOPS) * 1e12 / (HBM_PEAK_GBS * 1e9)
        return (kind, flops) if flops / bytes_ >= ridge else ("hbm", bytes_)
    # algorithmic work per call (bytes or flops), per-unit figures x units
    work = {
        "gather": ("hbm", (T + G) * H * es + 4 * G),                   # read T rows, write G rows
        # read attention output and residual, write residual and the gathered row; norm weight
        "entry": ("hbm", 3 * T * H * es + G * H * es + 4 * G + H * es),
        "route": ("mfma32", 2.0 * G * E * H),                          # exact fp32 fma chain + select
        # id passes (+ the x_perm copy when the up GEMM does not gather its rows itself)
        "dispatch": ("hbm", (2 * R * H * es if args.copy_permute else 0) + 3 * 4 * G * k + 8 * R),
        "gemm_up": gemm_work(mm, 4.0 * R * H * I,                     # gate+up: 2*R*H*2I
                             E_active * 2 * I * H * wb + R * H * es + R * I * es),
        "gemm_down": gemm_work(mm, 2.0 * R * I * H, E_active * H * I * wb + R * I * es + R * H * es),
        "combine": ("hbm", R * H * es + G * H * es + 8 * G * k),      # read R rows, write G rows
        "scatter": ("hbm", 2 * T * H * es),
        # read R rows, write the T real rows straight to the replicas
        "combine_scatter": ("hbm", R * H * es + T * H * es + 8 * T * k),
        "expert_load": ("hbm", 4 * G * k + 8 * EPLB["P"]),              # read the ids, add the bins
    }
    peaks = {"hbm": HBM_PEAK_GBS, "mfma32": FP32_MFMA_PEAK_TFLOPS, "mfma": BF16_MFMA_PEAK_TFLOPS,
             "mfma8": FP8_MFMA_PEAK_TFLOPS}
    kernels = {}
    for n in names:
        bound, amount = work[n]
        t_s = per[n] / 1e3
        if bound == "hbm":
            ach = amount / t_s / 1e9 if t_s > 0 else 0.0
            unit = "GB/s"
        else:
            ach = amount / t_s / 1e12 if t_s > 0 else 0.0
            unit = "TFLOP/s"
        kernels[n] = {"ms": round(per[n], 4), "p90_ms": round(float(np.percentile(per_all[n], 90)), 4),
                      "bound": "mfma" if bound.startswith("mfma") else bound,
                      "peak_kind": bound, "achieved": round(ach, 2), "peak": peaks[bound], "unit": unit,
                      "frac": round(ach / peaks[bound], 4)}
    if bf:
        # the FAST gate (bf16 matrix cores, near-tie tolerant ids) timed on its own; the step
        # above routes with the exact gate
        import combine_dp_gather_amd as m
        rc = m.make_route_cfg(cfg.route, E, k, cfg.n_group, cfg.topk_group, cfg.group_topn, cfg.renormalize,
                              gate="fast")
        ms = _time_ms(lambda: m.moe_route(layer.global_x, layer.row_valid, w.router, w.bias, rc, layer.logits,
                                          layer.topk_ids, layer.topk_w), iters=10)
        fb = G * H * 2 + E * H * 2 + G * E * 4 + G * k * 8
        kernels["route_fast"] = {"ms": round(ms, 4), "bound": "hbm", "achieved": round(fb / (ms / 1e3) / 1e9, 2),
                                 "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(fb / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                                 "note": "FAST gate + select, timed apart from the step (which uses the exact gate)"}
    if not args.entry:
        # the fused entry step timed on its own (the step above uses the plain gather); it
        # updates the residual in place, so every call adds the attention output once more
        ms = _time_ms(lambda: layer.entry(reps, res_dev, gamma_dev, ent.eps), iters=10)
        eb = work["entry"][1]
        kernels["entry"] = {"ms": round(ms, 4), "bound": "hbm", "achieved": round(eb / (ms / 1e3) / 1e9, 2),
                            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(eb / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                            "note": "fused residual add + RMSNorm + gather, timed apart from the step "
                                    "(which uses the plain gather)"}
    dom = "gemm_up"
    roof = dict(kernels[dom])
    roof.pop("ms")
    roof.pop("p90_ms")
    roof.pop("peak_kind")
    roof["launch_ms"] = kernels[dom]["ms"]
    roof["timing"] = "median over the timed steps' launches, each after the cache flush"
    fmt = "fp8" if mm == "mfma8" else "bf16"
    # bf16 weights: when no slot can hold more than 512 rows the streaming kernel takes every
    # slot alone (the same rule as the library's launch)
    slot_bound = args.seg_stride if 0 < args.seg_stride < G else G
    kname = ("grouped_gemm_fp8_kernel" if fmt == "fp8"
             else "grouped_gemm_pp_kernel<true, true>" if bf and fp8w
             else "grouped_gemm_stream_kernel<true>" if bf and slot_bound <= 512
             else "grouped_gemm_pp_kernel<true, false>" if bf
             else "generic_gemm_kernel<float, true>")
    roof["kernel"] = kname + (" (gate+up SwiGLU" + (", with its activation quantisation" if fmt == "fp8" else "")
                              + ")")
    from combine_dp_gather_amd.profiling import read_traffic_summary
    summary = os.path.join(ROOT, "profiles", f"grouped_gemm_{fmt}_up__{PROFILE_WORKLOAD[args.workload]}__traffic.txt")
    tb = read_traffic_summary(summary, GEMM_SOURCES[fmt])
    roof["traffic"] = round(tb) if tb is not None else None
    roof["algorithmic_bytes"] = R * H * es + E_active * 2 * I * H * (1 if fp8w else es) + R * I * es
    result = {
        "metric": "MoE-layer tokens/s at 1 GPU; grouped-GEMM % peak MFMA; dispatch/combine % HBM",
        "value": round(T * args.steps / (total_ms / 1e3), 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median": round(float(np.median(cold)), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": (("bf16 activations, fp8 e4m3 weights (fp8 matrix cores)" if mm == "mfma8" else
                   "bf16 activations, fp8 e4m3 weights dequantised to bf16 in the kernel") if fp8w else "bf16")
                 if bf else "f32",
        "data": "synthetic (seeded PCG64; random-init DeepSeek-V3-shaped expert weights)",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "name": cfg.name,
                   "launch": "one HIP graph per step" if args.graph else "eager calls",
                   "micro_batches": (("2, each replica halved, two streams pipelined by stages"
                                      + (f"; memory stages on {args.cu_split} CUs, "
                                         "GEMMs on the others" if args.cu_split else ""))
                                     if args.tbo else "1"),
                   "first_step": "fused residual add + RMSNorm + gather" if args.entry else "plain gather",
                   "last_step": "fused combine + scatter" if args.exit else "combine, then scatter",
                   "dispatch_layout": (f"fixed capacity, {args.seg_stride} rows per slot" if args.seg_stride
                                       else "packed segments"),
                   "permute": ("copy to x_perm in dispatch" if args.copy_permute
                               else "folded into the up GEMM's row loads"),
                   "tokens": T, "global_rows": G, "gather_mode": args.mode,
                   "routed_local_pairs": R, "slots_with_rows": E_active, "parallelism": "one EP rank's share on 1 GPU",
                   **({"placement": eplb_info} if eplb_info is not None else {})},
        "timing": {"cold": stats(cold), "warm": stats(warm),
                   "flush": f"{args.flush_mib} MiB written by a kernel before every cold step, outside its events"
                   if args.flush_mib else "none",
                   "value_from": "timed cold steps: tokens x steps / sum of step times"},
        "roofline": roof,
        "kernels": kernels,
        "wall_s_timed": round(wall, 3),
    }
    if args.ceilings:
        result["ceilings"] = ceilings(cfg, R)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_sample)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
