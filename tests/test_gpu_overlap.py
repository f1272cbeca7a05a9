"""Two-micro-batch overlap on one GPU: the step split into two micro-batches that run on two
streams, software-pipelined by stages.  Every per-token result of the path is independent of
the batch it rides in, so the replica outputs must equal the single-batch step's bit for bit;
the step is also checked against the oracle, and captured in one HIP graph (both streams)
whose replays must equal the eager overlapped step."""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from gpu_helpers import act_dtype, build_layer, replicas_to_device, resized, say, to_np, tol_for

pytestmark = pytest.mark.gpu


def _tbo(inp, layer):
    from combine_dp_gather_amd.layer import TwoBatchOverlap, spec_of
    cfg = inp.cfg
    return TwoBatchOverlap(spec_of(cfg), layer.w, layer.sizes, act_dtype(cfg), mode="sum")


CASES = {
    "dp-gather": lambda: moe_synth.CONFIGS["cfg2"],                       # ragged, one idle replica
    "decode": lambda: moe_synth.CONFIGS["cfg3"],                          # 16 x 24 (static bound)
    "mid": lambda: resized("cfg4", (611, 0, 1203, 377), hidden=2048, inter=1024, num_experts=64),
    "tiny-halves": lambda: resized("cfg2", (1, 3, 0, 2)),                 # micro-batch 0 nearly empty
    "skewed-fp8": lambda: resized("cfg5", (512, 300, 0, 77)),             # fp8 weights, replicated slots
}


@pytest.mark.parametrize("name", list(CASES))
def test_overlapped_step_equals_single_batch(name):
    cfg = CASES[name]()
    say(f"[overlap] {name}: tokens={cfg.num_tokens} H={cfg.hidden} E={cfg.num_experts}")
    inp = moe_synth.make_inputs(cfg)
    layer = build_layer(inp, "sum")
    reps = replicas_to_device(inp)
    single = [to_np(y).copy() for y in layer.forward(reps)]
    tbo = _tbo(inp, layer)
    outs = tbo.forward(reps)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(outs, single)):
        assert np.array_equal(to_np(a), b), f"replica {i}"
    # and the oracle
    ref = oracle.run_layer(inp, "sum")
    tol = tol_for(cfg)
    for i, y in enumerate(outs):
        if y.shape[0]:
            assert oracle.rel_err(oracle.as_f32(to_np(y)), ref["replicas_out"][i]) < tol
    say(f"  micro-batches {[sum(b - a for a, b in sl) for sl in tbo.slices]} tokens; outputs equal the single batch")


@pytest.mark.parametrize("name,split", [("decode", 32), ("mid", 64), ("skewed-fp8", 48)])
def test_cu_partitioned_step_equals_single_batch(name, split):
    """Memory stages on a stream confined to a few CUs, GEMMs on a stream confined to the rest:
    the persistent kernels size their grids to their stream's CUs, and every tile and row
    computes as before, so the outputs still equal the single-batch step bit for bit."""
    from combine_dp_gather_amd.layer import TwoBatchOverlap, spec_of
    cfg = CASES[name]()
    say(f"[overlap] CU split {split} {name}: tokens={cfg.num_tokens}")
    inp = moe_synth.make_inputs(cfg)
    layer = build_layer(inp, "sum")
    reps = replicas_to_device(inp)
    single = [to_np(y).copy() for y in layer.forward(reps)]
    tbo = TwoBatchOverlap(spec_of(cfg), layer.w, layer.sizes, act_dtype(cfg), mode="sum",
                          cu_split=split)
    for _ in range(2):
        outs = tbo.forward(reps)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, single)):
            assert np.array_equal(to_np(a), b), f"replica {i}"
    del tbo


def test_overlapped_step_graph_replays():
    """vLLM captures its two-micro-batch step as one full graph over both streams; the same
    here, replayed three times with eager work between replays."""
    cfg = moe_synth.CONFIGS["cfg3"]
    inp = moe_synth.make_inputs(cfg)
    layer = build_layer(inp, "sum")
    reps = replicas_to_device(inp)
    tbo = _tbo(inp, layer)
    eager = [to_np(y).copy() for y in tbo.forward(reps)]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        tbo.forward(reps)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        tbo.forward(reps)
    torch.cuda.synchronize()
    for replay in range(3):
        for y in tbo.replicas_out:
            y.fill_(float("nan"))
        for l in tbo.layers:
            l.out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(tbo.replicas_out, eager)):
            assert np.array_equal(to_np(a), b), f"replay {replay} replica {i}"
    say("  3 graph replays of the overlapped step equal the eager one")
