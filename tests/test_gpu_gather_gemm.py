"""The up GEMM with the permute folded into its loads (moe_expert_gemm_up_gather after a
plan-only moe_dispatch) against the copy path (moe_dispatch's permuted copy, then
moe_expert_gemm_up): the same rows in the same order reach the same kernels, so h must be
bit-identical on every routed row, in every kernel the up GEMM can take.  The copy path
itself is held to the oracle by the layer parity tests."""
import numpy as np
import pytest
import torch

import moe_synth
from gpu_helpers import build_layer, copy_path_rows, replicas_to_device, resized, say, to_np

pytestmark = pytest.mark.gpu


def _real_rows(plan, rows):
    counts, seg = to_np(plan.counts), to_np(plan.seg_offsets)
    real = np.zeros(rows, dtype=bool)
    for e in range(len(counts)):
        a = int(seg[e])
        real[a:min(a + int(counts[e]), rows)] = True
    return real


def _plan_arrays(plan, G, k):
    rows = min(int(to_np(plan.num_rows)[0]), plan.cap)
    return (to_np(plan.counts), to_np(plan.seg_offsets), to_np(plan.num_rows), to_np(plan.error_flag),
            to_np(plan.sorted_pair)[:rows], to_np(plan.pair_row)[:G * k])


# (what it covers, config, overrides, fp8_act, seg_stride)
CASES = [
    # slots of more and of fewer than 64 rows: ping-pong and streaming kernels in one call
    ("bf16 pp+stream", "cfg2", dict(num_tokens=(700, 0, 333, 95), hidden=1024, inter=512), "bf16", 0),
    # decode: every slot small (streaming kernel only), with a static-bound gather
    ("bf16 decode", "cfg3", dict(), "bf16", 0),
    # e4m3 weights, bf16 activations: the ping-pong kernel's dequantising form
    ("fp8 weights", "cfg5", dict(num_tokens=(300, 0, 277, 41), hidden=1024, inter=512), "bf16", 0),
    # e4m3 activations: the quantiser gathers, then the fp8 kernel
    ("fp8 e4m3 act", "cfg5", dict(num_tokens=(300, 0, 277, 41), hidden=1024, inter=512), "e4m3", 0),
    # H not a multiple of 256: the generic kernel (bf16 operands on the fp32 matrix cores)
    ("bf16 generic", "cfg2", dict(num_tokens=(200, 61), hidden=320, inter=192), "bf16", 0),
    # fp32 activations: the generic kernel
    ("fp32 generic", "cfg1", dict(), "bf16", 0),
    # the fixed-capacity layout (rows past a slot's pairs hold no pair)
    ("bf16 fixed capacity", "cfg2", dict(num_tokens=(400, 150), hidden=1024, inter=512), "bf16", 512),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gathered_up_gemm_equals_copy_path(case):
    label, name, over, fp8_act, stride = case
    over = dict(over)
    cfg = resized(name, over.pop("num_tokens"), **over) if "num_tokens" in over else \
        (resized(name, moe_synth.CONFIGS[name].num_tokens, **over) if over else moe_synth.CONFIGS[name])
    say(f"[gather-gemm] {label}: tokens={cfg.num_tokens} H={cfg.hidden} I={cfg.inter} "
        f"fp8_act={fp8_act} seg_stride={stride}")
    inp = moe_synth.make_inputs(cfg)
    mode = "max" if cfg.static_bound else "sum"
    layer = build_layer(inp, mode, fp8_act=fp8_act, seg_stride=stride)
    assert layer.fuse_permute and layer.x_perm is None
    layer.forward(replicas_to_device(inp))
    torch.cuda.synchronize()
    G, k = layer.G, cfg.top_k
    plan_only = _plan_arrays(layer.plan, G, k)
    xp, h_copy = copy_path_rows(layer)
    # the plan-only dispatch wrote the plan the copying one writes
    for a, b in zip(plan_only, _plan_arrays(layer.plan, G, k)):
        assert np.array_equal(a, b)
    rows = min(int(to_np(layer.plan.num_rows)[0]), layer.plan.cap)
    real = _real_rows(layer.plan, rows)
    assert real.any()
    assert np.array_equal(to_np(layer.h)[:rows][real], to_np(h_copy)[:rows][real])
    say(f"  h bitwise on {int(real.sum())} routed rows")


def test_gather_past_two_gib_takes_generic_kernel():
    """A global buffer of 2 GiB or more cannot sit behind one buffer resource: the gathering
    up GEMM then runs the generic kernel, held to the float64 SwiGLU of the routed rows."""
    import combine_dp_gather_amd as m
    H, I, El, k = 256, 128, 8, 1
    G = (1 << 22) + 64                        # G * H * 2 bytes just past 2 GiB
    assert G * H * 2 >= 1 << 31
    say(f"[gather-gemm] G={G} H={H} I={I}: global buffer {G * H * 2 / 2**30:.2f} GiB")
    gen = torch.Generator(device="cuda").manual_seed(7)
    gx = torch.randn((G, H), generator=gen, device="cuda").to(torch.bfloat16)
    ids = torch.full((G, k), -1, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(11)
    picked = np.unique(np.concatenate([rng.integers(0, G, 700), np.arange(G - 40, G), np.arange(0, 5)]))
    # slot e takes every pick with (index mod 8) == e, so some slots hold > 64 rows
    sel = torch.from_numpy(picked.astype(np.int64)).cuda()
    ids[sel, 0] = torch.from_numpy((np.arange(len(picked)) % El).astype(np.int32)).cuda()
    ids[sel[:300], 0] = 3
    w13 = (torch.randn((El, 2, I, H), generator=gen, device="cuda") * 0.05).to(torch.bfloat16)
    w2 = (torch.randn((El, H, I), generator=gen, device="cuda") * 0.05).to(torch.bfloat16)
    ew = m.make_expert_weights(w13, w2)
    emap = m.make_expert_map(El, 0, El)
    plan = m.PlanBuffers(G, k, El, 1, len(picked) + 64)
    ws = torch.empty(m.moe_dispatch_workspace_size(G, k, El), dtype=torch.uint8, device="cuda")
    m.moe_dispatch(gx, ids, emap, plan, None, ws)
    h = torch.zeros((plan.cap, I), dtype=torch.bfloat16, device="cuda")
    m.moe_expert_gemm_up_gather(gx, plan, ew, H, I, h)
    torch.cuda.synchronize()
    rows = int(to_np(plan.num_rows)[0])
    assert rows == len(picked) and int(to_np(plan.error_flag)[0]) == 0
    sp = to_np(plan.sorted_pair)[:rows]
    counts, seg = to_np(plan.counts), to_np(plan.seg_offsets)
    assert counts.max() > 64
    x = gx[torch.from_numpy(sp.astype(np.int64) // k).cuda()].float().cpu().double()
    w13c, hd = w13.float().cpu().double(), to_np(h)[:rows]
    worst = 0.0
    for e in range(El):
        a, n = int(seg[e]), int(counts[e])
        if n == 0:
            continue
        g = x[a:a + n] @ w13c[e, 0].T
        u = x[a:a + n] @ w13c[e, 1].T
        ref = (g / (1 + torch.exp(-g)) * u).numpy()
        got = (hd[a:a + n].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        # bf16 output rounding (2^-8 relative) plus fp32 accumulation over H products
        err = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30)
        worst = max(worst, err)
    say(f"  generic gathered h against float64: largest relative error {worst:.3e}")
    assert worst < 1e-2
