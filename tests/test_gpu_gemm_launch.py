"""Which grouped-GEMM kernels a call launches must not change its bits.

Batches whose slots can hold at most 512 rows (G, or the fixed capacity) run the streaming
kernel alone, over every slot; larger batches send the slots of more than 64 rows to the
ping-pong kernel.  The same routed rows in the same slots must give the same h and y either
way: here one hot slot of 400 rows runs on the streaming kernel (G = 500) and, with 100 more
global rows that route nowhere (G = 600), on the ping-pong kernel.  Both are also held to a
float64 SwiGLU of the same bf16 operands."""
import numpy as np
import pytest
import torch

from gpu_helpers import say, to_np

pytestmark = pytest.mark.gpu


def _run(m, gx, ids, ew, El, k, H, I):
    G = gx.shape[0]
    emap = m.make_expert_map(El, 0, El)
    plan = m.PlanBuffers(G, k, El, 1, G * k)
    ws = torch.empty(max(m.moe_dispatch_workspace_size(G, k, El), 16), dtype=torch.uint8, device="cuda")
    m.moe_dispatch(gx, ids, emap, plan, None, ws)
    h = torch.zeros((plan.cap, I), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros((plan.cap, H), dtype=torch.bfloat16, device="cuda")
    m.moe_expert_gemm_up_gather(gx, plan, ew, H, I, h)
    m.moe_expert_gemm_down(h, plan, ew, H, I, y)
    torch.cuda.synchronize()
    return plan, h, y


@pytest.mark.parametrize("H,I", [(1024, 512), (2048, 1408)])
def test_stream_only_small_batch_equals_split_launch(H, I):
    import combine_dp_gather_amd as m
    El, k, G0, extra = 8, 2, 500, 100
    say(f"[gemm-launch] H={H} I={I}: G={G0} (streaming kernel only) vs G={G0 + extra} (split launch)")
    gen = torch.Generator(device="cuda").manual_seed(5)
    gx = torch.randn((G0 + extra, H), generator=gen, device="cuda").to(torch.bfloat16)
    rng = np.random.default_rng(3)
    ids = np.full((G0 + extra, k), -1, dtype=np.int32)
    ids[:400, 0] = 0                                   # the hot slot: 400 rows
    ids[:G0, 1] = rng.integers(1, El, G0)               # the rest spread over slots 1..7
    ids_small = torch.from_numpy(ids[:G0].copy()).cuda()
    ids_large = torch.from_numpy(ids).cuda()           # rows 500..599 route nowhere
    w13 = (torch.randn((El, 2, I, H), generator=gen, device="cuda") * 0.03).to(torch.bfloat16)
    w2 = (torch.randn((El, H, I), generator=gen, device="cuda") * 0.03).to(torch.bfloat16)
    ew = m.make_expert_weights(w13, w2)
    ps, hs, ys = _run(m, gx[:G0].contiguous(), ids_small, ew, El, k, H, I)
    pl, hl, yl = _run(m, gx, ids_large, ew, El, k, H, I)
    R = int(to_np(ps.num_rows)[0])
    assert R == int(to_np(pl.num_rows)[0]) and R == 400 + G0
    for a, b in ((ps.counts, pl.counts), (ps.seg_offsets, pl.seg_offsets)):
        assert np.array_equal(to_np(a), to_np(b))
    assert np.array_equal(to_np(ps.sorted_pair)[:R], to_np(pl.sorted_pair)[:R])
    counts = to_np(ps.counts)
    assert counts[0] == 400 and counts[1:].max() <= 100
    assert np.array_equal(to_np(hs)[:R], to_np(hl)[:R])
    assert np.array_equal(to_np(ys)[:R], to_np(yl)[:R])
    say(f"  h and y bitwise equal on all {R} rows (hot slot: {counts[0]} rows)")
    # and both against float64 on the hot slot and one small slot
    seg = to_np(ps.seg_offsets)
    sp = to_np(ps.sorted_pair)[:R]
    x = gx[torch.from_numpy(sp.astype(np.int64) // k).cuda()].double().cpu()
    yd = ys.double().cpu().numpy()[:R]
    for e in (0, 3):
        a, n = int(seg[e]), int(counts[e])
        g = x[a:a + n] @ w13[e, 0].double().cpu().T
        u = x[a:a + n] @ w13[e, 1].double().cpu().T
        hh = g / (1 + torch.exp(-g)) * u
        ref = (hh @ w2[e].double().cpu().T).numpy()
        rows = np.abs(yd[a:a + n] - ref).max(axis=1) / np.maximum(np.abs(ref).max(axis=1), 1e-30)
        say(f"  slot {e} ({n} rows): largest per-row error {rows.max():.3e}")
        assert rows.max() < 2e-2
