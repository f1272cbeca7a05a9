"""GPU parity: every step of the HIP path, called through the C ABI, against the CPU oracle
on the same seeded inputs.

Bar: bit-exact for the gather buffer, row validity, logits (exact-order gate), expert ids,
the whole dispatch plan and the permuted rows; max relative error (infinity norm) within
2e-2 for bf16 outputs and 1e-4 for the fp32 configuration."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import moe_synth
import oracle
from gpu_helpers import (build_layer, check_combine_bound, copy_path_rows, replicas_to_device, resized, say,
                         to_np, tol_for)

pytestmark = pytest.mark.gpu


def run_and_compare(cfg, mode="sum", align=1, cap=None, check_mode_pair=None, fp8_act="bf16", seg_stride=0,
                    fuse_permute=True):
    return run_and_compare_inputs(moe_synth.make_inputs(cfg), mode, align, cap, fp8_act, seg_stride,
                                  fuse_permute)


def run_and_compare_inputs(inp, mode="sum", align=1, cap=None, fp8_act="bf16", seg_stride=0,
                           fuse_permute=True):
    """The six steps on the GPU against the oracle on the same inputs (expert table included).
    seg_stride > 0: the fixed-capacity dispatch layout on both sides.  fuse_permute (the
    layer's default): the up GEMM gathers its rows from global_x; the permuted copy and the
    plain up GEMM then run beside it, the copy is held to the oracle and the two h to each
    other bit for bit."""
    cfg = inp.cfg
    say(f"[parity] {cfg.name} tokens={cfg.num_tokens} H={cfg.hidden} I={cfg.inter} "
        f"E={cfg.num_experts} k={cfg.top_k} mode={mode} align={align} cap={cap} seg_stride={seg_stride} "
        f"fuse_permute={fuse_permute}")
    ref = oracle.run_layer(inp, mode, align=align, cap=cap, seg_stride=seg_stride, fp8_act=fp8_act)
    layer = build_layer(inp, mode, align, cap, fp8_act, seg_stride, fuse_permute)
    reps = replicas_to_device(inp)
    layer.forward(reps)
    torch.cuda.synchronize()
    G = layer.G
    assert G == ref["layout"][1]
    assert layer.offsets == ref["layout"][2]
    if G == 0:
        for r in layer.replicas_out:
            assert r.shape[0] == 0
        return layer, ref
    # S1 gather: bitwise
    assert np.array_equal(to_np(layer.global_x), ref["global_x"])
    assert np.array_equal(to_np(layer.row_valid)[:G], ref["row_valid"])
    # S2 route: logits and ids bitwise, weights to tolerance
    assert np.array_equal(to_np(layer.logits)[:G].view(np.uint32), ref["logits"].view(np.uint32))
    assert np.array_equal(to_np(layer.topk_ids)[:G], ref["ids"])
    assert oracle.rel_err(to_np(layer.topk_w)[:G], ref["weights"]) < 1e-5
    # S3 dispatch: plan bitwise
    plan, rp = layer.plan, ref["plan"]
    assert np.array_equal(to_np(plan.counts), rp["counts"])
    assert np.array_equal(to_np(plan.seg_offsets), rp["seg_offsets"])
    assert int(to_np(plan.num_rows)[0]) == rp["num_rows"]
    assert int(to_np(plan.error_flag)[0]) == rp["error_flag"]
    rows = min(rp["num_rows"], rp["cap"])
    assert np.array_equal(to_np(plan.sorted_pair)[:rows], rp["sorted_pair"])
    assert np.array_equal(to_np(plan.pair_row)[:G * cfg.top_k], rp["pair_row"])
    real = np.zeros(rows, dtype=bool)
    for e in range(cfg.num_local):
        a = int(rp["seg_offsets"][e])
        real[a:min(a + int(rp["counts"][e]), rows)] = True
    if layer.x_perm is None:
        xp_dev, h_copy = copy_path_rows(layer)
        assert np.array_equal(to_np(layer.h)[:rows][real], to_np(h_copy)[:rows][real])
        say(f"  gathering up GEMM: h bitwise equal to the copy path's on {int(real.sum())} rows")
    else:
        xp_dev = layer.x_perm
    xp_gpu = to_np(xp_dev)[:rows]
    if seg_stride:  # fixed capacity: rows past a segment's pairs are never written
        used = rp["sorted_pair"] >= 0
        assert np.array_equal(xp_gpu[used], ref["x_perm"][used])
    else:
        assert np.array_equal(xp_gpu, ref["x_perm"])
    # S4 experts: real rows of every segment.  With e4m3 activations the oracle quantises them
    # too (the codes of x_perm are the same bits; those of h can differ by one step where the
    # two sides' h land on opposite sides of a rounding boundary), held to the fp8 bar
    tol = tol_for(cfg)
    if real.any():
        y_gpu = oracle.as_f32(to_np(layer.y_perm)[:rows])[real]
        err = oracle.rel_err(y_gpu, ref["y_perm"][real])
        err_row = oracle.row_rel_err(y_gpu, ref["y_perm"][real])
        say(f"  y_perm rel err {err:.3e}, largest per-row {err_row:.3e}")
        assert err < tol and err_row < tol
    # S5 combine: in isolation on the device's own y_perm and weights (element bound), and
    # against the oracle's whole layer, per row
    worst = check_combine_bound(to_np(layer.out), to_np(layer.y_perm)[:max(rows, 1)],
                                to_np(layer.topk_w)[:G], rp["pair_row"], cfg.top_k)
    out = oracle.as_f32(to_np(layer.out))
    err = oracle.rel_err(out, ref["out"])
    err_row = oracle.row_rel_err(out, ref["out"])
    say(f"  combine {worst:.2f} of its bound; out rel err {err:.3e}, largest per-row {err_row:.3e}")
    assert err < tol and err_row < tol
    no_pair = (rp["pair_row"].reshape(G, cfg.top_k) < 0).all(axis=1)
    assert np.all(out[no_pair] == 0)           # rows with no local pair are exactly zero
    # S6 scatter: a copy of the GPU's own out, bitwise; and the oracle within tolerance
    out_np = to_np(layer.out)
    for i, y in enumerate(layer.replicas_out):
        a, n = layer.offsets[i], layer.sizes[i]
        assert np.array_equal(to_np(y), out_np[a:a + n])
        if n:
            assert oracle.rel_err(oracle.as_f32(to_np(y)), ref["replicas_out"][i]) < tol
    return layer, ref


def test_cfg1_tiny_fp32():
    run_and_compare(moe_synth.CONFIGS["cfg1"])


@pytest.mark.parametrize("mode", ["max", "sum"])
def test_cfg2_dp_gather_bf16(mode):
    run_and_compare(moe_synth.CONFIGS["cfg2"], mode)


def test_cfg2_modes_bitwise_equal():
    cfg = moe_synth.CONFIGS["cfg2"]
    outs = {}
    for mode in ("max", "sum"):
        inp = moe_synth.make_inputs(cfg)
        layer = build_layer(inp, mode)
        layer.forward(replicas_to_device(inp))
        torch.cuda.synchronize()
        outs[mode] = [to_np(y) for y in layer.replicas_out]
    for a, b in zip(outs["max"], outs["sum"]):
        assert np.array_equal(a, b)
    assert outs["sum"][1].shape[0] == 0           # idle replica


@pytest.mark.parametrize("mode", ["max", "sum"])
def test_cfg3_decode_static_bound(mode):
    run_and_compare(moe_synth.CONFIGS["cfg3"], mode)


@pytest.mark.parametrize("fp8_act", ["bf16", "e4m3"])
def test_cfg5_fp8_block_scaled_small(fp8_act):
    # Zipf-biased routing, 16 slots holding 12 logical experts (4 hot ones twice), e4m3
    # weights with 128x128 block scales; reduced H and I keep several tiles per slot.
    # Both ways of meeting the activations: bf16 with in-kernel weight dequantisation, and
    # per-1x128-group e4m3 activations on the fp8 matrix cores
    cfg = resized("cfg5", (300, 0, 277, 41), hidden=1024, inter=512)
    layer, ref = run_and_compare(cfg, fp8_act=fp8_act)
    if fp8_act == "e4m3":
        # what the quantisation itself costs against the unquantised experts (reported)
        exact = oracle.expert_ffn(ref["x_perm"], ref["plan"], moe_synth.make_inputs(cfg))
        rows = ref["plan"]["num_rows"]
        say(f"  e4m3 activations against unquantised experts: rel err "
            f"{oracle.rel_err(ref['y_perm'][:rows], exact[:rows]):.3e}, largest per-row "
            f"{oracle.row_rel_err(ref['y_perm'][:rows], exact[:rows]):.3e}")


@pytest.mark.parametrize("K", [1024, 640, 7168])
def test_quant_act_fp8_bitwise(K):
    """The per-token-group quantisation step on its own: every code and scale equals the
    oracle's, for rows of wildly different magnitudes, an all-zero group, a group of tiny
    values (subnormal codes) and a group whose values sit on code midpoints; rows past
    num_rows stay untouched.  K = 640 has five groups, so the kernel's last four-group step
    is partly masked."""
    import combine_dp_gather_amd as m
    rng = np.random.default_rng(17)
    cap, nrows = 700, 613
    x = (rng.standard_normal((cap, K)) * np.exp(rng.uniform(-30, 30, (cap, 1)))).astype(np.float32)
    x[5, 128:256] = 0.0
    x[6, :128] *= np.float32(2.0 ** -12)
    x[6, 0] = 1.0                       # the rest of the group falls below 2^-6 of its scale
    # group 2 of row 7: 448 and exact midpoints of e4m3 codes at scale 1
    pos = oracle.e4m3_decode(np.arange(0x08, 0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    x[7, 256:384] = np.resize(mids, 128).astype(np.float32)
    x[7, 256] = 448.0
    xb = oracle.bf16_rne(x.astype(np.float64))
    xd = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda()
    q = torch.full((cap, K), 0xAB, dtype=torch.uint8, device="cuda")
    st = torch.full((K // 128, cap), -1.0, dtype=torch.float32, device="cuda")
    m.moe_quant_act_fp8(xd, torch.tensor([nrows], dtype=torch.int64, device="cuda"), q, st)
    torch.cuda.synchronize()
    rq, rs = oracle.quant_group_e4m3(xb[:nrows])
    assert np.array_equal(q.cpu().numpy()[:nrows], rq)
    assert np.array_equal(st.cpu().numpy()[:, :nrows].view(np.uint32), rs.T.view(np.uint32))
    assert np.all(q.cpu().numpy()[nrows:] == 0xAB) and np.all(st.cpu().numpy()[:, nrows:] == -1.0)
    assert rs[5, 1] == 1.0 and not rq[5, 128:256].any()


def test_multi_tile_ragged_segments():
    # E=64 with 16 local slots gives ~2T/16 rows per slot: several 256-row tiles plus a
    # ragged tail per slot; replica counts ragged with an idle replica
    cfg = resized("cfg4", (611, 0, 1203, 377, 1, 809), hidden=2048, inter=1024, num_experts=64)
    run_and_compare(cfg)


def test_expert_gemm_unaligned_buffers_take_generic_path():
    # an output 2 bytes off an 8-byte boundary cannot take the tile epilogue's 8-byte stores,
    # nor an input off 16 bytes its DMAs: the bf16 GEMMs then run the generic kernel on the
    # fp32 matrix cores, held to the same bar against the oracle, and the query says so
    from combine_dp_gather_amd import moe_expert_gemm_down, moe_expert_gemm_fast_path, moe_expert_gemm_up
    cfg = resized("cfg4", (300, 0, 517), hidden=2048, inter=1024, num_experts=64)
    layer, ref = run_and_compare(cfg, fuse_permute=False)
    rp = ref["plan"]
    rows = min(rp["num_rows"], rp["cap"])
    real = np.zeros(rows, dtype=bool)
    for e in range(cfg.num_local):
        a = int(rp["seg_offsets"][e])
        real[a:min(a + int(rp["counts"][e]), rows)] = True
    assert real.any()
    H, I = cfg.hidden, cfg.inter
    hbuf = torch.zeros(layer.h.numel() + 1, dtype=layer.h.dtype, device=layer.h.device)
    h_odd = hbuf[1:].view(layer.h.shape)
    ybuf = torch.zeros(layer.y_perm.numel() + 1, dtype=layer.y_perm.dtype, device=layer.y_perm.device)
    y_odd = ybuf[1:].view(layer.y_perm.shape)
    layer.experts_up()  # h from the tile path
    assert moe_expert_gemm_fast_path(layer.x_perm, layer.w.ew, H, I, layer.h, layer.y_perm)
    assert not moe_expert_gemm_fast_path(layer.x_perm, layer.w.ew, H, I, h_odd, layer.y_perm)
    assert not moe_expert_gemm_fast_path(layer.x_perm, layer.w.ew, H, I, layer.h, y_odd)
    say("[parity] generic-path GEMMs: h and y_perm 2 bytes off alignment")
    moe_expert_gemm_up(layer.x_perm, layer.plan, layer.w.ew, H, I, h_odd, layer.gemm_ws)
    moe_expert_gemm_down(h_odd, layer.plan, layer.w.ew, H, I, y_odd, layer.gemm_ws)
    torch.cuda.synchronize()
    tol = tol_for(cfg)
    h_tile = oracle.as_f32(to_np(layer.h)[:rows])[real]
    err_h = oracle.rel_err(oracle.as_f32(to_np(h_odd)[:rows])[real], h_tile)
    err_y = oracle.rel_err(oracle.as_f32(to_np(y_odd)[:rows])[real], ref["y_perm"][real])
    say(f"  h vs tile path {err_h:.3e}, y_perm vs oracle {err_y:.3e}")
    assert err_h < tol and err_y < tol


def test_alignment_128():
    cfg = resized("cfg3", (17, 40, 0, 33), hidden=2048, inter=1024)
    run_and_compare(cfg, "sum", align=128)


def test_capacity_overflow_truncates_like_oracle():
    cfg = resized("cfg3", (40, 40), hidden=1024, inter=512, num_experts=64)
    run_and_compare(cfg, "sum", align=1, cap=37)


def test_all_idle_is_noop():
    cfg = resized("cfg2", (0, 0, 0))
    run_and_compare(cfg, "max")


def test_single_token():
    cfg = resized("cfg2", (0, 1, 0))
    run_and_compare(cfg, "sum")


def test_determinism_two_runs_bitwise():
    cfg = resized("cfg4", (300, 211, 0, 97), hidden=2048, inter=1024, num_experts=64)
    inp = moe_synth.make_inputs(cfg)
    layer = build_layer(inp)
    reps = replicas_to_device(inp)
    outs = []
    for _ in range(2):
        layer.forward(reps)
        torch.cuda.synchronize()
        outs.append([to_np(layer.out).copy(), to_np(layer.y_perm).copy(), to_np(layer.plan.sorted_pair).copy()])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_gather_then_scatter_identity_and_idle_rows():
    import combine_dp_gather_amd as m
    rng = np.random.default_rng(3)
    n = [5, 0, 33, 2, 0, 17]
    H = 72  # 144-byte rows: exercises the narrower copy unit
    for mode in ("max", "sum"):
        L = m.moe_gather_layout(n, mode)
        reps = [torch.from_numpy(rng.standard_normal((v, H)).astype(np.float32)).to(torch.bfloat16).cuda()
                for v in n]
        gx = torch.full((L.rows, H), float("nan"), dtype=torch.bfloat16, device="cuda")
        rv = torch.full((L.rows,), 7, dtype=torch.int32, device="cuda")
        m.moe_gather(L, reps, gx, rv)
        back = [torch.empty_like(r) for r in reps]
        m.moe_scatter(L, gx, back)
        torch.cuda.synchronize()
        for a, b in zip(reps, back):
            assert torch.equal(a, b)
        valid = rv.cpu().numpy()
        assert valid.sum() == sum(n)
        assert torch.all(gx[torch.from_numpy(valid == 0).cuda()] == 0)


@pytest.mark.parametrize("name,mode,tokens", [("cfg2", "sum", None), ("cfg2", "max", None),
                                               ("cfg3", "max", None), ("cfg2", "sum", (3, 0, 40, 0, 7, 1)),
                                               ("cfg1", "sum", None)])
def test_fused_exit_equals_combine_then_scatter(name, mode, tokens):
    """moe_combine_scatter writes the same bits into the replica buffers as moe_combine followed
    by moe_scatter (ragged and idle replicas, both padding modes; the oracle already checks the
    two-call path), and leaves the global output buffer untouched."""
    cfg = moe_synth.CONFIGS[name] if tokens is None else resized(name, tokens)
    inp = moe_synth.make_inputs(cfg)
    say(f"[fused-exit] {cfg.name} tokens={cfg.num_tokens} mode={mode}")
    layer = build_layer(inp, mode)
    reps = replicas_to_device(inp)
    two = [r.clone() for r in layer.forward(reps)]
    layer.out.fill_(3.0)
    fresh = [torch.full_like(r, 5.0) for r in two]
    layer.combine_scatter(fresh)
    torch.cuda.synchronize()
    for a, b in zip(two, fresh):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))  # bitwise, any dtype
    assert torch.all(layer.out == 3.0)
    again = [r.clone() for r in layer.forward(reps, fused_exit=True)]
    torch.cuda.synchronize()
    for a, b in zip(two, again):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_identity_experts_combine_returns_weighted_sum():
    import combine_dp_gather_amd as m
    cfg = resized("cfg3", (50, 31), hidden=1024, inter=512, num_experts=64, num_local=64)
    inp = moe_synth.make_inputs(cfg)
    layer = build_layer(inp, fuse_permute=False)
    layer.gather(replicas_to_device(inp))
    layer.route()
    layer.dispatch()
    out = torch.empty_like(layer.out)
    # y_perm := x_perm (identity experts)
    m.moe_combine(layer.x_perm, layer.plan, layer.topk_w, 1.0, out)
    torch.cuda.synchronize()
    # every element within one bf16 ulp plus the fp32 accumulation bound of the float64
    # sum_j w_j x_g, which (every expert local, weights renormalised) is x_g itself
    G, k = layer.G, cfg.top_k
    check_combine_bound(to_np(out), to_np(layer.x_perm), to_np(layer.topk_w)[:G],
                        to_np(layer.plan.pair_row)[:G * k], k)
    x = layer.global_x.float().cpu().double()
    w = layer.topk_w[:G].cpu().double()
    assert torch.allclose(w.sum(dim=1, keepdim=True) * x, x, atol=1e-5)
    pr = to_np(layer.plan.pair_row)[:G * k].reshape(G, k)
    assert np.array_equal(to_np(layer.x_perm)[pr], np.repeat(to_np(layer.global_x)[:, None, :], k, axis=1))


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_gate_kernels_bitwise(dt):
    # every gate kernel against the oracle's single ascending fma chain, bit for bit, with
    # ragged row and expert tiles (E = 200) and every 17th row a pad row:
    #   - small batches (at most one block per CU: two chain waves fed by two helper waves):
    #     G = 300 at H = 384 (subnormal products and partial sums), 448, 1000 (ragged last
    #     slice) and 232, G = 200 at the model's H = 7168, and tiny shapes (one row; one slice,
    #     whole or ragged: the helper waves stage mostly padding);
    #   - 16x16 chains, 16-byte loads (H a multiple of 64): G = 1000 at H = 7168;
    #   - 16x16 chains, element loads (ragged last slice): G = 6000 at H = 1000, and a batch
    #     large enough for 128-row blocks but with H = 232 (G = 16347);
    #   - the 32x32-chain kernels: G = 16384 (64-row blocks, 4 waves) and 33000 (128-row
    #     blocks, 8 waves) at H = 256 (also subnormal) and 384;
    #   - rows whose chain ends at -0 (one tiny negative product in the last real column of
    #     a ragged H): the padded columns must leave the sign of zero in place.
    import combine_dp_gather_amd as m
    rng = np.random.default_rng(21)
    cfg = m.make_route_cfg("softmax", 200, 4)
    cases = ((300, 384, 2.0 ** -66), (300, 448, 1.0), (200, 7168, 1.0), (1000, 7168, 1.0), (300, 1000, 1.0),
             (6000, 1000, 1.0), (1, 64, 1.0), (5, 40, 1.0), (17, 130, 1.0),
             (128 * 128 - 37, 232, 1.0), (16384, 256, 1.0), (33000, 384, 1.0), (33000, 256, 2.0 ** -66),
             (300, 232, "negzero"), (33000, 200, "negzero"))
    for G, H, scale in cases:
        say(f"[gate] dtype={dt} G={G} H={H} E=200 scale={scale}")
        s = 1.0 if scale == "negzero" else scale
        xf = (rng.standard_normal((G, H)) * s).astype(np.float32)
        wf = (rng.standard_normal((200, H)) * 0.05 * s).astype(np.float32)
        if scale == "negzero":
            # rows 1, 5, 9, ...: only the last column is non-zero, and its products with
            # every expert round to -0
            xf[1::4] = 0.0
            xf[1::4, H - 1] = -(2.0 ** -100)
            wf[:, H - 1] = 2.0 ** -100
        x = torch.from_numpy(xf).to(dt)
        w = torch.from_numpy(wf).to(dt)
        rv = np.ones(G, dtype=np.int32)
        rv[16::17] = 0
        xb = x.view(torch.int16).numpy().view(np.uint16) if dt == torch.bfloat16 else x.numpy()
        wb = w.view(torch.int16).numpy().view(np.uint16) if dt == torch.bfloat16 else w.numpy()
        ref = oracle.gate_logits(xb, wb, row_valid=rv)
        if scale == "negzero":
            neg = ref[1::4][rv[1::4] != 0]
            assert np.all(np.signbit(neg)) and np.all(neg == 0)
        elif scale < 1:
            assert np.any((ref != 0) & (np.abs(ref) < np.finfo(np.float32).tiny))
        xd, wd, rvd = x.cuda(), w.cuda(), torch.from_numpy(rv).cuda()
        lg = torch.full((G, 200), float("nan"), device="cuda")
        ids = torch.empty((G, 4), dtype=torch.int32, device="cuda")
        tw = torch.empty((G, 4), dtype=torch.float32, device="cuda")
        m.moe_route(xd, rvd, wd, None, cfg, lg, ids, tw)
        torch.cuda.synchronize()
        assert np.array_equal(lg.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_route_from_logits_ties_and_fake_balance():
    import combine_dp_gather_amd as m
    # constructed exact ties: equal logits -> lowest ids, in order
    G, E = 8, 256
    lg = np.zeros((G, E), dtype=np.float32)
    lg[1, 200] = 1.0
    cfg = m.make_route_cfg("grouped", E, 8, 8, 4, 2, True)
    ids = torch.empty((G, 8), dtype=torch.int32, device="cuda")
    w = torch.empty((G, 8), dtype=torch.float32, device="cuda")
    m.moe_route_from_logits(torch.from_numpy(lg).cuda(), None, None, cfg, ids, w)
    torch.cuda.synchronize()
    ref_ids, ref_w = oracle.select_grouped(lg, None, 8, 4, 8, True)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert list(ref_ids[0]) == list(range(8))
    # the fake dispatch: logits U(5,10), no bias -> near-uniform load, ids bitwise
    G = 4096
    lg = moe_synth.fake_uniform_logits(0, G, E)
    ids = torch.empty((G, 8), dtype=torch.int32, device="cuda")
    w = torch.empty((G, 8), dtype=torch.float32, device="cuda")
    m.moe_route_from_logits(torch.from_numpy(lg).cuda(), None, torch.zeros(E, device="cuda"), cfg, ids, w)
    torch.cuda.synchronize()
    ref_ids, ref_w = oracle.select_grouped(lg, np.zeros(E, np.float32), 8, 4, 8, True)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert oracle.rel_err(w.cpu().numpy(), ref_w) < 1e-6
    hist = np.bincount(ref_ids.ravel(), minlength=E)
    assert hist.max() < 1.4 * G * 8 / E
    # softmax path with ties
    lg = np.random.default_rng(1).standard_normal((500, 64)).astype(np.float32)
    lg[:, 7] = lg[:, 3]
    cfgs = m.make_route_cfg("softmax", 64, 6, renormalize=True)
    ids = torch.empty((500, 6), dtype=torch.int32, device="cuda")
    w = torch.empty((500, 6), dtype=torch.float32, device="cuda")
    m.moe_route_from_logits(torch.from_numpy(lg).cuda(), None, None, cfgs, ids, w)
    torch.cuda.synchronize()
    ref_ids, ref_w = oracle.select_softmax(lg, 6, True)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert oracle.rel_err(w.cpu().numpy(), ref_w) < 1e-5


def test_route_picks_near_ties():
    """Keys that differ in fp64 but round to one fp32 value, exactly equal keys, and +0 / -0
    logits: the picks follow the exact (key, lower id) order, as in the oracle."""
    import combine_dp_gather_amd as m
    rng = np.random.default_rng(7)
    G, E = 64, 256
    lg = rng.uniform(-1.0, 1.0, (G, E)).astype(np.float32)
    for r in range(G):
        # 24 experts spread over the lanes and groups at consecutive fp32 logits near 2: their
        # sigmoids are ~2.5e-8 apart, below fp32's spacing there, so codes collide in runs
        cols = rng.permutation(E)[:24]
        base = np.float32(2.0) if r % 2 == 0 else np.float32(-0.25)
        vals = [base]
        for _ in range(23):
            vals.append(np.nextafter(vals[-1], np.float32(np.inf), dtype=np.float32))
        vals = np.array(vals, dtype=np.float32)
        if r % 4 == 3:
            vals[::3] = vals[0]  # exactly equal keys too: lower id first
        lg[r, cols] = rng.permutation(vals)
    bias = np.zeros(E, dtype=np.float32)
    bias[rng.permutation(E)[:64]] = np.float32(2.0 ** -24)  # shifts a key by about one fp32 step
    cfg = m.make_route_cfg("grouped", E, 8, 8, 4, 2, True)
    # the 64 constructed rows, and the same rows tiled to 2049 with every 7th a pad row
    big = np.tile(lg, (33, 1))[:2049]
    rv_big = (np.arange(2049) % 7 != 3).astype(np.int32)
    for rows, rv in ((lg, None), (big, rv_big)):
        Gr = rows.shape[0]
        for b in (None, bias):
            ids = torch.empty((Gr, 8), dtype=torch.int32, device="cuda")
            w = torch.empty((Gr, 8), dtype=torch.float32, device="cuda")
            m.moe_route_from_logits(torch.from_numpy(rows).cuda(), None if rv is None else torch.from_numpy(rv).cuda(),
                                    None if b is None else torch.from_numpy(b).cuda(), cfg, ids, w)
            torch.cuda.synchronize()
            ref_ids, ref_w = oracle.select_grouped(rows, b, 8, 4, 8, True, row_valid=rv)
            assert np.array_equal(ids.cpu().numpy(), ref_ids), (Gr, b is None)
            assert oracle.rel_err(w.cpu().numpy(), ref_w) < 1e-6
    # softmax router: +0 and -0 logits are equal keys (lower id first), the rest below them
    lg = -rng.uniform(0.5, 1.0, (16, 64)).astype(np.float32)
    for r in range(16):
        cols = rng.permutation(64)[:10]
        lg[r, cols[:5]] = np.float32(0.0)
        lg[r, cols[5:]] = np.float32(-0.0)
    cfgs = m.make_route_cfg("softmax", 64, 6, renormalize=True)
    for rows in (lg, np.tile(lg, (131, 1))[:2095]):
        Gr = rows.shape[0]
        ids = torch.empty((Gr, 6), dtype=torch.int32, device="cuda")
        w = torch.empty((Gr, 6), dtype=torch.float32, device="cuda")
        m.moe_route_from_logits(torch.from_numpy(rows).cuda(), None, None, cfgs, ids, w)
        torch.cuda.synchronize()
        ref_ids, ref_w = oracle.select_softmax(rows, 6, True)
        assert np.array_equal(ids.cpu().numpy(), ref_ids), Gr
        assert oracle.rel_err(w.cpu().numpy(), ref_w) < 1e-5


@pytest.mark.parametrize("name,stride", [("cfg3", 384), ("cfg3", 8), ("cfg2", 170), ("cfg2", 5)])
def test_fixed_capacity_layout(name, stride):
    """The masked layout: slot e's rows at e * stride.  stride = G never overflows (decode:
    16 replicas x the static bound 24; the DP-gather workload: 170 rows); the small strides
    overflow, drop the late pairs and raise the flag, on both sides alike."""
    layer, ref = run_and_compare(moe_synth.CONFIGS[name], "sum", seg_stride=stride)
    flag = int(to_np(layer.plan.error_flag)[0])
    say(f"  fixed capacity {stride}: error_flag {flag}, counts {to_np(layer.plan.counts).tolist()[:8]}...")
    assert flag == (1 if stride < 20 else 0)


@pytest.mark.parametrize("tokens,align,stride", [((8192,), 1, 0), ((8200,), 1, 0), ((8200,), 128, 0),
                                                  ((8192,), 1, 64), ((8200,), 1, 64),
                                                  ((1024,), 1, 0), ((1025,), 1, 0), ((1024,), 128, 0),
                                                  ((1024,), 1, 8), ((700, 0, 324), 1, 0),
                                                  ((128,), 1, 0), ((129,), 1, 0), ((256,), 1, 0),
                                                  ((257,), 1, 0), ((512,), 1, 0), ((513,), 1, 0),
                                                  ((128,), 128, 0), ((100,), 1, 2), ((70, 0, 57), 1, 0),
                                                  ((512,), 128, 0), ((300,), 1, 2), ((200, 0, 57), 1, 0)])
def test_dispatch_fused_and_scan_layouts(tokens, align, stride):
    """The three ways dispatch derives the plan's layout: with 1024 local slots and top-8, 8192
    rows make 64 count blocks of 1024 pairs, a 65536-entry count table that the place blocks
    add up themselves; 8200 rows make 65 blocks and take the separate scan kernel.  Batches of
    up to 16384 pairs use blocks of 256 pairs (1024 or 1025 rows: 32 or 33 blocks, one case
    with an idle replica) and take the first way.  Up to 1024 pairs (128 rows) one place block
    takes every pair and counts them itself; 129 to 513 rows make 5 to 17 blocks of 256 pairs.
    All of them, with alignment 128 and with the fixed-capacity layout (64, 8 or 2 rows per
    slot, so slots overflow), give the oracle's plan bit for bit."""
    cfg = replace(moe_synth.CONFIGS["cfg2"], num_tokens=tokens, hidden=256, inter=128,
                  num_experts=1024, num_local=1024, top_k=8, name=f"dispatch-{tokens[0]}")
    run_and_compare_inputs(moe_synth.make_inputs(cfg), "sum", align=align, seg_stride=stride)
