"""C-ABI checks that need no GPU: the library loads, exports every declared entry point,
computes gather layouts like the oracle, and rejects bad arguments before touching HIP."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def m():
    import combine_dp_gather_amd as m
    if not os.path.exists(os.path.join(ROOT, "combine_dp_gather_amd", "libmoe_hip.so")):
        from combine_dp_gather_amd import build
        build.build()
    m.lib()
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(m):
    from combine_dp_gather_amd import _lib
    names = declared_functions()
    assert len(names) >= 14
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) <= set(_lib.SIGNATURES)
    assert m.moe_version().endswith("gfx950")


def test_layout_matches_oracle_golden(m):
    cases = json.load(open(os.path.join(ROOT, "tests", "golden", "gather_layouts.json")))["cases"]
    for c in cases:
        L = m.moe_gather_layout(c["num_tokens"], c["mode"], c["is_extend"], c["max_len_with_idle"],
                                c["static_bound"])
        assert m.layout_mode(L) == c["expect_mode"]
        assert L.rows == c["expect_G"]
        assert m.layout_offsets(L) == c["expect_offsets"]


def test_layout_matches_oracle_random(m):
    rng = np.random.default_rng(0)
    for _ in range(300):
        W = int(rng.integers(1, 40))
        n = [int(v) for v in rng.integers(0, 100, W) * (rng.random(W) > 0.2)]
        mode = ["auto", "max", "sum"][int(rng.integers(3))]
        ext = bool(rng.integers(2))
        idle = bool(rng.integers(2))
        B = int(rng.integers(0, 2)) * 100
        L = m.moe_gather_layout(n, mode, ext, idle, B)
        om, G, offs, sizes = oracle.gather_layout(n, mode, ext, idle, B)
        assert (m.layout_mode(L), L.rows, m.layout_offsets(L), m.layout_sizes(L)) == (om, G, offs, sizes)


def test_layout_rejects(m):
    from combine_dp_gather_amd import MoEError
    for bad in ([], [1, -2]):
        with pytest.raises(MoEError):
            m.moe_gather_layout(bad, "sum")
    with pytest.raises(MoEError):
        m.moe_gather_layout([30], "sum", static_bound=24)
    with pytest.raises(MoEError):
        m.moe_gather_layout([1] * 257, "sum")


def test_argument_errors_return_before_any_launch(m):
    from combine_dp_gather_amd import _lib
    lib = m.lib()
    L = m.moe_gather_layout([3, 4], "sum")
    # NULL replica array / bad dtype / bad H
    assert lib.moe_gather(None, None, 16, _lib.MOE_BF16, None, None, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_gather(ctypes.byref(L), None, 16, _lib.MOE_BF16, None, None, None) == _lib.MOE_ERR_INVALID_ARG
    arr = (ctypes.c_void_p * 2)(None, None)
    assert lib.moe_gather(ctypes.byref(L), ctypes.cast(arr, ctypes.c_void_p), 0, _lib.MOE_BF16,
                          None, None, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_gather(ctypes.byref(L), ctypes.cast(arr, ctypes.c_void_p), 16, 7, None, None,
                          None) == _lib.MOE_ERR_INVALID_ARG
    # all replicas idle: a no-op that succeeds without any pointer
    L0 = m.moe_gather_layout([0, 0], "max")
    assert lib.moe_gather(ctypes.byref(L0), ctypes.cast(arr, ctypes.c_void_p), 16, _lib.MOE_BF16,
                          None, None, None) == _lib.MOE_OK
    # routing configuration checks
    bad = [m.make_route_cfg("softmax", 0, 1), m.make_route_cfg("softmax", 8, 9), m.make_route_cfg("softmax", 64, 33),
           m.make_route_cfg("grouped", 1024, 8, 128, 4), m.make_route_cfg("grouped", 1024, 8, 64, 8, 5),
           m.make_route_cfg("softmax", 2048, 2), m.make_route_cfg("grouped", 256, 8, 7, 4),
           m.make_route_cfg("grouped", 256, 8, 8, 9), m.make_route_cfg("grouped", 256, 8, 8, 4, 40),
           m.make_route_cfg("grouped", 16, 8, 4, 1)]
    for c in bad:
        assert lib.moe_route_from_logits(1, None, 4, None, ctypes.byref(c), 1, 1, None) == \
            _lib.MOE_ERR_INVALID_ARG
    badmode = m.make_route_cfg("grouped", 256, 8, 8, 4, 2, True)
    badmode.gate_mode = 2
    assert lib.moe_route_from_logits(1, None, 4, None, ctypes.byref(badmode), 1, 1, None) == \
        _lib.MOE_ERR_INVALID_ARG
    # the fast gate takes bf16 inputs only; rejected before any launch
    fast = m.make_route_cfg("grouped", 256, 8, 8, 4, 2, True, gate="fast")
    assert lib.moe_route(1, None, 4, 256, _lib.MOE_F32, 1, None, ctypes.byref(fast), 1, 1, 1,
                         None) == _lib.MOE_ERR_UNSUPPORTED
    good = m.make_route_cfg("grouped", 256, 8, 8, 4, 2, True)
    assert lib.moe_route_from_logits(1, None, 0, None, ctypes.byref(good), None, None, None) == _lib.MOE_OK
    # dispatch: plan / map mismatch, workspace too small
    emap = _lib.ExpertMap(16, 1, None, None, 0, 16)
    plan = _lib.Plan(1, 1, 1, 1, 1, 1, 100, 10, 2, 16, 1, 0)
    assert lib.moe_dispatch(1, 1, 10, 3, 64, _lib.MOE_BF16, ctypes.byref(emap), ctypes.byref(plan),
                            1, 1, 1 << 20, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch(1, 1, 10, 2, 64, _lib.MOE_BF16, ctypes.byref(emap), ctypes.byref(plan),
                            1, 1, 0, None) == _lib.MOE_ERR_CAPACITY
    # experts: fp8 weights need bf16 activations and both scale tables; a misaligned
    # workspace is rejected; dtype mismatch is invalid
    w = _lib.ExpertWeights(_lib.MOE_FP8_E4M3, 0, 1, 1, 1, 1)
    assert lib.moe_expert_gemm(1, _lib.MOE_F32, ctypes.byref(plan), ctypes.byref(w), 256, 128, 1, 1,
                               1 << 30, None) == _lib.MOE_ERR_UNSUPPORTED
    assert lib.moe_expert_gemm(1, _lib.MOE_BF16, ctypes.byref(plan), ctypes.byref(w), 256, 128, 1, 1,
                               1 << 30, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_gemm(1, _lib.MOE_BF16, ctypes.byref(plan), ctypes.byref(w), 256, 128, 1, 256,
                               16, None) == _lib.MOE_ERR_CAPACITY
    w_noscale = _lib.ExpertWeights(_lib.MOE_FP8_E4M3, 0, 1, 1, None, None)
    assert lib.moe_expert_gemm(1, _lib.MOE_BF16, ctypes.byref(plan), ctypes.byref(w_noscale), 256, 128,
                               1, 256, 1 << 30, None) == _lib.MOE_ERR_INVALID_ARG
    w_badmode = _lib.ExpertWeights(_lib.MOE_FP8_E4M3, 2, 1, 1, 1, 1)
    assert lib.moe_expert_gemm(1, _lib.MOE_BF16, ctypes.byref(plan), ctypes.byref(w_badmode), 256, 128, 1,
                               256, 1 << 30, None) == _lib.MOE_ERR_INVALID_ARG
    w = _lib.ExpertWeights(_lib.MOE_F32, 0, 1, 1, None, None)
    assert lib.moe_expert_gemm(1, _lib.MOE_BF16, ctypes.byref(plan), ctypes.byref(w), 256, 128, 1, 1,
                               1 << 30, None) == _lib.MOE_ERR_INVALID_ARG
    # the gathering up GEMM reads sorted_pair, top_k and G: a plan without sorted_pair, a
    # zero top_k or a missing global buffer are rejected; with no global rows it is a no-op
    w = _lib.ExpertWeights(_lib.MOE_BF16, 0, 1, 1, None, None)
    nosp = _lib.Plan(1, 1, None, 1, 1, 1, 100, 10, 2, 16, 1, 0)
    assert lib.moe_expert_gemm_up_gather(1, _lib.MOE_BF16, ctypes.byref(nosp), ctypes.byref(w), 256, 128, 1,
                                         None, 0, None) == _lib.MOE_ERR_INVALID_ARG
    k0 = _lib.Plan(1, 1, 1, 1, 1, 1, 100, 10, 0, 16, 1, 0)
    assert lib.moe_expert_gemm_up_gather(1, _lib.MOE_BF16, ctypes.byref(k0), ctypes.byref(w), 256, 128, 1,
                                         None, 0, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_gemm_up_gather(None, _lib.MOE_BF16, ctypes.byref(plan), ctypes.byref(w), 256, 128,
                                         1, None, 0, None) == _lib.MOE_ERR_INVALID_ARG
    g0 = _lib.Plan(1, 1, 1, 1, 1, 1, 100, 0, 2, 16, 1, 0)
    assert lib.moe_expert_gemm_up_gather(None, _lib.MOE_BF16, ctypes.byref(g0), ctypes.byref(w), 256, 128,
                                         1, None, 0, None) == _lib.MOE_OK
    # combine: bad dtype
    assert lib.moe_combine(1, 9, ctypes.byref(plan), 1, 1.0, 64, 1, None) == _lib.MOE_ERR_INVALID_ARG
    # fused exit: bad dtype; layout rows that do not match the plan; an unaligned replica
    # buffer is refused before anything is enqueued
    L = m.moe_gather_layout([3, 5], "sum")
    ptrs = (ctypes.c_void_p * 2)(256, 512)
    assert lib.moe_combine_scatter(1, 9, ctypes.byref(plan), 1, 1.0, 64, ctypes.byref(L), ptrs,
                                   None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_combine_scatter(1, _lib.MOE_BF16, ctypes.byref(plan), 1, 1.0, 64, ctypes.byref(L),
                                   ptrs, None) == _lib.MOE_ERR_INVALID_ARG
    plan8 = _lib.Plan(1, 1, 1, 1, 1, 1, 16, 8, 2, 4, 1, 0)
    bad = (ctypes.c_void_p * 2)(256, 520)
    assert lib.moe_combine_scatter(256, _lib.MOE_BF16, ctypes.byref(plan8), 256, 1.0, 64, ctypes.byref(L),
                                   bad, None) == _lib.MOE_ERR_UNSUPPORTED
    assert lib.moe_combine_scatter(256, _lib.MOE_BF16, ctypes.byref(plan8), 256, 1.0, 64, None, ptrs,
                                   None) == _lib.MOE_ERR_INVALID_ARG


def test_grid_limits_rejected_before_any_launch(m):
    """A launch's x dimension counts work-items in 32 bits.  Sizes whose grid would need 2^32
    or more are refused as unsupported before anything is enqueued (the pointers here are never
    dereferenced)."""
    from combine_dp_gather_amd import _lib
    lib = m.lib()
    c = m.make_route_cfg("grouped", 256, 8, 8, 4, 2, True)
    # the select runs one 64-lane wave per row: G = 2^26 rows is 2^32 work-items
    assert lib.moe_route_from_logits(256, None, 1 << 26, None, ctypes.byref(c), 256, 256, None) == \
        _lib.MOE_ERR_UNSUPPORTED
    assert lib.moe_route(256, None, 1 << 26, 64, _lib.MOE_BF16, 256, None, ctypes.byref(c), 256, 256, 256,
                         None) == _lib.MOE_ERR_UNSUPPORTED
    # combine, 16-byte path: one 256-thread block per row, so G = 2^24 rows is the first refused
    big = _lib.Plan(1, 1, 1, 1, 1, 1, 16, 1 << 24, 2, 4, 1, 0)
    assert lib.moe_combine(256, _lib.MOE_BF16, ctypes.byref(big), 256, 1.0, 64, 256, None) == \
        _lib.MOE_ERR_UNSUPPORTED
    # gather: 2^24 rows of 16 KB in 8 KB chunks, one per 256-thread block: 2^33 work-items
    L = m.moe_gather_layout([1 << 24], "sum")
    arr = (ctypes.c_void_p * 1)(256)
    assert lib.moe_gather(ctypes.byref(L), ctypes.cast(arr, ctypes.c_void_p), 8192, _lib.MOE_BF16, 256, 256,
                          None) == _lib.MOE_ERR_UNSUPPORTED


def test_workspace_sizes(m):
    assert m.moe_dispatch_workspace_size(0, 8, 16) >= 0
    a = m.moe_dispatch_workspace_size(32768, 8, 16)
    assert a >= 2 * (32768 * 8 // 1024) * 16 * 4
    import torch
    assert m.moe_expert_gemm_workspace_size(1000, 7168, 2048, torch.bfloat16, torch.bfloat16) >= 1000 * 2048 * 2


def test_status_strings(m):
    lib = m.lib()
    assert lib.moe_status_string(0) == b"ok"
    assert b"invalid" in lib.moe_status_string(1)


def test_entry_gather_argument_errors(m):
    """Fused entry step: NULL norm weight or residual of a non-idle replica, bad eps, bad H or
    dtype are rejected before any launch; an all-idle layout is a no-op."""
    from combine_dp_gather_amd import _lib
    lib = m.lib()
    L = m.moe_gather_layout([3, 4], "sum")
    fake = ctypes.c_void_p(4096)  # never dereferenced: every case fails its host checks first
    hs = (ctypes.c_void_p * 2)(fake, fake)
    none2 = (ctypes.c_void_p * 2)(None, None)

    def call(layout, h, r, w, eps, H=16, dt=_lib.MOE_BF16, gx=fake, rv=fake):
        return lib.moe_entry_gather(layout, ctypes.cast(h, ctypes.c_void_p) if h is not None else None,
                                    ctypes.cast(r, ctypes.c_void_p) if r is not None else None, w, eps, H,
                                    dt, gx, rv, None)

    E = _lib.MOE_ERR_INVALID_ARG
    assert call(None, hs, hs, fake, 1e-6) == E
    assert call(ctypes.byref(L), None, hs, fake, 1e-6) == E
    assert call(ctypes.byref(L), hs, None, fake, 1e-6) == E
    assert call(ctypes.byref(L), hs, none2, fake, 1e-6) == E        # residual of a real replica
    assert call(ctypes.byref(L), none2, hs, fake, 1e-6) == E        # input of a real replica
    assert call(ctypes.byref(L), hs, hs, None, 1e-6) == E           # norm weight
    assert call(ctypes.byref(L), hs, hs, fake, -1.0) == E
    assert call(ctypes.byref(L), hs, hs, fake, float("nan")) == E
    assert call(ctypes.byref(L), hs, hs, fake, float("inf")) == E
    assert call(ctypes.byref(L), hs, hs, fake, 1e-6, H=0) == E
    assert call(ctypes.byref(L), hs, hs, fake, 1e-6, dt=_lib.MOE_FP8_E4M3) == E
    assert call(ctypes.byref(L), hs, hs, fake, 1e-6, gx=None) == E
    assert call(ctypes.byref(L), hs, hs, fake, 1e-6, rv=None) == E
    L0 = m.moe_gather_layout([0, 0], "max")
    assert call(ctypes.byref(L0), none2, none2, None, 1e-6, gx=None, rv=None) == _lib.MOE_OK


def test_fixed_capacity_plan_errors(m):
    """A fixed-capacity plan needs cap >= E_l * seg_stride and a non-negative stride."""
    from combine_dp_gather_amd import _lib
    lib = m.lib()
    fake = 4096
    emap = m.make_expert_map(16, 0, 4)
    ws = (ctypes.c_uint8 * 64)()
    for stride, cap in [(-1, 100), (8, 31), (1 << 30, 1 << 40)]:
        plan = _lib.Plan(fake, fake, fake, fake, fake, fake, cap, 3, 2, 4, 1, stride)
        assert lib.moe_dispatch(fake, fake, 3, 2, 16, _lib.MOE_BF16, ctypes.byref(emap), ctypes.byref(plan),
                                fake, ws, 64, None) == _lib.MOE_ERR_INVALID_ARG


def test_cu_masked_stream_rejects_bad_masks(m):
    """The stream helpers check their arguments before any HIP call."""
    from combine_dp_gather_amd import _lib
    lib = m.lib()
    out = ctypes.c_void_p()
    empty = (ctypes.c_uint32 * 8)()
    assert lib.moe_stream_create_cu_masked(empty, 8, ctypes.byref(out)) == _lib.MOE_ERR_INVALID_ARG
    one = (ctypes.c_uint32 * 1)(1)
    assert lib.moe_stream_create_cu_masked(one, 0, ctypes.byref(out)) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_stream_create_cu_masked(one, 33, ctypes.byref(out)) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_stream_create_cu_masked(None, 1, ctypes.byref(out)) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_stream_create_cu_masked(one, 1, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_stream_destroy(None) == _lib.MOE_ERR_INVALID_ARG
