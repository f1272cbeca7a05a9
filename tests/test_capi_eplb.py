"""EPLB host calls of the C ABI against the oracle, on the CPU: the library's placement,
balancedness and dispatch table must equal the oracle's exactly (integer loads make every
floating-point comparison in the placement independent of summation order), and bad
arguments are rejected before anything runs."""
import ctypes

import numpy as np
import pytest

import oracle


@pytest.fixture(scope="module")
def m():
    import combine_dp_gather_amd as m
    m.lib()
    return m


SHAPES = [(16, 20, 4, 2, 4), (256, 288, 8, 2, 18), (256, 288, 8, 1, 16), (256, 256, 8, 4, 16),
          (64, 64, 8, 4, 8), (12, 18, 3, 3, 6), (8, 8, 1, 1, 1), (256, 320, 8, 8, 32)]


def _loads(kind, L, E, rng):
    if kind == "zipf":
        return np.floor(1e6 / (rng.permutation(E) + 1.0) ** 1.2)[None, :].repeat(L, 0)
    if kind == "pareto":
        return np.floor(rng.pareto(1.1, (L, E)) * 1000)
    if kind == "equal":
        return np.full((L, E), 37.0)
    if kind == "zeros":
        return np.zeros((L, E))
    return rng.integers(0, 5, (L, E)).astype(np.float64)   # many ties


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("kind", ["zipf", "pareto", "equal", "zeros", "ties"])
def test_rebalance_equals_oracle(m, shape, kind):
    E, P, groups, nodes, gpus = shape
    rng = np.random.default_rng(E * 7 + P)
    w = _loads(kind, 2, E, rng)
    got = m.moe_eplb_rebalance(w, P, groups, nodes, gpus)
    want = oracle.rebalance_hierarchical(w, P, groups, nodes, gpus)
    for g, x in zip(got, want):
        assert np.array_equal(g, x)
    for l in range(2):
        mr = int(got[2][l].max())
        po, nr = m.moe_eplb_logical_to_physical(got[0][l], got[1][l], E, mr + 1)
        po_o, nr_o = oracle.logical_to_physical(got[0][l], got[1][l], E, mr + 1)
        assert np.array_equal(po, po_o) and np.array_equal(nr, nr_o)


def test_balancedness_equals_oracle(m):
    rng = np.random.default_rng(4)
    for gpus, P in [(18, 288), (16, 256), (1, 7), (4, 4)]:
        pc = rng.integers(0, 10000, (3, P)).astype(np.int64)
        got = m.moe_eplb_balancedness(pc, gpus)
        want = oracle.utilization_rate(oracle.gpu_counts(pc, gpus))
        assert np.array_equal(got, want)
    assert m.moe_eplb_balancedness(np.zeros((1, 8), np.int64), 4)[0] == 1.0


def test_eplb_host_argument_errors(m):
    from combine_dp_gather_amd import _lib
    lib = m.lib()
    E = _lib.MOE_ERR_INVALID_ARG
    w = np.ones((1, 16))
    for args in [(16, 4, 3, 4), (16, 3, 1, 4), (20, 4, 2, 3), (18, 4, 2, 4), (14, 4, 2, 2)]:
        with pytest.raises(_lib.MoEError):
            m.moe_eplb_rebalance(w, *args)
    for bad in (np.full((1, 16), -1.0), np.full((1, 16), np.nan), np.full((1, 16), np.inf)):
        with pytest.raises(_lib.MoEError):
            m.moe_eplb_rebalance(bad, 16, 4, 2, 4)
    # dispatch table: too few columns, bad entries, repeated or missing replicas
    p2l, rk, cnt = m.moe_eplb_rebalance(np.array([[100.0, 1, 1, 1]]), 6, 1, 1, 2)
    mr = int(cnt.max())
    assert lib.moe_eplb_logical_to_physical(p2l[0].ctypes.data_as(ctypes.c_void_p), rk[0].ctypes.data_as(ctypes.c_void_p),
                                            6, 4, mr - 1, np.empty((4, mr), np.int32).ctypes.data_as(ctypes.c_void_p),
                                            np.empty(4, np.int32).ctypes.data_as(ctypes.c_void_p)) == _lib.MOE_ERR_CAPACITY
    for a, r in [([0, 1, 2, 5], [0, 0, 0, 0]), ([0, 1, 2, 2], [0, 0, 0, 0]), ([0, 1, 2, 2], [0, 0, 0, 2]),
                 ([0, 1, 1, 1], [0, 0, 1, 2])]:
        with pytest.raises(_lib.MoEError):
            m.moe_eplb_logical_to_physical(np.array(a), np.array(r), 4, 4)
    # device calls reject before any launch
    assert lib.moe_expert_load(None, 4, 2, None, 16, None, None) == E
    emap = m.make_expert_map(4, 0, 4)
    assert lib.moe_expert_load(None, 4, 0, ctypes.byref(emap), 16, None, None) == E
    assert lib.moe_expert_load(None, 4, 2, ctypes.byref(emap), 0, None, None) == E
    assert lib.moe_expert_load(None, 4, 2, ctypes.byref(emap), 8193, None, None) == E
    assert lib.moe_physical_to_logical_count(None, None, 1, 8, 4097, None, None) == E
    assert lib.moe_physical_to_logical_count(None, None, 1, 8, 4, None, None) == E
    assert lib.moe_physical_to_logical_count(None, None, 0, 8, 4, None, None) == _lib.MOE_OK
