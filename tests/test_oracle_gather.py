"""Pins of the oracle's gather / scatter step (O1, O6) against the pages' own sizes,
closed forms and brute force."""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "gather_layouts.json")


@pytest.mark.parametrize("case", json.load(open(GOLD))["cases"], ids=lambda c: c["source"][:40])
def test_layout_golden(case):
    mode, G, offs, sizes = oracle.gather_layout(case["num_tokens"], case["mode"], case["is_extend"],
                                                case["max_len_with_idle"], case["static_bound"])
    assert mode == case["expect_mode"]
    assert G == case["expect_G"]
    assert offs == case["expect_offsets"]


def test_layout_closed_forms():
    rng = np.random.default_rng(5)
    for _ in range(200):
        W = int(rng.integers(1, 20))
        n = [int(v) for v in rng.integers(0, 50, W)]
        _, G, offs, _ = oracle.gather_layout(n, "sum")
        assert offs == [int(v) for v in np.concatenate([[0], np.cumsum(n)])]
        assert G == sum(n)
        _, G, offs, _ = oracle.gather_layout(n, "max")
        if sum(n):
            assert offs == [i * max(n) for i in range(W + 1)] and G == W * max(n)
        else:
            assert G == 0
        # decode cost rule
        m, *_ = oracle.gather_layout(n, "auto")
        if sum(n):
            assert m == ("max" if 2 * sum(n) >= max(n) * W else "sum")


def test_layout_rejects_bad():
    with pytest.raises(ValueError):
        oracle.gather_layout([3, -1], "sum")
    with pytest.raises(ValueError):
        oracle.gather_layout([25, 1], "sum", static_bound=24)
    with pytest.raises(ValueError):
        oracle.gather_layout([], "sum")


def _brute_gather(n, xs, H, mode):
    # row-by-row walk: replica i's rows follow the rows of replicas 0..i-1, each replica
    # occupying n_i rows (sum) or max(n) rows (max)
    rows, valid = [], []
    width = max(n) if mode == "max" else None
    for i, x in enumerate(xs):
        span = width if mode == "max" else n[i]
        for r in range(span):
            if r < n[i]:
                rows.append(x[r])
                valid.append(1)
            else:
                rows.append(np.zeros(H, dtype=x.dtype))
                valid.append(0)
    if not rows:
        return np.zeros((0, H), dtype=xs[0].dtype), np.zeros(0, dtype=np.int32)
    return np.stack(rows), np.array(valid, dtype=np.int32)


@pytest.mark.parametrize("mode", ["max", "sum"])
def test_gather_bruteforce_and_roundtrip(mode):
    rng = np.random.default_rng(7)
    for trial in range(30):
        W = int(rng.integers(1, 7))
        n = [int(v) for v in rng.integers(0, 9, W)]
        H = int(rng.integers(1, 6))
        xs = [rng.integers(0, 65535, (ni, H)).astype(np.uint16) for ni in n]
        lay = oracle.gather_layout(n, mode)
        if lay[1] == 0:
            assert sum(n) == 0
            continue
        g, v = oracle.gather(lay, xs, H, np.uint16)
        bg, bv = _brute_gather(n, xs, H, mode)
        assert np.array_equal(g, bg) and np.array_equal(v, bv)
        # idle replicas contribute zero valid rows; the valid count is sum(n)
        assert int(v.sum()) == sum(n)
        back = oracle.scatter(lay, g)
        for i in range(W):
            assert np.array_equal(back[i], xs[i])


def test_max_and_sum_agree_per_replica():
    rng = np.random.default_rng(11)
    n = [37, 0, 128, 5]
    xs = [rng.standard_normal((ni, 4)).astype(np.float32) for ni in n]
    outs = {}
    for mode in ("max", "sum"):
        lay = oracle.gather_layout(n, mode)
        g, _ = oracle.gather(lay, xs, 4, np.float32)
        outs[mode] = oracle.scatter(lay, g * 3.0)
    for a, b in zip(outs["max"], outs["sum"]):
        assert np.array_equal(a, b)
