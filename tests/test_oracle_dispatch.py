"""Pins of the oracle's dispatch plan (O3): Python's stable sort, the permutation /
inverse identity, count sums, alignment, capacity overflow and the rank-invariant
replica choice."""
import numpy as np
import pytest

import moe_synth
import oracle


def _random_ids(rng, G, k, E, pad_frac=0.1):
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(G)]).astype(np.int32)
    pad = rng.random(G) < pad_frac
    ids[pad] = -1
    return ids


@pytest.mark.parametrize("align", [1, 4, 128])
def test_dispatch_equals_stable_sort(align):
    rng = np.random.default_rng(21)
    G, k, E = 157, 6, 40
    p0, El = 8, 20
    phys = np.arange(E, dtype=np.int32).reshape(E, 1)
    nrep = np.ones(E, dtype=np.int32)
    ids = _random_ids(rng, G, k, E)
    plan = oracle.dispatch(ids, phys, nrep, p0, El, align)
    flat = ids.ravel()
    local = [f for f in range(G * k) if flat[f] >= 0 and p0 <= flat[f] < p0 + El]
    order = sorted(local, key=lambda f: flat[f] - p0)          # Python's sort is stable
    counts = np.bincount([flat[f] - p0 for f in local], minlength=El)
    assert np.array_equal(plan["counts"], counts)
    assert int(plan["counts"].sum()) == len(local)
    seg = plan["seg_offsets"]
    assert seg[0] == 0 and np.all(np.diff(seg) == (counts + align - 1) // align * align)
    assert plan["num_rows"] == seg[-1]
    rows = [plan["sorted_pair"][r] for e in range(El) for r in range(seg[e], seg[e] + counts[e])]
    assert rows == order
    for e in range(El):       # alignment pad rows
        assert np.all(plan["sorted_pair"][seg[e] + counts[e]:seg[e + 1]] == -1)
    # permutation composed with its inverse is the identity
    pr = plan["pair_row"]
    for f in local:
        assert plan["sorted_pair"][pr[f]] == f
    assert np.all(pr[[f for f in range(G * k) if f not in set(local)]] == -1)


def test_all_local_counts_sum_to_T_times_k():
    rng = np.random.default_rng(22)
    G, k, E = 300, 8, 16
    ids = _random_ids(rng, G, k, E, pad_frac=0.0)
    plan = oracle.dispatch(ids, np.arange(E, dtype=np.int32)[:, None], np.ones(E, np.int32), 0, E)
    assert int(plan["counts"].sum()) == G * k == plan["num_rows"]


def test_permute_rows():
    rng = np.random.default_rng(23)
    G, k, E, H = 50, 3, 10, 5
    ids = _random_ids(rng, G, k, E)
    x = rng.integers(0, 1000, (G, H)).astype(np.uint16)
    plan = oracle.dispatch(ids, np.arange(E, dtype=np.int32)[:, None], np.ones(E, np.int32), 0, E, 4)
    xp = oracle.permute_rows(x, plan)
    for r, f in enumerate(plan["sorted_pair"]):
        if f >= 0:
            assert np.array_equal(xp[r], x[f // k])
        else:
            assert np.all(xp[r] == 0)


def test_capacity_overflow_flag():
    G, k, E = 40, 2, 4
    ids = np.tile(np.array([[0, 1]], dtype=np.int32), (G, 1))
    plan = oracle.dispatch(ids, np.arange(E, dtype=np.int32)[:, None], np.ones(E, np.int32), 0, E,
                           cap=50)
    assert plan["error_flag"] == 1 and plan["num_rows"] == 80
    kept = plan["pair_row"] >= 0
    assert kept.sum() == 50
    # the first 40 rows are expert 0's pairs (f = 0, 2, 4, ...), then 10 pairs of expert 1
    assert list(plan["sorted_pair"][:3]) == [0, 2, 4]
    assert list(plan["sorted_pair"][40:43]) == [1, 3, 5]


def test_replica_round_robin_is_rank_invariant():
    cfg = moe_synth.CONFIGS["cfg5"]
    phys, nrep = moe_synth.expert_map(cfg)
    assert list(nrep[:4]) == [2, 2, 2, 2] and np.all(nrep[4:] == 1)
    G, k = 64, 8
    ids = np.zeros((G, k), dtype=np.int32) - 1
    ids[:, 0] = 0          # every token picks hot expert 0 in slot 0
    ids[:, 1] = 5          # and logical 5 (slot 9)
    plan = oracle.dispatch(ids, phys, nrep, 0, 16)
    # logical 0 lives in slots 0 and 1: token g goes to slot g % 2
    assert plan["counts"][0] == 32 and plan["counts"][1] == 32 and plan["counts"][9] == 64
    seg = plan["seg_offsets"]
    assert [f // k for f in plan["sorted_pair"][seg[0]:seg[1]]] == list(range(0, G, 2))
    assert [f // k for f in plan["sorted_pair"][seg[1]:seg[2]]] == list(range(1, G, 2))
    # a rank owning slots [16, 32) sees none of these pairs
    other = oracle.dispatch(ids, phys, nrep, 16, 16)
    assert other["num_rows"] == 0 and np.all(other["pair_row"] == -1)


def test_empty_and_all_pad():
    E = 8
    phys = np.arange(E, dtype=np.int32)[:, None]
    plan = oracle.dispatch(np.zeros((0, 2), np.int32), phys, np.ones(E, np.int32), 0, E)
    assert plan["num_rows"] == 0 and np.all(plan["counts"] == 0)
    plan = oracle.dispatch(np.full((5, 2), -1, np.int32), phys, np.ones(E, np.int32), 0, E, 128)
    assert plan["num_rows"] == 0 and np.all(plan["pair_row"] == -1)


# ------------------------------------------------------------------ fixed-capacity (masked) layout

def _random_case(seed, G=300, k=6, E=40, El=12, p0=5, max_rep=3):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(G)]).astype(np.int32)
    ids[::9] = -1
    n_rep = rng.integers(1, max_rep + 1, E).astype(np.int32)
    phys = np.full((E, max_rep), -1, np.int32)
    pool = rng.permutation(E * max_rep)
    c = 0
    for e in range(E):
        phys[e, :n_rep[e]] = pool[c:c + n_rep[e]]
        c += n_rep[e]
    return ids, phys, n_rep, p0, El


@pytest.mark.parametrize("seed", range(5))
def test_masked_layout_with_room_is_the_packed_plan_moved(seed):
    """With a stride no slot overflows, each slot's rows are the packed plan's rows of that
    slot (from the C counting sort), in the same order, starting at e * stride."""
    ids, phys, n_rep, p0, El = _random_case(seed)
    packed = oracle.dispatch(ids, phys, n_rep, p0, El)
    stride = int(packed["counts"].max()) + 3
    mk = oracle.dispatch_masked(ids, phys, n_rep, p0, El, stride)
    assert mk["error_flag"] == 0 and mk["num_rows"] == El * stride
    assert np.array_equal(mk["counts"], packed["counts"])
    assert np.array_equal(mk["seg_offsets"], np.arange(El + 1) * stride)
    for e in range(El):
        a, c = int(packed["seg_offsets"][e]), int(packed["counts"][e])
        assert np.array_equal(mk["sorted_pair"][e * stride:e * stride + c], packed["sorted_pair"][a:a + c])
        assert np.all(mk["sorted_pair"][e * stride + c:(e + 1) * stride] == -1)
    # pair_row inverts sorted_pair
    for f in np.nonzero(mk["pair_row"] >= 0)[0]:
        assert mk["sorted_pair"][mk["pair_row"][f]] == f
    assert np.array_equal(mk["pair_row"] >= 0, packed["pair_row"] >= 0)


@pytest.mark.parametrize("stride", [1, 4, 9])
def test_masked_layout_overflow_keeps_the_first_pairs(stride):
    """A slot over capacity keeps its stride lowest flat indices (brute force on the packed
    plan's per-slot lists) and raises the flag; everything else is dropped."""
    ids, phys, n_rep, p0, El = _random_case(11)
    packed = oracle.dispatch(ids, phys, n_rep, p0, El)
    mk = oracle.dispatch_masked(ids, phys, n_rep, p0, El, stride)
    assert mk["error_flag"] == int(packed["counts"].max() > stride)
    assert np.array_equal(mk["counts"], np.minimum(packed["counts"], stride))
    kept = set()
    for e in range(El):
        a, c = int(packed["seg_offsets"][e]), int(packed["counts"][e])
        lst = packed["sorted_pair"][a:a + c][:stride]
        kept |= set(lst.tolist())
        assert np.array_equal(mk["sorted_pair"][e * stride:e * stride + len(lst)], lst)
    assert set(np.nonzero(mk["pair_row"] >= 0)[0].tolist()) == kept
