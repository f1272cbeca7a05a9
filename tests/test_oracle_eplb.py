"""Pins of the oracle's EPLB statistics and placement against brute force, library routines,
closed forms and the invariants the placement must keep."""
import itertools

import numpy as np
import pytest

import oracle


# ------------------------------------------------------------------ counts

def test_physical_counts_brute_force_and_bincount():
    rng = np.random.default_rng(0)
    E, G, k, P = 12, 50, 3, 17
    ids = rng.integers(-1, E, (G, k)).astype(np.int32)          # -1: pad rows / unused picks
    n_rep = rng.integers(1, 4, E).astype(np.int32)
    phys_of = np.full((E, 3), -1, dtype=np.int32)
    for e in range(E):
        phys_of[e, :n_rep[e]] = rng.choice(P + 2, n_rep[e], replace=False)  # some slots >= P
    got = oracle.physical_counts(ids, phys_of, n_rep, P)
    want = np.zeros(P, dtype=np.int64)
    for g in range(G):
        for j in range(k):
            e = int(ids[g, j])
            if 0 <= e < E:
                p = int(phys_of[e, g % n_rep[e]])
                if 0 <= p < P:
                    want[p] += 1
    assert np.array_equal(got, want)
    # trivial map: the histogram of the ids
    triv = oracle.physical_counts(ids, np.arange(E, dtype=np.int32)[:, None], np.ones(E, np.int32), E)
    v = ids[ids >= 0]
    assert np.array_equal(triv, np.bincount(v, minlength=E))


def test_physical_to_logical_is_weighted_bincount():
    rng = np.random.default_rng(1)
    L, P, E = 3, 40, 29
    phy2log = rng.integers(0, E, (L, P)).astype(np.int32)
    pc = rng.integers(0, 1000, (L, P)).astype(np.int64)
    got = oracle.physical_to_logical_count(pc, phy2log, E)
    for l in range(L):
        assert np.array_equal(got[l], np.bincount(phy2log[l], weights=pc[l], minlength=E).astype(np.int64))
    assert np.array_equal(got.sum(axis=1), pc.sum(axis=1))


def test_utilization_rate_closed_forms():
    assert oracle.utilization_rate(np.array([7, 7, 7, 7]))[()] == pytest.approx(1.0, abs=0)
    c = 1000.0
    assert oracle.utilization_rate(np.array([c, 0, 0, 0])) == pytest.approx((c / 4 + 1e-5) / (c + 1e-5), rel=1e-15)
    assert oracle.utilization_rate(np.zeros(5)) == pytest.approx(1.0)
    x = np.array([[1, 2, 3], [4, 4, 4]])
    assert np.allclose(oracle.utilization_rate(x), [(2 + 1e-5) / (3 + 1e-5), 1.0], rtol=1e-15)
    # per-GPU sums are contiguous slot blocks
    assert np.array_equal(oracle.gpu_counts(np.arange(12), 3), [0 + 1 + 2 + 3, 4 + 5 + 6 + 7, 8 + 9 + 10 + 11])


# ------------------------------------------------------------------ replication

@pytest.mark.parametrize("seed", range(30))
def test_replicate_minimises_the_largest_per_replica_load(seed):
    """Against every way of giving num_phy slots to n experts (each at least one)."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 5))
    num_phy = n + int(rng.integers(0, 5))
    w = [float(v) for v in rng.integers(0, 50, n)]
    phy2log, rank, cnt = oracle.replicate_experts(w, num_phy)
    best = min(max(w[i] / c[i] for i in range(n))
               for c in itertools.product(range(1, num_phy + 1), repeat=n) if sum(c) == num_phy)
    assert max(w[i] / cnt[i] for i in range(n)) == best
    # structure: one slot per expert first, replica ranks 0..cnt-1, counts add up
    assert phy2log[:n] == list(range(n)) and rank[:n] == [0] * n
    assert sum(cnt) == num_phy
    for e in range(n):
        assert sorted(r for p, r in zip(phy2log, rank) if p == e) == list(range(cnt[e]))


# ------------------------------------------------------------------ packing

def _check_packing(w, m, pack, rank):
    n = len(w)
    per = n // m
    for q in range(m):
        members = [i for i in range(n) if pack[i] == q]
        assert len(members) == per
        assert sorted(rank[i] for i in members) == list(range(per))


def test_packing_one_pack_is_the_stable_descending_order():
    w = [3.0, 9.0, 3.0, 1.0, 9.0, 0.0]
    pack, rank = oracle.balanced_packing(w, 1)
    assert pack == [0] * 6
    order = np.argsort(-np.array(w), kind="stable")
    assert [rank[i] for i in order] == list(range(6))


def test_packing_one_item_per_pack_goes_heaviest_first():
    w = [3.0, 9.0, 3.0, 1.0, 9.0, 0.0]
    pack, rank = oracle.balanced_packing(w, 6)
    order = np.argsort(-np.array(w), kind="stable")
    assert [pack[i] for i in order] == list(range(6)) and rank == [0] * 6


def test_packing_equal_weights_round_robin():
    pack, rank = oracle.balanced_packing([2.0] * 12, 4)
    assert pack == [i % 4 for i in range(12)] and rank == [i // 4 for i in range(12)]


def test_packing_two_by_two_closed_form():
    """a >= b >= c >= d into two packs of two: a alone first, b to the other, c to b's pack
    (b < a or, on a tie, the lower index), d to a's pack: loads {a + d, b + c}."""
    rng = np.random.default_rng(5)
    for _ in range(50):
        a, b, c, d = sorted(rng.integers(1, 100, 4).astype(float), reverse=True)
        if a == b:
            continue
        perm = rng.permutation(4)
        w = [0.0] * 4
        for v, i in zip((a, b, c, d), perm):
            w[i] = v
        pack, rank = oracle.balanced_packing(w, 2)
        _check_packing(w, 2, pack, rank)
        loads = sorted(sum(w[i] for i in range(4) if pack[i] == q) for q in range(2))
        assert loads == sorted([a + d, b + c])


@pytest.mark.parametrize("seed", range(10))
def test_packing_invariants(seed):
    rng = np.random.default_rng(seed)
    m = int(rng.integers(1, 6))
    n = m * int(rng.integers(1, 7))
    w = [float(v) for v in rng.integers(0, 30, n)]
    pack, rank = oracle.balanced_packing(w, m)
    _check_packing(w, m, pack, rank)


# ------------------------------------------------------------------ the hierarchy

def _check_placement(w, P, groups, nodes, gpus, phy2log, phy_rank, log_count):
    L, E = w.shape
    p_node, e_node, gs = P // nodes, E // nodes, E // groups
    for l in range(L):
        c = np.bincount(phy2log[l], minlength=E)
        assert np.array_equal(c, log_count[l]) and c.min() >= 1 and c.sum() == P
        for e in range(E):
            slots = np.nonzero(phy2log[l] == e)[0]
            assert sorted(phy_rank[l, slots].tolist()) == list(range(len(slots)))
            assert len(set(slots // p_node)) == 1            # replicas stay on one node
        node_of = {}
        for p in range(P):
            node_of.setdefault(int(phy2log[l, p]), p // p_node)
        for q in range(groups):                               # whole groups per node
            assert len({node_of[e] for e in range(q * gs, (q + 1) * gs)}) == 1
        for nd in range(nodes):                               # a node holds e_node experts
            assert len(set(phy2log[l, nd * p_node:(nd + 1) * p_node].tolist())) == e_node


@pytest.mark.parametrize("shape", [(16, 20, 4, 2, 4), (256, 288, 8, 2, 18), (256, 288, 8, 1, 16),
                                   (64, 64, 8, 4, 8), (12, 18, 3, 3, 6)])
def test_rebalance_invariants(shape):
    E, P, groups, nodes, gpus = shape
    rng = np.random.default_rng(E + P)
    w = np.floor(rng.pareto(1.2, (2, E)) * 100)
    phy2log, phy_rank, log_count = oracle.rebalance_hierarchical(w, P, groups, nodes, gpus)
    _check_placement(w, P, groups, nodes, gpus, phy2log, phy_rank, log_count)
    phys_of, n_rep = oracle.logical_to_physical(phy2log[0], phy_rank[0], E, int(log_count.max()))
    assert np.array_equal(n_rep, log_count[0])
    for p in range(P):
        assert phys_of[phy2log[0, p], phy_rank[0, p]] == p


def test_rebalance_single_node_reduces_to_replicate_then_pack():
    """One node and one group: the hierarchy is replication of all experts followed by
    packing the per-replica shares onto the GPUs."""
    rng = np.random.default_rng(3)
    E, P, gpus = 10, 15, 5
    w = np.floor(rng.pareto(1.0, (1, E)) * 50)
    phy2log, phy_rank, log_count = oracle.rebalance_hierarchical(w, P, 1, 1, gpus)
    s2l, srank, cnt = oracle.replicate_experts(list(w[0]), P)
    share = [w[0][s2l[i]] / cnt[s2l[i]] for i in range(P)]
    gpu, pos = oracle.balanced_packing(share, gpus)
    for i in range(P):
        slot = gpu[i] * (P // gpus) + pos[i]
        assert phy2log[0, slot] == s2l[i] and phy_rank[0, slot] == srank[i]
    assert log_count[0].tolist() == cnt


def test_rebalance_improves_skewed_balance():
    """Zipf-like loads on 256 experts, 18 GPUs x 16 slots: the placement's per-GPU load
    (replicas sharing their expert's load) is far better balanced than the trivial one
    (expert e on slot e, the 32 extra slots idle)."""
    E, P, gpus = 256, 288, 18
    w = np.floor(1e6 / (np.arange(E) + 1.0) ** 1.2)[None, :]
    phy2log, phy_rank, log_count = oracle.rebalance_hierarchical(w, P, 8, 2, gpus)
    share = w[0][phy2log[0]] / log_count[0][phy2log[0]]
    after = oracle.utilization_rate(oracle.gpu_counts(share, gpus))
    trivial = np.zeros(P)
    trivial[:E] = w[0]
    before = oracle.utilization_rate(oracle.gpu_counts(trivial, gpus))
    assert before < 0.1 and after > 0.5
