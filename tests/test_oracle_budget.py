"""Pins of the tree-budget oracle."""
import numpy as np
import pytest

import workloads
from oracle import budget as BU
from oracle import tree as T


def test_hand_computed_four_node_case():
    """One head with exact-rank hits 0.5, 0.3, 0.1: greedy admits them in that order, so
    E[A] = 0, 0.5, 0.8, 0.9 for 1..4 rows.  With a per-layer cost of N us (one layer):
    fixed 10 -> rates 1/11, 1.5/12, 1.8/13, 1.9/14, best N = 3; fixed 0 -> 1, .75, .6,
    .475, best N = 1 (the root alone)."""
    a = [[0.5, 0.3, 0.1]]
    r = BU.tree_budget(a, [1, 4], [1.0, 4.0], 10.0, 1)
    assert [round(r["table"][n][0], 12) for n in (1, 2, 3, 4)] == [1.0, 1.5, 1.8, 1.9]
    assert r["best_n"] == 3
    assert abs(r["table"][3][1] - 1.8 / 13) < 1e-15
    assert BU.tree_budget(a, [1, 4], [1.0, 4.0], 0.0, 1)["best_n"] == 1


def test_flat_cost_takes_the_largest_tree():
    """When a round costs the same at every size, more rows only add expected tokens."""
    a = workloads.rank_hit_table(4, 10)
    r = BU.tree_budget(a, [8, 40], [50.0, 50.0], 1000.0, 32)
    assert r["best_n"] == 40


def test_interpolation_between_measured_counts():
    nodes, us = [16, 32, 64], [10.0, 12.0, 20.0]
    assert BU.cost(nodes, us, 16) == 10.0 and BU.cost(nodes, us, 64) == 20.0
    assert BU.cost(nodes, us, 24) == 11.0 and BU.cost(nodes, us, 48) == 16.0


def test_expected_accept_is_the_greedy_prefix_sum():
    """E[A] of T_N equals the sum of the first N - 1 greedy admissions' weights."""
    a = workloads.rank_hit_table(4, 10)
    picks = T.greedy_frontier(np.asarray(a), 63)
    w = [float(np.prod([a[d][r] for d, r in enumerate(p)])) for p in picks]
    for n in (2, 10, 33, 64):
        assert abs(BU.expected_accept(a, n) - sum(w[: n - 1])) < 1e-12


@pytest.mark.parametrize("seed", range(6))
def test_best_count_never_grows_with_the_per_node_cost(seed):
    """With cost base + slope * N, log rate has decreasing differences in (N, slope), so the
    best N cannot grow when the slope (longer contexts) grows (Topkis)."""
    rng = np.random.default_rng(seed)
    a = rng.uniform(0.0, 1.0, (3, 4))
    a = a / a.sum(axis=1, keepdims=True) * rng.uniform(0.3, 0.9, (3, 1))
    best = []
    for slope in (0.05, 0.2, 0.8, 3.2):
        nodes = [2, 30]
        best.append(BU.tree_budget(a, nodes, [5.0 + slope * n for n in nodes], 40.0, 4)["best_n"])
    assert best == sorted(best, reverse=True), best
    assert best[0] > best[-1]
