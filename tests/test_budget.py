"""medusa_tree_budget (host, through the C ABI) against the oracle."""
import numpy as np
import pytest

import medusa_tree_attention_amd as M
import workloads
from oracle import budget as BU


def compare(a, nodes, us, fixed, layers):
    best, et, rt = M.medusa_tree_budget(a, nodes, us, fixed, layers)
    ref = BU.tree_budget(a, nodes, us, fixed, layers)
    for n, (tokens, rate) in ref["table"].items():
        assert abs(et[n] - tokens) <= 1e-12 * tokens, n
        assert abs(rt[n] - rate) <= 1e-12 * rate, n
    rates = sorted((r for _, r in ref["table"].values()), reverse=True)
    if len(rates) < 2 or rates[0] - rates[1] > 1e-9 * rates[0]:   # a clear winner
        assert best == ref["best_n"]
    else:                                                          # a near-tie: either is right
        assert abs(ref["table"][best][1] - rates[0]) <= 1e-9 * rates[0]
    assert rt[: nodes[0]].sum() == 0.0
    return best


def test_hand_computed_case():
    assert compare([[0.5, 0.3, 0.1]], [1, 4], [1.0, 4.0], 10.0, 1) == 3
    assert compare([[0.5, 0.3, 0.1]], [1, 4], [1.0, 4.0], 0.0, 1) == 1


@pytest.mark.parametrize("seed", range(8))
def test_random_tables_and_curves(seed):
    rng = np.random.default_rng(seed)
    K, TOPK = int(rng.integers(1, 5)), int(rng.integers(2, 8))
    a = rng.uniform(0.0, 1.0, (K, TOPK))
    a = a / a.sum(axis=1, keepdims=True) * rng.uniform(0.2, 0.95, (K, 1))
    cap = sum(TOPK ** d for d in range(1, K + 1)) + 1
    hi = int(min(cap, rng.integers(8, 120)))
    nodes = sorted(set([1, hi] + [int(x) for x in rng.integers(1, hi, 3)]))
    us = np.cumsum(rng.uniform(0.5, 5.0, len(nodes)))
    compare(a, nodes, us, float(rng.uniform(0, 200)), int(rng.integers(0, 40)))


def test_the_workload_rank_table():
    a = workloads.rank_hit_table(4, 10)
    compare(a, [16, 32, 64, 128], [30.0, 33.0, 39.0, 52.0], 2000.0, 32)


def test_errors():
    a = [[0.5, 0.3, 0.1]]
    for args in ([a, [4, 2], [1.0, 2.0], 1.0, 1], [a, [0, 2], [1.0, 2.0], 1.0, 1],
                 [a, [1, 2], [1.0, -2.0], 1.0, 1], [a, [1, 2], [1.0, 2.0], -1.0, 1],
                 [[[1.5, 0.3, 0.1]], [1, 2], [1.0, 2.0], 1.0, 1], [a, [1, 2], [1.0, 2.0], 0.0, 0]):
        with pytest.raises(M.MedusaError):
            M.medusa_tree_budget(*args)
    with pytest.raises(M.MedusaError):      # one head of 3 ranks holds 4 rows at most
        M.medusa_tree_budget(a, [1, 5], [1.0, 2.0], 1.0, 1)
