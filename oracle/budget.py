"""Oracle: the context-dependent tree budget.

TEST INFRASTRUCTURE (see the package docstring).

Follows:

* [M7.2] §0x04B "Calibration Probabilities And Expected Accepted Length": the expected accepted
  length of a tree is the sum of its non-root path weights.
* [M7.2] §0x04C "Greedy Frontier Search And Its Boundary": the greedy search maximises the
  expected accepted length per round, which is not tokens per second, because nodes carry
  kernel and cache costs.
* [Chai] section "局限与适用场景": in long contexts every tree query reads the history KV, so
  attention traffic grows with context length and node count, and the best node count
  should change with context length.

Reading taken (the pages give no formula): for the nested greedy trees T_N (N rows including
the root), a round publishes 1 + E[A](N) tokens on average and costs
fixed_us + n_layers * t(N) microseconds, where t(N) is the measured per-layer cost of the
tree-dependent work at the round's context length, interpolated linearly between measured
node counts, and fixed_us the tree-independent part (the backbone's weight stream).  The
budget is the N in the measured range with the largest (1 + E[A](N)) / cost, the smallest N
on exact ties.  Arithmetic in binary64.
"""
from __future__ import annotations

import numpy as np

from oracle import tree as T


def expected_accept(rank_hit, n_nodes: int) -> float:
    """E[A] of the greedy tree with n_nodes rows: grow it, compile it, sum its weights."""
    if n_nodes == 1:
        return 0.0
    return T.expected_accept_length(T.compile_greedy(rank_hit, n_nodes))


def cost(cost_nodes, cost_us, n: int) -> float:
    """Per-layer cost of an n-row round, linear between the measured node counts."""
    return float(np.interp(n, np.asarray(cost_nodes, np.float64), np.asarray(cost_us, np.float64)))


def tree_budget(rank_hit, cost_nodes, cost_us, fixed_us: float, n_layers: int) -> dict:
    """Best node count over [cost_nodes[0], cost_nodes[-1]] and the table behind it."""
    lo, hi = int(cost_nodes[0]), int(cost_nodes[-1])
    table = {}
    for n in range(lo, hi + 1):
        ea = expected_accept(rank_hit, n)
        table[n] = (1.0 + ea, (1.0 + ea) / (fixed_us + n_layers * cost(cost_nodes, cost_us, n)))
    best = max(table, key=lambda n: (table[n][1], -n))
    return {"best_n": best, "table": table}
