"""Pins of the oracle head step and candidate pool (CPU only).

Each pin fixes the oracle by something other than its own formula: the pages' statement
that a zero residual projection leaves the head equal to an unembedding of h, SiLU's limits,
matrices whose products are known by construction (a shift, a coordinate selection), the
defining property of a ranking checked by brute force, and the slot layout of the tree
compiler's candidate gather.
"""
import itertools

import numpy as np
import pytest

from oracle import heads as HD
from oracle import tree as T


def test_zero_residual_projection_is_the_unembedding():
    # [Math] "The Medusa head: math and shapes": W1 near zero gives SiLU(0) + h = h
    rng = np.random.default_rng(0)
    d, V = 16, 40
    h = rng.standard_normal(d)
    W2 = rng.standard_normal((V, d))
    got = HD.head_logits(h, np.zeros((d, d)), W2)
    assert np.array_equal(got, W2 @ h)


def test_silu_limits_not_sigmoid():
    # large positive inputs pass through, large negative ones vanish, zero maps to zero
    x = np.array([-60.0, -30.0, 0.0, 30.0, 60.0])
    y = HD.silu(x)
    assert y[2] == 0.0
    assert abs(y[0]) < 1e-20 and abs(y[1]) < 1e-11
    assert abs(y[3] - 30.0) < 1e-11 and y[4] == 60.0


def test_residual_projection_orientation():
    # W1 shifts coordinates: (W1 h)[o] = h[o + 1]; a transposed W1 would shift the other way
    d = 6
    h = np.array([0.5, -1.0, 2.0, -0.25, 1.5, 3.0])
    W1 = np.eye(d, k=1)
    W2 = np.eye(d)
    u = HD.head_logits(h, W1, W2)
    shifted = np.append(h[1:], 0.0)
    expect = h + shifted / (1.0 + np.exp(-shifted))
    assert np.allclose(u, expect, rtol=0, atol=1e-15)
    assert not np.allclose(u, h + np.append(0.0, h[:-1]) / (1.0 + np.exp(-np.append(0.0, h[:-1]))))


def test_unembedding_orientation_selects_coordinates():
    # W2 row v picks coordinate v % d of u: logits[v] = u[v % d]
    d, V = 5, 12
    h = np.array([0.3, -2.0, 1.0, 0.7, -0.1])
    W2 = np.zeros((V, d))
    W2[np.arange(V), np.arange(V) % d] = 1.0
    got = HD.head_logits(h, np.zeros((d, d)), W2)
    assert np.array_equal(got, h[np.arange(V) % d])


@pytest.mark.parametrize("seed", range(6))
def test_ranking_matches_its_definition_by_brute_force(seed):
    # values from a small set, so that ties are frequent
    rng = np.random.default_rng(seed)
    V, k = 9, 4
    x = rng.integers(0, 4, V).astype(np.float64)
    got = HD.top_ranked(x, k)
    assert len(set(got)) == k
    rest = [j for j in range(V) if j not in got]
    for i in got:
        for j in rest:
            assert x[i] > x[j] or (x[i] == x[j] and i < j)
    for a, b in zip(got, got[1:]):
        assert x[a] > x[b] or (x[a] == x[b] and a < b)
    # and no other k-subset in rank order satisfies the same conditions
    winners = [c for c in itertools.permutations(range(V), k)
               if all(x[i] > x[j] or (x[i] == x[j] and i < j) for i in c for j in range(V) if j not in c)
               and all(x[a] > x[b] or (x[a] == x[b] and a < b) for a, b in zip(c, c[1:]))]
    assert winners == [tuple(got)]


def test_candidate_slots_feed_the_tree_gather():
    # [M7.2] 0x01B: slot(j, r) = 1 + j*TOPK + r, read by tree_indices; the token of a depth-d
    # node with last rank r is head d-1's rank-r token
    rng = np.random.default_rng(3)
    K, topk, d, V, B = 3, 4, 8, 30, 2
    h = rng.standard_normal((B, d))
    W1 = rng.standard_normal((K, d, d)) * 0.1
    W2 = rng.standard_normal((K, V, d))
    root = np.array([7, 11])
    res = HD.head_candidates(h, W1, W2, root, topk)
    paths = [(a,) for a in range(topk)] + [(a, b) for a in range(2) for b in range(topk)] + [(0, 0, 1)]
    tree = T.compile_tree(paths, K, topk)
    for b in range(B):
        tokens = res["candidates"][b][tree["tree_indices"]]
        assert tokens[0] == root[b]
        for u, p in enumerate(tree["paths"], start=1):  # the list starts at row 1 (the root has no path)
            depth, rank = len(p), p[-1]
            ranked = np.argsort(-res["logits"][depth - 1, b], kind="stable")
            assert tokens[u] == ranked[rank]
