"""Pins of the oracle tree compiler against what the pages print and what the mathematics fixes."""
import itertools
import random

import numpy as np
import pytest

import workloads
from oracle import tree as T
from conftest import load_golden


def _children(parent):
    ch = {}
    for v, p in enumerate(parent):
        if p >= 0:
            ch.setdefault(int(p), []).append(v)
    return ch


# ---------------------------------------------------------------- printed counts

@pytest.mark.parametrize("case", load_golden("regular_trees.json")["cases"])
def test_regular_tree_counts(case):
    br = case["branching"]
    t = T.compile_tree(workloads.cartesian_paths(br), len(br), max(br))
    if "non_root_nodes" in case:
        assert t["n_nodes"] - 1 == case["non_root_nodes"]
    if "per_depth" in case:
        counts = [int((t["depth"] == k).sum()) for k in range(1, len(br) + 1)]
        assert counts == case["per_depth"]
    if "full_paths" in case:
        assert t["n_paths"] == case["full_paths"]


def test_wide_cartesian_shape():
    t = T.compile_tree(workloads.cartesian_paths((4, 4, 4, 4)), 4, 4)
    assert (t["n_nodes"], t["n_paths"], t["path_width"], t["mask_words"]) == (341, 256, 5, 6)


# ---------------------------------------------------------------- a/b/u tree

def test_abu_tree_printed_and_derived():
    g = load_golden("abu_tree.json")
    d = g["derived_by_hand"]
    t = T.compile_tree([tuple(p) for p in d["rank_paths"]], d["num_heads"], d["topk"])
    names = g["printed"]["flattened_nodes"]
    assert t["n_nodes"] == len(names) == 7
    # the page's flattening order: a, b, u, c|b, v|b, c|u, v|u
    sym = {(): "a", (0,): "b", (1,): "u", (0, 0): "c|b", (0, 1): "v|b", (1, 0): "c|u", (1, 1): "v|u"}
    assert [sym[p] for p in [()] + t["paths"]] == names
    assert list(t["depth"]) == g["printed"]["positions_offset_from_L"]
    cu = names.index("c|u")
    seen = [names[v] for v in range(7) if t["mask"][cu, v]]
    assert sorted(seen) == sorted(g["printed"]["visible_to_c|u"])
    assert t["n_paths"] * t["path_width"] == g["printed"]["batch_token_count_without_tree"]
    assert list(t["tree_indices"]) == d["tree_indices"]
    assert t["retrieve"].tolist() == d["retrieve"]


# ---------------------------------------------------------------- A31 tree

def test_a31_tree_coordinates():
    g = load_golden("a31_round.json")
    pr = g["printed"]
    t = T.compile_tree([tuple(p) for p in pr["rank_paths"]], pr["num_heads"], pr["topk"])
    cand = [pr["root_token"]] + pr["head0_ranks"] + pr["head1_ranks"]
    tokens = T.tree_tokens(t, cand)
    assert tokens.tolist() == g["derived_by_hand"]["row_tokens"]
    P = pr["prefix_len"]
    assert T.positions(t, P).tolist() == pr["positions"]
    n = t["n_nodes"]
    assert [1, 1, n, P + n] == pr["rect_mask_shape"]
    assert t["n_paths"] == pr["n_paths"]
    assert [P + u for u in range(n)] == pr["staged_rows"]
    slots, counts = np.unique(t["tree_indices"], return_counts=True)
    assert sorted(int(s) for s, c in zip(slots, counts) if c == 2) == pr["slots_appearing_twice"]


def test_six_node_mask_example():
    # M7.2 §0x03B: root; A(A1, A2); B(B1), flattened [A, B, A1, A2, B1]
    t = T.compile_tree([(0,), (1,), (0, 0), (0, 1), (1, 0)], 2, 2)
    A, B, A1, A2, B1 = 1, 2, 3, 4, 5
    m = t["mask"]
    assert m[A1, A] and m[A1, 0] and m[A1, A1]
    assert not (m[A1, B] or m[A1, A2] or m[A1, B1])
    # §0x03A: siblings share a position; positions follow depth, not packed order
    assert list(t["depth"][1:]) == [1, 1, 2, 2, 2]


# ---------------------------------------------------------------- invariants on random trees

def _random_prefix_closed(rng, num_heads, topk, size):
    size = min(size, sum(topk ** d for d in range(1, num_heads + 1)))
    paths = set()
    while len(paths) < size:
        p = ()
        depth = rng.randint(1, num_heads)
        for _ in range(depth):
            p = p + (rng.randrange(topk),)
            paths.add(p)
            if len(paths) >= size:
                break
    return list(paths)


@pytest.mark.parametrize("seed", range(6))
def test_mask_and_buffer_invariants(seed):
    rng = random.Random(seed)
    K, TOPK = rng.randint(1, 4), rng.randint(1, 5)
    paths = _random_prefix_closed(rng, K, TOPK, rng.randint(1, 30))
    t = T.compile_tree(paths, K, TOPK)
    n, m, parent, depth = t["n_nodes"], t["mask"], t["parent"], t["depth"]
    rows = [()] + t["paths"]
    # canonical order: sorted by (len, path), never re-sorted
    assert t["paths"] == sorted(t["paths"], key=lambda p: (len(p), p))
    for u in range(n):
        assert m[u, u] and m[u, 0]                          # reflexive, root visible
        assert depth[u] == len(rows[u])                     # position == len(path)
        for v in range(n):
            if m[u, v]:                                     # ancestor-transitive
                assert all(m[u, w] for w in range(n) if m[v, w])
            if v != u and parent[v] == parent[u] and parent[u] >= 0:
                assert not m[u, v]                          # sibling-exclusive
        if u:
            p = rows[u]
            assert t["tree_indices"][u] == 1 + (len(p) - 1) * TOPK + p[-1]
            assert rows[parent[u]] == p[:-1]
    # packed bits agree with the dense mask
    for u in range(n):
        for v in range(n):
            bit = (int(t["mask_packed"][u, v // 64]) >> (v % 64)) & 1
            assert bit == int(m[u, v])
    # retrieve: maximal paths only, each step a parent->child edge, sentinel after the end
    ch = _children(parent)
    leaves = sorted(u for u in range(n) if u not in ch)
    assert t["retrieve"].shape == (len(leaves), int(depth.max()) + 1)
    for i, r in enumerate(t["retrieve"]):
        real = [int(x) for x in r if x >= 0]
        assert real[0] == 0 and real[-1] == leaves[i]
        assert all(x == -1 for x in r[len(real):])
        for a, b in zip(real, real[1:]):
            assert parent[b] == a and m[b, a]


# ---------------------------------------------------------------- greedy growth

def test_partII_greedy_order():
    g = load_golden("greedy_toys.json")["partII"]["printed"]
    a = g["rank_hit"]
    for key, w in g["scores"].items():
        p = tuple(int(x) for x in key.split(","))
        assert T.path_weight(a, p) == pytest.approx(w, rel=1e-12)
    order = [tuple(p) for p in g["greedy_order"]]
    assert T.greedy_frontier(a, len(order)) == order
    assert T.greedy_top_b(a, len(order)) == order


def test_m72_toy_budget_ten():
    g = load_golden("greedy_toys.json")["m72"]
    a, budget = g["printed"]["rank_hit"], g["printed"]["budget"]
    want = sorted(tuple(p) for p in g["derived_by_hand"]["selected"])
    assert sorted(T.greedy_frontier(a, budget)) == want
    assert sorted(T.greedy_top_b(a, budget)) == want


def _all_paths(K, TOPK):
    return [p for d in range(1, K + 1) for p in itertools.product(range(TOPK), repeat=d)]


@pytest.mark.parametrize("K,TOPK,seed", [(3, 2, 0), (2, 3, 1), (3, 2, 2), (2, 2, 3)])
def test_greedy_is_optimal_by_brute_force(K, TOPK, seed):
    """Exhaustive: the greedy set maximises sum(w) over every prefix-closed set of its size."""
    rng = np.random.default_rng(seed)
    a = rng.uniform(0.0, 1.0, size=(K, TOPK))
    every = _all_paths(K, TOPK)
    best = {}
    for mask in range(1 << len(every)):
        chosen = [every[i] for i in range(len(every)) if mask >> i & 1]
        s = set(chosen)
        if any(p[:k] not in s for p in chosen for k in range(1, len(p))):
            continue
        total = sum(T.path_weight(a, p) for p in chosen)
        best[len(chosen)] = max(best.get(len(chosen), -1.0), total)
    for budget in range(len(every) + 1):
        got = T.greedy_frontier(a, budget)
        assert sorted(got) == sorted(T.greedy_top_b(a, budget))
        assert sum(T.path_weight(a, p) for p in got) == pytest.approx(best[budget], rel=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_expected_length_tail_sum(seed):
    """sum_u w(u) equals E[accepted depth] under the independent exact-rank model, by enumeration."""
    rng = np.random.default_rng(seed)
    K, TOPK = 3, 3
    a = rng.uniform(0.0, 1.0, size=(K, TOPK))
    a = a / a.sum(axis=1, keepdims=True) * rng.uniform(0.5, 1.0, size=(K, 1))
    t = T.compile_greedy(a, 9)
    chosen = set(t["paths"])
    # outcome per head: the correct rank, or None (not in the pool) with the remaining mass
    per_head = [[(r, a[k, r]) for r in range(TOPK)] + [(None, 1.0 - a[k].sum())] for k in range(K)]
    expect = 0.0
    for outcome in itertools.product(*per_head):
        prob = np.prod([w for _, w in outcome])
        depth = 0
        for k in range(K):
            p = tuple(r for r, _ in outcome[: k + 1])
            if None in p or p not in chosen:
                break
            depth = k + 1
        expect += prob * depth
    assert T.expected_accept_length(t) == pytest.approx(expect, rel=1e-12)


def test_synthetic_rank_hit_tree_shape():
    """The 64-row tree of the rank-hit table used by the 64-node workloads (a derived regression value)."""
    t = T.compile_greedy(workloads.rank_hit_table(4, 10), 64)
    counts = [int((t["depth"] == k).sum()) for k in range(1, 5)]
    assert counts == [9, 28, 25, 1]
    assert (t["n_paths"], t["path_width"]) == (44, 5)
    # the boundary cuts the tie class (depth 3, rank sum 4) after its 5 smallest members
    deep = sorted(p for p in t["paths"] if len(p) == 3 and sum(p) == 4)
    assert deep == [(0, 0, 4), (0, 1, 3), (0, 2, 2), (0, 3, 1), (0, 4, 0)]


# ---------------------------------------------------------------- rejected specifications

@pytest.mark.parametrize("paths,K,TOPK,code", [
    ([(0, 1)], 2, 2, "ENOT_PREFIX_CLOSED"),
    ([(0,), (0, 2)], 2, 2, "EINVAL"),
    ([(0,), (0, 0), (0, 0, 0)], 2, 2, "EINVAL"),
    ([(0,), (0,)], 2, 2, "EINVAL"),
    ([()], 2, 2, "EINVAL"),
])
def test_invalid_specs(paths, K, TOPK, code):
    with pytest.raises(T.TreeError) as e:
        T.compile_tree(paths, K, TOPK)
    assert e.value.code == code


def test_invalid_greedy():
    with pytest.raises(T.TreeError):
        T.greedy_frontier([[0.5, 0.5]], 3)
    with pytest.raises(T.TreeError):
        T.greedy_frontier([[1.5, 0.5]], 1)
    with pytest.raises(T.TreeError):
        T.greedy_frontier([[np.nan, 0.5]], 1)


def test_root_only_tree():
    t = T.compile_tree([], 2, 2)
    assert t["n_nodes"] == 1 and t["retrieve"].tolist() == [[0]]
    assert T.compile_greedy([[0.5, 0.25]], 1)["n_nodes"] == 1
