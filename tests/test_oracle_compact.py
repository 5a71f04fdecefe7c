"""Pins of the oracle K/V compaction."""
import numpy as np
import pytest

from oracle import compact as C
from oracle import tree as T
from conftest import load_golden


def _a31_tree():
    g = load_golden("a31_round.json")
    pr = g["printed"]
    return g, T.compile_tree([tuple(p) for p in pr["rank_paths"]], pr["num_heads"], pr["topk"])


def test_a31_commit_trace():
    g, t = _a31_tree()
    c = g["printed"]["commit"]
    P = g["printed"]["prefix_len"]
    best = g["derived_by_hand"]["commit_path_index_ascending_leaves"]
    assert t["retrieve"][best, : c["G"]].tolist() == c["retrieve_rows"]
    src, dst = C.commit_plan(t["retrieve"], best, c["accept_len"], P, t["n_nodes"], P + t["n_nodes"])
    assert src == c["source_rows"] and dst == c["destination_rows"]
    # row contents tagged by their row index, two layers, K and V
    S = P + t["n_nodes"]
    caches = [np.arange(S, dtype=np.float64)[None, None, :, None] * np.ones((1, 2, S, 3)) + 1000 * i
              for i in range(4)]
    before = [x.copy() for x in caches]
    new_len = C.kv_compact(caches, t["retrieve"], [best], [c["accept_len"]], [P], t["n_nodes"])
    assert new_len.tolist() == [c["new_length"]]
    for x, x0 in zip(caches, before):
        assert np.array_equal(x[0, :, dst], x0[0, :, src])              # gathered winning rows
        assert np.array_equal(x[0, :, :P], x0[0, :, :P])                # committed prefix untouched
        assert np.array_equal(x[0, :, P + c["G"]:], x0[0, :, P + c["G"]:])   # stale rows stay
    assert t["retrieve"][best, c["accept_len"]] == c["terminal_frontier_row"]


def test_overlapping_rows_need_the_snapshot():
    # rows [0,2,6] at P=5 overlap: destination 7 is the source of j=1 ... and a
    # reverse-order in-place copy would read an overwritten row
    g, t = _a31_tree()
    P = 5
    S = P + t["n_nodes"]
    x = np.arange(S, dtype=np.float64).reshape(1, 1, S, 1)
    ref = x.copy()
    C.kv_compact([x], t["retrieve"], [3], [2], [P], t["n_nodes"])
    assert x[0, 0, 5:8, 0].tolist() == [5.0, 7.0, 11.0]
    bad = ref.copy()
    for j, s in reversed(list(enumerate([5, 7, 11]))):
        bad[0, 0, P + j] = bad[0, 0, s]
    assert bad[0, 0, 5:8, 0].tolist() != [5.0, 7.0, 11.0]


@pytest.mark.parametrize("best,alen,P,code", [
    (6, 0, 5, "path"), (-1, 0, 5, "path"), (0, 3, 5, "length"), (0, 0, 6, "capacity"), (0, 0, -1, "capacity")])
def test_validation_happens_before_mutation(best, alen, P, code):
    _, t = _a31_tree()
    S = 5 + t["n_nodes"]
    x = np.random.default_rng(0).standard_normal((2, 1, S, 4))
    x0 = x.copy()
    with pytest.raises(C.CompactError):
        # sequence 0 is valid, sequence 1 is not: nothing may change
        C.kv_compact([x], t["retrieve"], [0, best], [1, alen], [5, P], t["n_nodes"])
    assert np.array_equal(x, x0)


def test_sentinel_inside_published_rows_is_rejected():
    t = T.compile_tree([(0,), (1,), (1, 0)], 2, 2)     # retrieve row 0 = [0, 1, -1]
    x = np.zeros((1, 1, 10, 2))
    with pytest.raises(C.CompactError):
        C.kv_compact([x], t["retrieve"], [0], [2], [3], t["n_nodes"])
