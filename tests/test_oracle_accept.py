"""Pins of the oracle greedy and typical acceptance."""
import itertools

import numpy as np
import pytest

import workloads
from oracle import accept as AC
from oracle import tree as T
from oracle import typical as TY
from conftest import load_golden


def a31():
    g = load_golden("a31_round.json")["printed"]
    t = T.compile_tree([tuple(p) for p in g["rank_paths"]], g["num_heads"], g["topk"])
    cand = [g["root_token"]] + g["head0_ranks"] + g["head1_ranks"]
    return g, t, T.tree_tokens(t, cand)


def test_a31_greedy_winner():
    g, t, tokens = a31()
    target = np.full(t["n_nodes"], 999, np.int32)
    target[0] = 21          # after the root 11 the target wants 21
    target[1] = 31          # after (11, 21) it wants 31
    res = AC.greedy_accept(tokens, target, t["retrieve"])
    assert res["accepted_tokens"] == g["greedy_winner_tokens"]
    assert res["accept_len"] == g["greedy_winner_accept_len"]
    assert int((res["per_path"] == 2).sum()) == 1            # the only two-edge match
    assert res["frontier_row"] == 3                           # row of path (0,0)


def test_all_fail_defaults_to_path_zero():
    gold = load_golden("acceptance.json")["all_fail"]
    _, t, tokens = a31()
    target = np.full(t["n_nodes"], 999, np.int32)
    res = AC.greedy_accept(tokens, target, t["retrieve"])
    assert res["best_path"] == gold["best_path"] and res["accept_len"] == gold["accept_len"]
    assert len(res["accepted_tokens"]) == gold["published"] == 1
    assert res["accepted_tokens"] == [11]


def test_partII_match_vector():
    gold = load_golden("acceptance.json")["partII_match_vector"]
    t = T.compile_tree(workloads.cartesian_paths((1, 1, 1, 1)), 4, 1)
    tokens = np.array([100, 101, 102, 103, 104], np.int32)
    target = np.zeros(5, np.int32)
    for j, ok in enumerate(gold["raw_matches"]):
        target[j] = tokens[j + 1] if ok else 7
    assert AC.greedy_accept(tokens, target, t["retrieve"])["accept_len"] == gold["accepted_length"]


def test_sentinel_is_never_a_match():
    # a depth-1 leaf followed by a sentinel: the padded slot must not match anything,
    # even when the target of the leaf equals the token of the last row (what index -1 would read)
    t = T.compile_tree([(0,), (1,), (1, 0)], 2, 2)
    tokens = np.array([5, 6, 7, 8], np.int32)
    target = np.array([6, 8, 9, 9], np.int32)      # root->6 matches (0); target[(0)] = tokens[-1] = 8
    res = AC.greedy_accept(tokens, target, t["retrieve"])
    assert t["retrieve"][0].tolist() == [0, 1, -1]
    assert res["accept_len"] == 1 and res["best_path"] == 0


def test_argmax_lowest_index_and_nan():
    assert AC.row_argmax([1.0, 3.0, 3.0, 2.0]) == 1
    assert AC.row_argmax_fast(np.array([1.0, 3.0, 3.0], np.float32)) == 1
    with pytest.raises(AC.AcceptError):
        AC.row_argmax([1.0, np.nan])


def _longest_prefix(path_tokens, greedy):
    """[Chai] A(c) = max{a : c_j = g_j for all j <= a}."""
    best = 0
    for a in range(1, len(path_tokens) + 1):
        if all(path_tokens[j] == greedy[j] for j in range(a)):
            best = a
    return best


@pytest.mark.parametrize("seed,paths", [
    (0, [(0,), (1,), (0, 0), (0, 1), (1, 0), (1, 1)]),
    (1, [(0,), (1,), (0, 0), (0, 1), (1, 0), (1, 1)]),
    (2, [(0,), (1,), (0, 0), (0, 0, 0), (0, 0, 1)]),
    (3, [(1,), (0,), (1, 1), (1, 1, 0)]),
])
def test_brute_force_and_tree_walk(seed, paths):
    """Every target assignment over a 3-token vocabulary against [Chai]'s longest-prefix formula."""
    rng = np.random.default_rng(seed)
    K, TOPK, V = 3, 2, 3
    t = T.compile_tree(paths, K, TOPK)
    n = t["n_nodes"]
    cand = np.concatenate([[0], rng.permutation(V)[:TOPK], rng.permutation(V)[:TOPK],
                           rng.permutation(V)[:TOPK]]).astype(np.int32)
    tokens = T.tree_tokens(t, cand)
    for target in itertools.product(range(V), repeat=n):
        target = np.array(target, np.int32)
        res = AC.greedy_accept(tokens, target, t["retrieve"])
        per_path = []
        for r in t["retrieve"]:
            rows = [int(x) for x in r if x >= 0]
            per_path.append(_longest_prefix([tokens[v] for v in rows[1:]],
                                            [target[v] for v in rows[:-1]]))
        assert res["accept_len"] == max(per_path)
        assert res["best_path"] == per_path.index(max(per_path))
        walk = AC.tree_walk_accept(tokens, target, t["parent"])
        assert walk == res["rows"]


@pytest.mark.parametrize("name", ["tiny", "llama7b"])
def test_planted_acceptance_recovers_planted_depth(name):
    w = workloads.WORKLOADS[name]
    spec = workloads.tree_spec(w)
    t = (T.compile_tree(spec["paths"], w.num_heads, w.topk) if spec["paths"] is not None
         else T.compile_greedy(spec["rank_hit"], spec["n_nodes"]))
    x = workloads.draw_round(w)
    rng = np.random.default_rng(100)
    for trial in range(4):
        path = int(rng.integers(0, t["n_paths"]))
        real = int((t["retrieve"][path] >= 0).sum()) - 1
        depth = int(rng.integers(0, real + 1))
        y = dict(x)
        y["logits"] = None if x["logits"] is None else x["logits"].copy()
        y["target_ids"] = None if x["target_ids"] is None else x["target_ids"].copy()
        tokens = T.tree_tokens(t, x["candidates"][0])
        workloads.plant_acceptance(rng, y, tokens, t["retrieve"], t["parent"], 0, path, depth)
        res = AC.accept_batch(t, x["candidates"], logits=y["logits"], target_ids=y["target_ids"])
        assert res["accept_len"][0] == depth
        rows = [int(r) for r in t["retrieve"][res["best_path"][0], : depth + 1]]
        assert rows == [int(r) for r in t["retrieve"][path, : depth + 1]]


# ---------------------------------------------------------------- frontier carry

@pytest.mark.parametrize("seed,paths", [
    (0, [(0,), (1,), (0, 0), (0, 1), (1, 0), (1, 1)]),
    (2, [(0,), (1,), (0, 0), (0, 0, 0), (0, 0, 1)]),
])
def test_frontier_carry_is_where_the_tree_walk_stops(seed, paths):
    """[M7.2] §0x06C: the next round starts from the row after the last accepted input.
    The tree walk (an independent algorithm) stops at a row whose target token no child
    carries: that row must be the frontier, and the token it stops on the next root."""
    rng = np.random.default_rng(seed)
    K, TOPK, V = 3, 2, 3
    t = T.compile_tree(paths, K, TOPK)
    n = t["n_nodes"]
    cand = np.concatenate([[0], rng.permutation(V)[:TOPK], rng.permutation(V)[:TOPK],
                           rng.permutation(V)[:TOPK]]).astype(np.int32)[None, :]
    hidden = rng.standard_normal((1, n, 4))
    for target in itertools.product(range(V), repeat=n):
        target = np.array(target, np.int32)[None, :]
        res = AC.accept_batch(t, cand, target_ids=target)
        carry = AC.frontier_carry(res, hidden)
        walk = AC.tree_walk_accept(T.tree_tokens(t, cand[0]), target[0], t["parent"])
        assert int(res["frontier_row"][0]) == walk[-1]
        assert int(carry["next_root"][0]) == int(target[0][walk[-1]])
        children = [v for v, par in enumerate(t["parent"]) if par == walk[-1]]
        tokens = T.tree_tokens(t, cand[0])
        assert all(int(tokens[c]) != int(carry["next_root"][0]) for c in children)
        assert np.array_equal(carry["h_next"][0], hidden[0, walk[-1]])


def test_frontier_carry_a31_trace():
    """The A31 commit trace ([M7.2] §0x06B-§0x06C): tokens [11, 22, 31] on rows [0, 2, 6] are
    published (a = 2) and the printed terminal frontier is row 6, so the next round starts
    from row 6's distributions -- not row 2's (a - 1) nor another path's."""
    g, t, tokens = a31()
    commit = g["commit"]
    target = np.full(t["n_nodes"], 999, np.int32)
    target[0] = 22          # after the root the target wants 22 (row 2)
    target[2] = 31          # after (11, 22) it wants 31 (row 6)
    target[6] = 777         # the token the target emits after the accepted prefix
    res = AC.accept_batch(t, np.array([[g["root_token"]] + g["head0_ranks"] + g["head1_ranks"]]),
                          target_ids=target[None, :])
    assert res["accepted_tokens"][0][: commit["G"]].tolist() == commit["tokens"]
    assert int(res["frontier_row"][0]) == commit["terminal_frontier_row"] == 6
    hidden = np.arange(t["n_nodes"] * 3, dtype=np.float64).reshape(1, t["n_nodes"], 3)
    carry = AC.frontier_carry(res, hidden)
    assert int(carry["next_root"][0]) == 777
    assert np.array_equal(carry["h_next"][0], hidden[0, 6])


# ---------------------------------------------------------------- typical acceptance

def test_typical_five_token_distribution_all_pass():
    gold = load_golden("acceptance.json")["typical_five_token"]
    p = np.array(gold["probabilities"])
    probs = TY.softmax(np.log(p), 1.0)
    assert np.allclose(probs, p)
    tau = TY.threshold(probs)
    assert all(pc > tau for pc in probs) == gold["all_pass_typical"]
    assert int(np.argmax(probs)) == gold["greedy_token_index"]


def test_typical_threshold_closed_forms():
    # uniform over V: H = log V (up to the 1e-5 guard), tau = min(eps, alpha / V)
    V = 50
    p = np.full(V, 1.0 / V)
    assert TY.entropy(p) == pytest.approx(np.log(V), rel=1e-3)
    assert TY.threshold(p) == pytest.approx(min(0.3, 0.09 / V), rel=1e-3)
    # a sharp distribution: H -> 0, tau -> min(eps, alpha) = alpha
    sharp = TY.softmax(np.array([50.0, 0.0, 0.0]), 1.0)
    assert TY.threshold(sharp) == pytest.approx(0.09, rel=1e-4)
    # the comparison is strict: p(c) == tau does not pass, p(c) just above tau does
    t = T.compile_tree([(0,)], 1, 1)
    tokens = np.array([0, 1], np.int32)
    logits = np.log(np.array([[0.91, 0.09], [0.5, 0.5]]))
    pc = TY.softmax(logits[0], 1.0)[1]
    at = TY.typical_accept(tokens, logits, t["retrieve"], 1.0, epsilon=pc, alpha=10.0)
    below = TY.typical_accept(tokens, logits, t["retrieve"], 1.0, epsilon=np.nextafter(pc, 0.0), alpha=10.0)
    assert at["accept_len"] == 0 and below["accept_len"] == 1


def test_typical_low_temperature_is_greedy():
    rng = np.random.default_rng(7)
    t = T.compile_greedy(workloads.rank_hit_table(3, 4), 20)
    V = 12
    for _ in range(10):
        cand = np.concatenate([[0]] + [rng.permutation(V)[:4] for _ in range(3)]).astype(np.int32)
        tokens = T.tree_tokens(t, cand)
        logits = rng.standard_normal((t["n_nodes"], V)) * 3
        for r in range(t["n_nodes"]):
            if rng.random() < 0.5:
                kids = [v for v in range(t["n_nodes"]) if t["parent"][v] == r]
                if kids:
                    logits[r, tokens[kids[0]]] += 10.0
        greedy = AC.greedy_accept(tokens, logits.argmax(axis=1), t["retrieve"])
        typ = TY.typical_accept(tokens, logits, t["retrieve"], 1e-3)
        assert typ["accept_len"] == greedy["accept_len"]
        assert typ["rows"] == greedy["rows"]


def test_typical_tie_break_uses_log_likelihood_not_probability_sum():
    # two depth-2 paths both pass twice; path B has the larger product of
    # probabilities but the smaller sum, so a raw-probability tie-break picks A
    t = T.compile_tree([(0,), (1,), (0, 0), (1, 0)], 2, 2)
    tokens = np.array([0, 1, 2, 3, 4], np.int32)     # rows: root, (0), (1), (0,0), (1,0)
    V = 5

    def row(pmap):
        p = np.full(V, 1e-6)
        for k, v in pmap.items():
            p[k] = v
        return np.log(p / p.sum())
    logits = np.stack([
        row({1: 0.60, 2: 0.40}),          # root: p(1)=.60 (path A), p(2)=.40 (path B)
        row({3: 0.15, 0: 0.85}),          # after (0): p(3)=.15
        row({4: 0.30, 0: 0.70}),          # after (1): p(4)=.30
        row({0: 1.0}), row({0: 1.0})])
    res = TY.typical_accept(tokens, logits, t["retrieve"], 1.0, epsilon=0.1, alpha=10.0)
    assert res["accept_len"] == 2
    # A: .60*.15 = .090 (sum .75); B: .40*.30 = .120 (sum .70) -> B by likelihood
    assert res["rows"] == [0, 2, 4]
