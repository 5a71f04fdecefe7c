"""Planted mistakes in the oracle must be caught by its pins.

Each case patches one plausible error into the oracle (on the CPU) and runs
the pin test that is meant to catch it; the pin must fail.  The mistakes
follow the failure lists the pages give for their own oracles ([M7.2]
§0x03F, §0x04G, §0x06E) plus a few arithmetic slips.
"""
import numpy as np
import pytest

import test_oracle_accept as PA
import test_oracle_attention as PT
import test_oracle_budget as PB
import test_oracle_compact as PC
import test_oracle_heads as PH
import test_oracle_tree as PR
from oracle import accept as AC
from oracle import attention as A
from oracle import budget as BU
from oracle import compact as C
from oracle import heads as HD
from oracle import tree as T
from oracle import typical as TY


def must_fail(pin, *args):
    with pytest.raises(Exception):
        pin(*args)


# ---------------------------------------------------------------- attention

def test_packed_row_positions_are_caught(monkeypatch):
    real = A.tree_attention

    def packed_positions(*args, **kw):
        kw["depth"] = np.arange(len(kw["depth"]))          # position P + u instead of P + depth(u)
        return real(*args, **kw)
    monkeypatch.setattr(A, "tree_attention", packed_positions)
    must_fail(PT.test_every_small_tree_matches_per_path_causal_attention)


def test_sibling_leak_is_caught(monkeypatch):
    monkeypatch.setattr(A, "root_path", lambda parent, u: list(range(u + 1)))   # causal over packed order
    must_fail(PT.test_every_small_tree_matches_per_path_causal_attention)


def test_hidden_prompt_key_is_caught(monkeypatch):
    real = A.causal_last_row
    monkeypatch.setattr(A, "causal_last_row", lambda q, k, v: real(q, k[1:], v[1:]))
    must_fail(PT.test_root_only_is_single_query_decode)


def test_interleaved_rope_pairing_is_caught(monkeypatch):
    def interleaved(x, pos, base):
        x = np.asarray(x, np.float64)
        d = x.shape[-1]
        ang = pos * A.rope_inv_freq(d, base)
        c, s = np.cos(ang), np.sin(ang)
        out = x.copy()
        out[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
        out[..., 1::2] = x[..., 1::2] * c + x[..., 0::2] * s
        return out
    monkeypatch.setattr(A, "rope", interleaved)
    must_fail(PT.test_rope_matches_complex_form_and_properties)


def test_missing_softmax_scale_is_caught(monkeypatch):
    def unscaled(q_row, keys, values):
        s = keys @ q_row
        p = np.exp(s - s.max())
        return (p / p.sum()) @ values
    monkeypatch.setattr(A, "causal_last_row", unscaled)
    must_fail(PT.test_chain_tree_is_ordinary_causal_attention)


def test_wrong_gqa_mapping_is_caught(monkeypatch):
    real = A.tree_attention

    def modulo_groups(q, k_new, v_new, k_cache, v_cache, prefix_len, depth, parent, rope_base, rows=None):
        # head h -> kv h % Hkv instead of h // (Hq / Hkv): permute query heads to emulate it
        Hq, Hkv = q.shape[2], k_new.shape[2]
        perm = [(h % Hkv) * (Hq // Hkv) + h // Hkv for h in range(Hq)]
        out, sk, sv = real(q[:, :, perm], k_new, v_new, k_cache, v_cache, prefix_len, depth, parent, rope_base)
        inv = np.argsort(perm)
        return out[:, :, inv], sk, sv
    monkeypatch.setattr(A, "tree_attention", modulo_groups)
    must_fail(PT.test_every_small_tree_matches_per_path_causal_attention)


# ---------------------------------------------------------------- tree

def test_causal_mask_instead_of_ancestor_mask_is_caught(monkeypatch):
    real = T.compile_tree

    def causal(*a, **k):
        t = real(*a, **k)
        n = t["n_nodes"]
        t["mask"] = np.tril(np.ones((n, n), bool))
        return t
    monkeypatch.setattr(T, "compile_tree", causal)
    must_fail(PR.test_six_node_mask_example)


def test_slot_formula_off_by_one_is_caught(monkeypatch):
    real = T.compile_tree

    def shifted(*a, **k):
        t = real(*a, **k)
        t["tree_indices"] = np.where(t["depth"] > 0, t["tree_indices"] + t["topk"], 0).astype(np.int32)
        return t
    monkeypatch.setattr(T, "compile_tree", shifted)
    must_fail(PR.test_a31_tree_coordinates)


def test_last_rank_score_instead_of_path_product_is_caught(monkeypatch):
    # scoring a frontier path by its own head's rank mass only, not the product along the path
    monkeypatch.setattr(T, "path_weight", lambda a, p: float(a[len(p) - 1][p[-1]]))
    must_fail(PR.test_greedy_is_optimal_by_brute_force, 3, 2, 0)


def test_cumulative_instead_of_exact_rank_mass_is_caught(monkeypatch):
    monkeypatch.setattr(T, "path_weight", lambda a, p: float(np.prod([sum(a[j][: r + 1]) for j, r in enumerate(p)])))
    must_fail(PR.test_partII_greedy_order)


# ---------------------------------------------------------------- acceptance

def test_non_prefix_counting_is_caught(monkeypatch):
    def count_all(tokens, target, retrieve):
        a = np.zeros(len(retrieve), np.int32)
        for i, r in enumerate(retrieve):
            rows = [int(x) for x in r if x >= 0]
            a[i] = sum(int(tokens[v]) == int(target[u]) for u, v in zip(rows, rows[1:]))
        return a
    monkeypatch.setattr(AC, "path_accept_lengths", count_all)
    must_fail(PA.test_partII_match_vector)


def test_self_aligned_logits_are_caught(monkeypatch):
    def self_aligned(tokens, target, retrieve):
        a = np.zeros(len(retrieve), np.int32)
        for i, r in enumerate(retrieve):
            rows = [int(x) for x in r if x >= 0]
            for v in rows[1:]:
                if int(tokens[v]) != int(target[v]):
                    break
                a[i] += 1
        return a
    monkeypatch.setattr(AC, "path_accept_lengths", self_aligned)
    must_fail(PA.test_a31_greedy_winner)


def test_sentinel_as_index_is_caught(monkeypatch):
    def sentinel_reads_last_row(tokens, target, retrieve):
        a = np.zeros(len(retrieve), np.int32)
        for i, r in enumerate(retrieve):
            for j in range(len(r) - 1):
                if int(tokens[int(r[j + 1])]) != int(target[int(r[j])]):
                    break
                a[i] += 1
        return a
    monkeypatch.setattr(AC, "path_accept_lengths", sentinel_reads_last_row)
    must_fail(PA.test_sentinel_is_never_a_match)


def test_frontier_from_row_a_minus_one_is_caught(monkeypatch):
    real = AC.greedy_accept

    def one_short(tokens, target, retrieve):
        res = real(tokens, target, retrieve)
        res["frontier_row"] = res["rows"][-2] if len(res["rows"]) > 1 else res["rows"][-1]
        return res
    monkeypatch.setattr(AC, "greedy_accept", one_short)
    must_fail(PA.test_frontier_carry_a31_trace)
    must_fail(PA.test_frontier_carry_is_where_the_tree_walk_stops, 0,
              [(0,), (1,), (0, 0), (0, 1), (1, 0), (1, 1)])


def test_frontier_from_another_path_is_caught(monkeypatch):
    real = AC.greedy_accept

    def other_path(tokens, target, retrieve):
        res = real(tokens, target, retrieve)
        alt = int(retrieve[(res["best_path"] + 1) % len(retrieve)][res["accept_len"]])
        res["frontier_row"] = alt if alt >= 0 else res["frontier_row"]
        return res
    monkeypatch.setattr(AC, "greedy_accept", other_path)
    must_fail(PA.test_frontier_carry_a31_trace)


def test_budget_by_accepted_length_alone_is_caught(monkeypatch):
    """[M7.2] §0x04C: maximising E[A] per round is not maximising tokens per second."""
    monkeypatch.setattr(BU, "cost", lambda nodes, us, n: 1.0)
    must_fail(PB.test_hand_computed_four_node_case)


def test_budget_without_the_fixed_cost_is_caught(monkeypatch):
    real = BU.tree_budget
    monkeypatch.setattr(BU, "tree_budget", lambda a, nodes, us, fixed, layers: real(a, nodes, us, 0.0, layers))
    must_fail(PB.test_hand_computed_four_node_case)


def test_typical_max_instead_of_min_is_caught(monkeypatch):
    monkeypatch.setattr(TY, "threshold", lambda p, epsilon=TY.EPSILON, alpha=TY.ALPHA:
                        max(epsilon, alpha * float(np.exp(-TY.entropy(p)))))
    must_fail(PA.test_typical_threshold_closed_forms)


def test_typical_entropy_sign_is_caught(monkeypatch):
    monkeypatch.setattr(TY, "entropy", lambda p: float((p * np.log(p + TY.LOG_GUARD)).sum()))
    must_fail(PA.test_typical_threshold_closed_forms)


def test_typical_probability_sum_tie_break_is_caught(monkeypatch):
    real_log = np.log

    class FakeNp:
        def __getattr__(self, name):
            return getattr(np, name)

        @staticmethod
        def log(x):
            return x if np.ndim(x) == 0 else real_log(x)
    monkeypatch.setattr(TY, "np", FakeNp())
    must_fail(PA.test_typical_tie_break_uses_log_likelihood_not_probability_sum)


# ---------------------------------------------------------------- compaction

def test_a_rows_instead_of_a_plus_one_is_caught(monkeypatch):
    real = C.commit_plan
    monkeypatch.setattr(C, "commit_plan", lambda r, b, a, P, n, s: real(r, b, max(a - 1, 0), P, n, s))
    must_fail(PC.test_a31_commit_trace)


def test_contiguous_suffix_commit_is_caught(monkeypatch):
    real = C.commit_plan

    def contiguous(r, b, a, P, n, s):
        src, dst = real(r, b, a, P, n, s)
        return list(dst), dst
    monkeypatch.setattr(C, "commit_plan", contiguous)
    must_fail(PC.test_a31_commit_trace)


def test_in_place_reverse_copy_is_caught(monkeypatch):
    def no_snapshot(caches, retrieve, best_path, accept_len, prefix_len, n_nodes):
        for cache in caches:
            for b in range(len(prefix_len)):
                src, dst = C.commit_plan(retrieve, int(best_path[b]), int(accept_len[b]),
                                         int(prefix_len[b]), n_nodes, cache.shape[2])
                for s, d in reversed(list(zip(src, dst))):
                    cache[b][:, d, :] = cache[b][:, s, :]
        return np.array([int(p) + int(a) + 1 for p, a in zip(prefix_len, accept_len)], np.int32)
    monkeypatch.setattr(C, "kv_compact", no_snapshot)
    must_fail(PC.test_a31_commit_trace)


# ---------------------------------------------------------------- head step

def test_sigmoid_instead_of_silu_is_caught(monkeypatch):
    monkeypatch.setattr(HD, "silu", lambda x: 1.0 / (1.0 + np.exp(-np.asarray(x, np.float64))))
    must_fail(PH.test_silu_limits_not_sigmoid)
    must_fail(PH.test_zero_residual_projection_is_the_unembedding)


def test_missing_residual_is_caught(monkeypatch):
    def no_residual(h, W1, W2):
        h = np.asarray(h, np.float64)
        return np.asarray(W2, np.float64) @ HD.silu(np.asarray(W1, np.float64) @ h)
    monkeypatch.setattr(HD, "head_logits", no_residual)
    must_fail(PH.test_zero_residual_projection_is_the_unembedding)


def test_transposed_residual_projection_is_caught(monkeypatch):
    def transposed(h, W1, W2):
        h = np.asarray(h, np.float64)
        return np.asarray(W2, np.float64) @ (HD.silu(np.asarray(W1, np.float64).T @ h) + h)
    monkeypatch.setattr(HD, "head_logits", transposed)
    must_fail(PH.test_residual_projection_orientation)


def test_tie_to_higher_index_is_caught(monkeypatch):
    def higher_first(row, k):
        row = np.asarray(row, np.float64)
        order = sorted(range(row.shape[0]), key=lambda i: (-row[i], -i))
        return order[:k]
    monkeypatch.setattr(HD, "top_ranked", higher_first)
    must_fail(PH.test_ranking_matches_its_definition_by_brute_force, 0)


def test_slot_of_wrong_head_is_caught(monkeypatch):
    real = HD.head_candidates

    def shifted(h, W1, W2, root, topk):
        res = real(h, W1, W2, root, topk)
        c = res["candidates"]
        K = len(W1)
        heads = c[:, 1:].reshape(c.shape[0], K, topk)[:, ::-1].reshape(c.shape[0], -1)   # heads reversed
        res["candidates"] = np.concatenate([c[:, :1], heads], axis=1)
        return res
    monkeypatch.setattr(HD, "head_candidates", shifted)
    must_fail(PH.test_candidate_slots_feed_the_tree_gather)

