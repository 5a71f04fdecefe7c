"""Pins of the oracle tree attention.

Independent references used here:
* RoPE in its complex form, z = x1 + i*x2 multiplied by exp(i * pos * theta);
* torch's CPU scaled_dot_product_attention (float64) on an ordinary causal
  sequence, the textbook routine the tree mask must reproduce per path.
"""
import itertools

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as A
from oracle import tree as T


def rope_complex(x, pos, base):
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    theta = np.array([base ** (-2.0 * i / d) for i in range(d // 2)])
    z = (x[..., : d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * pos * theta)
    return np.concatenate([z.real, z.imag], axis=-1)


def sdpa_causal(q_rows, keys, values):
    """Ordinary causal attention: query i is sequence position L - n + i of an L-row sequence."""
    q = torch.from_numpy(np.asarray(q_rows, np.float64))[None, None]
    k = torch.from_numpy(np.asarray(keys, np.float64))[None, None]
    v = torch.from_numpy(np.asarray(values, np.float64))[None, None]
    n, L = q.shape[2], k.shape[2]
    mask = torch.ones(n, L, dtype=torch.bool).tril(diagonal=L - n)
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    return out[0, 0].numpy()


def _inputs(rng, B, N, Hq, Hkv, d, P):
    return dict(q=rng.standard_normal((B, N, Hq, d)), k_new=rng.standard_normal((B, N, Hkv, d)),
                v_new=rng.standard_normal((B, N, Hkv, d)),
                k_cache=rng.standard_normal((B, Hkv, P + N, d)),
                v_cache=rng.standard_normal((B, Hkv, P + N, d)))


# ---------------------------------------------------------------- RoPE

def test_rope_matches_complex_form_and_properties():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 64))
    for pos in (0, 1, 7, 4096, 8259):
        got = A.rope(x, pos, 10000.0)
        assert np.allclose(got, rope_complex(x, pos, 10000.0), atol=1e-12)
        pairs = lambda y: y[:, :32] ** 2 + y[:, 32:] ** 2
        assert np.allclose(pairs(got), pairs(x), atol=1e-12)   # a rotation per pair
    assert np.allclose(A.rope(x, 0, 10000.0), x)
    # d = 2: theta_0 = 1, a plain rotation by pos radians
    assert np.allclose(A.rope([1.0, 0.0], 3, 10000.0), [np.cos(3.0), np.sin(3.0)])
    # relative-position property: <R(m)q, R(n)k> depends on m - n only
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    ref = A.rope(q, 10, 10000.0) @ A.rope(k, 4, 10000.0)
    assert A.rope(q, 1010, 10000.0) @ A.rope(k, 1004, 10000.0) == pytest.approx(ref, abs=1e-9)


# ---------------------------------------------------------------- special cases with textbook answers

def test_root_only_is_single_query_decode():
    rng = np.random.default_rng(1)
    x = _inputs(rng, 1, 1, 2, 1, 16, 9)
    out, sk, sv = A.tree_attention(**x, prefix_len=[9], depth=[0], parent=[-1], rope_base=10000.0)
    keys = np.concatenate([x["k_cache"][0, 0, :9], rope_complex(x["k_new"][0, 0, 0], 9, 1e4)[None]])
    vals = np.concatenate([x["v_cache"][0, 0, :9], x["v_new"][0, 0, 0][None]])
    for h in range(2):
        q = rope_complex(x["q"][0, 0, h], 9, 1e4)
        assert np.allclose(out[0, 0, h], sdpa_causal(q[None], keys, vals)[0], atol=1e-12)
    assert np.allclose(sk[0, 0, 0], keys[-1]) and np.allclose(sv[0, 0, 0], vals[-1])


def test_chain_tree_is_ordinary_causal_attention():
    rng = np.random.default_rng(2)
    t = T.compile_tree(workloads.cartesian_paths((1, 1, 1)), 3, 1)
    P, d = 11, 32
    x = _inputs(rng, 1, t["n_nodes"], 1, 1, d, P)
    out, _, _ = A.tree_attention(**x, prefix_len=[P], depth=t["depth"], parent=t["parent"],
                                 rope_base=500.0)
    n = t["n_nodes"]
    keys = np.concatenate([x["k_cache"][0, 0, :P]] +
                          [rope_complex(x["k_new"][0, u, 0], P + u, 500.0)[None] for u in range(n)])
    vals = np.concatenate([x["v_cache"][0, 0, :P], x["v_new"][0, :, 0]])
    qs = np.stack([rope_complex(x["q"][0, u, 0], P + u, 500.0) for u in range(n)])
    assert np.allclose(out[0, :, 0], sdpa_causal(qs, keys, vals), atol=1e-12)


def _prefix_closed_sets(K, TOPK, max_size):
    every = [p for d in range(1, K + 1) for p in itertools.product(range(TOPK), repeat=d)]
    for size in range(0, max_size + 1):
        for combo in itertools.combinations(every, size):
            s = set(combo)
            if all(p[:k] in s for p in combo for k in range(1, len(p))):
                yield list(combo)


def test_every_small_tree_matches_per_path_causal_attention():
    """Brute force: every prefix-closed tree with at most 5 rows (K <= 3, TOPK <= 2)."""
    rng = np.random.default_rng(3)
    trees = list(_prefix_closed_sets(3, 2, 4))
    assert len(trees) > 40
    for paths in trees:
        t = T.compile_tree(paths, 3, 2)
        n, P, d, Hq, Hkv = t["n_nodes"], int(rng.integers(0, 6)), 8, 4, 2
        x = _inputs(rng, 1, n, Hq, Hkv, d, P)
        out, _, _ = A.tree_attention(**x, prefix_len=[P], depth=t["depth"], parent=t["parent"],
                                     rope_base=10000.0)
        rows = [()] + t["paths"]
        for u in range(n):
            # the path's rows, found from the path tuples rather than the parent array
            chain = [rows.index(rows[u][:k]) for k in range(len(rows[u]) + 1)]
            for h in range(Hq):
                g = h // (Hq // Hkv)
                keys = np.concatenate([x["k_cache"][0, g, :P]] + [
                    rope_complex(x["k_new"][0, v, g], P + len(rows[v]), 1e4)[None] for v in chain])
                vals = np.concatenate([x["v_cache"][0, g, :P]] + [x["v_new"][0, v, g][None] for v in chain])
                q = rope_complex(x["q"][0, u, h], P + len(rows[u]), 1e4)
                ref = sdpa_causal(q[None], keys, vals)[0]
                assert np.allclose(out[0, u, h], ref, atol=1e-12), (paths, u, h)


def test_sibling_subtrees_are_equivariant():
    rng = np.random.default_rng(4)
    t = T.compile_tree(workloads.cartesian_paths((2, 2)), 2, 2)
    P = 6
    x = _inputs(rng, 1, 7, 2, 2, 16, P)
    out, _, _ = A.tree_attention(**x, prefix_len=[P], depth=t["depth"], parent=t["parent"], rope_base=1e4)
    perm = [0, 2, 1, 5, 6, 3, 4]      # swap subtree (0) <-> (1)
    y = dict(x)
    for key in ("q", "k_new", "v_new"):
        y[key] = x[key][:, perm]
    out2, _, _ = A.tree_attention(**y, prefix_len=[P], depth=t["depth"], parent=t["parent"], rope_base=1e4)
    assert np.allclose(out2[0], out[0, perm], atol=1e-12)


def test_batch_rows_use_their_own_prefix_length():
    rng = np.random.default_rng(5)
    t = T.compile_tree(workloads.cartesian_paths((2,)), 1, 2)
    x = _inputs(rng, 2, 3, 1, 1, 8, 7)
    out, _, _ = A.tree_attention(**x, prefix_len=[7, 3], depth=t["depth"], parent=t["parent"], rope_base=1e4)
    solo = {k: v[1:2] for k, v in x.items()}
    out1, _, _ = A.tree_attention(**solo, prefix_len=[3], depth=t["depth"], parent=t["parent"], rope_base=1e4)
    assert np.allclose(out[1], out1[0], atol=1e-12)


def test_rows_subset_equals_full():
    rng = np.random.default_rng(6)
    t = T.compile_tree(workloads.cartesian_paths((2, 2)), 2, 2)
    x = _inputs(rng, 1, 7, 4, 2, 8, 5)
    full, _, _ = A.tree_attention(**x, prefix_len=[5], depth=t["depth"], parent=t["parent"], rope_base=1e4)
    part, _, _ = A.tree_attention(**x, prefix_len=[5], depth=t["depth"], parent=t["parent"], rope_base=1e4,
                                  rows=[(0, 6, 3), (0, 2, 0)])
    assert np.allclose(part[0, 6, 3], full[0, 6, 3]) and np.allclose(part[0, 2, 0], full[0, 2, 0])
    assert np.isnan(part[0, 1, 1]).all()
