"""The C-ABI library: it loads, exports every declared symbol, and its host tree
compiler matches the oracle bit for bit (no GPU needed: compilation is host code)."""
import ctypes
import itertools
import os
import random
import re

import numpy as np
import pytest

import workloads
from conftest import ROOT, load_golden
from oracle import tree as T

lib_mod = pytest.importorskip("medusa_tree_attention_amd")
if not os.path.exists(lib_mod.LIBRARY):
    pytest.skip("libmedusa.so is not built", allow_module_level=True)


def declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn), encoding="utf-8").read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(medusa_\w+)\s*\(", text))
    return sorted(names)


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"medusa_tree_compile", "medusa_tree_attn", "medusa_accept", "medusa_kv_compact"} <= set(names)
    lib = ctypes.CDLL(lib_mod.LIBRARY)
    for name in names:
        assert hasattr(lib, name), name


def _same(lib_tree, ora):
    assert lib_tree["n_nodes"] == ora["n_nodes"]
    assert np.array_equal(lib_tree["tree_indices"], ora["tree_indices"])
    assert np.array_equal(lib_tree["depth"], ora["depth"])
    assert np.array_equal(lib_tree["parent"], ora["parent"])
    assert np.array_equal(lib_tree["tree_mask"], ora["mask_packed"])
    assert np.array_equal(lib_tree["retrieve"], ora["retrieve"])
    if "node_weight" in ora and "node_weight" in lib_tree:
        assert lib_tree["node_weight"].tobytes() == ora["node_weight"].tobytes()


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_workload_trees_match_oracle(name):
    w = workloads.WORKLOADS[name]
    spec = workloads.tree_spec(w)
    if spec["paths"] is not None:
        ora = T.compile_tree(spec["paths"], w.num_heads, w.topk)
        got = lib_mod.medusa_tree_compile(w.num_heads, w.topk, paths=spec["paths"])
    else:
        ora = T.compile_greedy(spec["rank_hit"], spec["n_nodes"])
        got = lib_mod.medusa_tree_compile(w.num_heads, w.topk, rank_hit=spec["rank_hit"],
                                          n_nodes=spec["n_nodes"])
    _same(got, ora)


def test_literal_normalisation_reading_matches_oracle():
    # the other reading of the synthetic table: each head's row normalised to one
    a = np.array([[0.6 ** k * 0.5 ** i for i in range(10)] for k in range(4)])
    a = a / a.sum(axis=1, keepdims=True)
    for n in (2, 17, 64, 200):
        _same(lib_mod.medusa_tree_compile(4, 10, rank_hit=a, n_nodes=n), T.compile_greedy(a, n))


def test_page_toys_match_oracle():
    g = load_golden("greedy_toys.json")
    for key in ("partII", "m72"):
        a = np.array(g[key]["printed"]["rank_hit"])
        K, TOPK = a.shape
        total = sum(TOPK ** d for d in range(1, K + 1))
        for n in range(1, total + 2):
            _same(lib_mod.medusa_tree_compile(K, TOPK, rank_hit=a, n_nodes=n), T.compile_greedy(a, n))
    for fixture in ("a31_round.json", "abu_tree.json"):
        gg = load_golden(fixture)
        src = gg["printed"] if "rank_paths" in gg["printed"] else gg["derived_by_hand"]
        paths = [tuple(p) for p in src["rank_paths"]]
        _same(lib_mod.medusa_tree_compile(src["num_heads"], src["topk"], paths=paths),
              T.compile_tree(paths, src["num_heads"], src["topk"]))


@pytest.mark.parametrize("seed", range(20))
def test_random_trees_match_oracle(seed):
    rng = random.Random(seed)
    K, TOPK = rng.randint(1, 5), rng.randint(1, 6)
    every = [p for d in range(1, K + 1) for p in itertools.product(range(TOPK), repeat=d)]
    # random prefix-closed family, handed over in a shuffled order
    chosen = set()
    for p in rng.sample(every, min(len(every), rng.randint(0, 70))):
        for k in range(1, len(p) + 1):
            chosen.add(p[:k])
    paths = list(chosen)
    rng.shuffle(paths)
    _same(lib_mod.medusa_tree_compile(K, TOPK, paths=paths), T.compile_tree(paths, K, TOPK))
    # greedy growth with ties: ranks drawn from a few dyadic values
    a = np.array([[rng.choice([0.5, 0.25, 0.125, 0.0, 1.0]) for _ in range(TOPK)] for _ in range(K)])
    n = rng.randint(1, len(every) + 1)
    _same(lib_mod.medusa_tree_compile(K, TOPK, rank_hit=a, n_nodes=n), T.compile_greedy(a, n))


@pytest.mark.parametrize("kw,code", [
    (dict(num_heads=2, topk=2, paths=[(0, 1)]), "MEDUSA_ENOT_PREFIX_CLOSED"),
    (dict(num_heads=2, topk=2, paths=[(0,), (0, 2)]), "MEDUSA_EINVAL"),
    (dict(num_heads=1, topk=2, paths=[(0,), (0, 0)]), "MEDUSA_EINVAL"),
    (dict(num_heads=2, topk=2, paths=[(1,), (1,)]), "MEDUSA_EINVAL"),
    (dict(num_heads=1, topk=2, rank_hit=[[0.5, 0.4]], n_nodes=4), "MEDUSA_ECAPACITY"),
    (dict(num_heads=1, topk=2, rank_hit=[[0.5, np.nan]], n_nodes=2), "MEDUSA_EINVAL"),
    (dict(num_heads=1, topk=2, rank_hit=[[1.5, 0.4]], n_nodes=2), "MEDUSA_EINVAL"),
    (dict(num_heads=1, topk=2, rank_hit=[[0.5, 0.4]], n_nodes=0), "MEDUSA_EINVAL"),
    (dict(num_heads=0, topk=2, paths=[]), "MEDUSA_EINVAL"),
])
def test_invalid_specs_return_status(kw, code):
    with pytest.raises(lib_mod.MedusaError) as e:
        lib_mod.medusa_tree_compile(**kw)
    assert e.value.name == code


def test_small_buffers_are_rejected_without_writes():
    from medusa_tree_attention_amd import _binding as B
    lib = B.load()
    paths = [(0,), (1,), (0, 0)]
    lens = np.array([1, 1, 2], np.int32)
    flat = np.array([0, 1, 0, 0], np.int32)
    spec = B.TreeSpec(num_heads=2, topk=2, n_paths=3,
                      path_len=lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                      path_ranks=flat.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    bufs = [np.full(8, 77, np.int32) for _ in range(4)]
    mask = np.full(8, 77, np.uint64)
    tree = B.Tree(n_nodes=3, n_paths=8, path_width=8, mask_words=8)   # 3 < 4 rows needed
    tree.tree_indices, tree.depth, tree.parent, tree.retrieve_indices = [
        b.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) for b in bufs]
    tree.tree_mask = mask.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))
    assert lib.medusa_tree_compile(ctypes.byref(spec), ctypes.byref(tree)) == -5
    assert all((b == 77).all() for b in bufs) and (mask == 77).all()
    assert len(paths) == 3
