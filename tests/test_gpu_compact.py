"""K/V compaction on the GPU: bit-exact against the oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import medusa_tree_attention_amd as M
from oracle import compact as C

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from conftest import load_golden  # noqa: E402
from gpu_support import announce, dev  # noqa: E402


def a31_tree():
    g = load_golden("a31_round.json")
    pr = g["printed"]
    lib = M.medusa_tree_compile(pr["num_heads"], pr["topk"], paths=[tuple(p) for p in pr["rank_paths"]])
    return g, lib


def run_compact(caches_k, caches_v, tree, best, alen, prefix, status_init=0):
    status = torch.full((1,), status_init, dtype=torch.int32, device="cuda")
    pl = dev(np.asarray(prefix, np.int32))
    M.medusa_kv_compact(caches_k, caches_v, dev(tree["retrieve"]), dev(np.asarray(best, np.int32)),
                        dev(np.asarray(alen, np.int32)), pl, tree["n_nodes"], status)
    torch.cuda.synchronize()
    return int(status.item()), pl.cpu().numpy()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_a31_commit_trace(dtype):
    announce(f"compact A31 trace {dtype}")
    g, tree = a31_tree()
    c, P = g["printed"]["commit"], g["printed"]["prefix_len"]
    S = P + tree["n_nodes"]
    # row r of every cache holds the value r (exact in bf16 for r < 256)
    base = np.broadcast_to(np.arange(S, dtype=np.float32)[None, None, :, None], (1, 2, S, 64)).copy()
    k = [dev(base, dtype) for _ in range(2)]
    v = [dev(base + 100, dtype) for _ in range(2)]
    best = g["derived_by_hand"]["commit_path_index_ascending_leaves"]
    status, pl = run_compact(k, v, tree, [best], [c["accept_len"]], [P])
    assert status == 0 and pl.tolist() == [c["new_length"]]
    for t, off in [(k[0], 0), (k[1], 0), (v[0], 100), (v[1], 100)]:
        rows = t[0, :, :, 0].float().cpu().numpy()
        assert rows[:, P:P + c["G"]].tolist() == [[s + off for s in c["source_rows"]]] * 2
        assert rows[:, :P].tolist() == [[r + off for r in range(P)]] * 2
        assert rows[:, P + c["G"]:].tolist() == [[r + off for r in range(P + c["G"], S)]] * 2


@pytest.mark.parametrize("n_layers,dtype,d", [(1, torch.bfloat16, 128), (3, torch.float32, 64),
                                              (40, torch.bfloat16, 128)])
def test_random_plans_match_oracle(n_layers, dtype, d):
    announce(f"compact random plans layers={n_layers} {dtype} d={d}")
    rng = np.random.default_rng(n_layers)
    paths = ([(a,) for a in range(4)] + [(a, b) for a in range(4) for b in range(4)] +
             [(0, 0, c) for c in range(4)] + [(0, 0, 0, 0)])
    tree = M.medusa_tree_compile(4, 4, paths=paths)
    B, Hkv, N = 3, 2, tree["n_nodes"]
    prefix = [0, 45, 300]
    S = max(prefix) + N + 3
    caches = [rng.standard_normal((B, Hkv, S, d)).astype(np.float32) for _ in range(2 * n_layers)]
    if dtype == torch.bfloat16:
        caches = [torch.from_numpy(c).to(torch.bfloat16).float().numpy() for c in caches]
    best = [int(rng.integers(0, tree["n_paths"])) for _ in range(B)]
    alen = [int(rng.integers(0, (tree["retrieve"][p] >= 0).sum())) for p in best]
    k = [dev(c, dtype) for c in caches[:n_layers]]
    v = [dev(c, dtype) for c in caches[n_layers:]]
    status, pl = run_compact(k, v, tree, best, alen, prefix)
    assert status == 0
    new_len = C.kv_compact(caches, tree["retrieve"], best, alen, prefix, N)
    assert pl.tolist() == new_len.tolist()
    for got, ref in zip(k + v, caches):
        assert np.array_equal(got.float().cpu().numpy(), ref)


@pytest.mark.parametrize("best,alen,prefix,code", [
    ([0, 9], [1, 0], [5, 5], -1),      # best path out of range
    ([0, 0], [1, 3], [5, 5], -1),      # accept length beyond the path width
    ([0, 0], [2, 0], [5, 5], -1),      # path 0 = [0, 1, -1]: a sentinel among the published rows
    ([0, 0], [1, 0], [5, 9], -3),      # staged rows beyond the cache
])
def test_invalid_plans_store_nothing(best, alen, prefix, code):
    announce(f"compact invalid plan {best} {alen} {prefix}")
    tree = M.medusa_tree_compile(2, 2, paths=[(0,), (1,), (1, 0)])    # retrieve [[0,1,-1],[0,2,3]]
    S = 5 + tree["n_nodes"] + 1
    base = np.random.default_rng(0).standard_normal((2, 1, S, 64)).astype(np.float32)
    k, v = [dev(base)], [dev(base * 2)]
    status, pl = run_compact(k, v, tree, best, alen, prefix)
    assert status == code and pl.tolist() == prefix
    assert np.array_equal(k[0].cpu().numpy(), base) and np.array_equal(v[0].cpu().numpy(), base * 2)


def test_sticky_status_skips_compaction():
    announce("compact with a failed round")
    tree = M.medusa_tree_compile(2, 2, paths=[(0,), (1,), (1, 0)])
    base = np.random.default_rng(1).standard_normal((1, 1, 12, 64)).astype(np.float32)
    k, v = [dev(base)], [dev(base)]
    status, pl = run_compact(k, v, tree, [1], [2], [5], status_init=-1)
    assert status == -1 and pl.tolist() == [5]
    assert np.array_equal(k[0].cpu().numpy(), base)
