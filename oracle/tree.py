"""Oracle: compile a rank-path tree into its flattened buffers.

TEST INFRASTRUCTURE (see the package docstring).

Follows [M7.2] (title in ``oracle/__init__``):

* §0x01B "Coordinate Domains Must Not Alias": candidate slot
  slot(j, r) = 1 + j*TOPK + r with slot 0 the ordinary LM root; logical
  position = prefix length + depth, depth(root) = 0.
* §0x04A "Sparse Tree Construction": prefix closure; the canonical order
  sorts non-root paths by (length, path); row(empty) = 0 and
  row(p) = 1 + index in that order; tree_indices[row(p)] = 1+(len-1)*TOPK+p[-1];
  M[u, v] = 1 iff path(v) is a prefix of path(u); depth = len(path);
  retrieve rows list the maximal paths [0, row(p[:1]), ..., row(p)] padded
  with a negative sentinel.
* §0x04B "Calibration Probabilities And Expected Accepted Length": the path
  weight w(r_1..r_d) = prod_j a_j^(r_j) and the objective sum_u w(u).
* §0x04C "Greedy Frontier Search And Its Boundary": the frontier loop.
  [PartII] Part 3 Step 3 states the same loop ("add the highest-scoring node
  whose parent is already present").

Readings where the pages are silent:

* Ties in the greedy argmax are broken by the key (-w, len(p), p): higher
  weight, then the shorter path, then the lexicographically smaller one.
* Maximal retrieve rows are listed by ascending canonical row of their leaf;
  the sentinel is -1.
* Weights are products taken left to right in binary64.
"""
from __future__ import annotations

import itertools

import numpy as np


class TreeError(ValueError):
    """An invalid tree specification; ``code`` names the violated rule."""

    def __init__(self, code: str, msg: str):
        super().__init__(f"{code}: {msg}")
        self.code = code


def validate_paths(paths, num_heads: int, topk: int) -> list:
    """Check a rank-path family: ranks < TOPK, 1 <= len <= K, unique, prefix-closed."""
    if num_heads < 1 or topk < 1:
        raise TreeError("EINVAL", "num_heads and topk must be positive")
    out = [tuple(int(r) for r in p) for p in paths]
    seen = set()
    for p in out:
        if not 1 <= len(p) <= num_heads:
            raise TreeError("EINVAL", f"path {p} length outside 1..{num_heads}")
        if any(r < 0 or r >= topk for r in p):
            raise TreeError("EINVAL", f"path {p} has a rank outside 0..{topk - 1}")
        if p in seen:
            raise TreeError("EINVAL", f"duplicate path {p}")
        seen.add(p)
    # [M7.2] §0x04A: if (0,1,0) exists, (0) and (0,1) must exist too.
    for p in out:
        for k in range(1, len(p)):
            if p[:k] not in seen:
                raise TreeError("ENOT_PREFIX_CLOSED", f"{p} lacks its prefix {p[:k]}")
    return out


def path_weight(rank_hit, path) -> float:
    """w(r_1..r_d) = a_1^(r_1) * ... * a_d^(r_d), multiplied left to right ([M7.2] §0x04B)."""
    w = 1.0
    for depth, rank in enumerate(path):
        w = w * float(rank_hit[depth][rank])
    return w


def _order_key(rank_hit, path):
    return (-path_weight(rank_hit, path), len(path), tuple(path))


def _check_rank_hit(rank_hit):
    a = np.asarray(rank_hit, dtype=np.float64)
    if a.ndim != 2 or a.size == 0:
        raise TreeError("EINVAL", "rank_hit must be a non-empty [K, TOPK] table")
    if not np.all(np.isfinite(a)) or np.any(a < 0.0) or np.any(a > 1.0):
        raise TreeError("EINVAL", "rank_hit entries must be probabilities in [0, 1]")
    return a


def greedy_frontier(rank_hit, budget: int) -> list:
    """[M7.2] §0x04C: grow a prefix-closed path set one max-weight frontier path at a time.

    Returns the admitted non-root paths in admission order.
    """
    a = _check_rank_hit(rank_hit)
    num_heads, topk = a.shape
    total = sum(topk ** depth for depth in range(1, num_heads + 1))
    if budget < 0 or budget > total:
        raise TreeError("ECAPACITY", f"budget {budget} outside 0..{total}")
    tree = []
    frontier = [(r,) for r in range(topk)]
    while len(tree) < budget:
        best = min(frontier, key=lambda p: _order_key(a, p))
        frontier.remove(best)
        tree.append(best)
        if len(best) < num_heads:
            for r in range(topk):
                frontier.append(best + (r,))
    return tree


def greedy_top_b(rank_hit, budget: int) -> list:
    """Second, independent selection: sort every rank tuple by (-w, len, p) and keep the first ``budget``.

    Equal to ``greedy_frontier`` whenever every a <= 1, because a child then
    never outranks its parent.
    """
    a = _check_rank_hit(rank_hit)
    num_heads, topk = a.shape
    every = [p for depth in range(1, num_heads + 1)
             for p in itertools.product(range(topk), repeat=depth)]
    if budget < 0 or budget > len(every):
        raise TreeError("ECAPACITY", f"budget {budget} outside 0..{len(every)}")
    every.sort(key=lambda p: _order_key(a, p))
    return every[:budget]


def compile_tree(paths, num_heads: int, topk: int, rank_hit=None) -> dict:
    """Compile a prefix-closed rank-path family into the four buffers of [M7.2] §0x04A.

    Returns a dict with
      paths        canonical non-root paths (row r holds paths[r-1])
      tree_indices int32 [N]   candidate slot of each row (0 for the root)
      depth        int32 [N]   |path(u)|; logical position = prefix + depth
      parent       int32 [N]   row of path(u)[:-1]; -1 for the root
      mask         bool  [N,N] M[u, v] = path(v) is a prefix of path(u)
      mask_words   int
      mask_packed  uint64 [N, mask_words]  bit v%64 of word v//64 of row u
      retrieve     int32 [n_paths, W]      maximal paths, -1 padded, W = max depth + 1
      node_weight  float64 [N] (only when rank_hit is given; w(root) = 1)
    """
    canon = sorted(validate_paths(paths, num_heads, topk), key=lambda p: (len(p), p))
    row = {(): 0}
    for i, p in enumerate(canon):
        row[p] = 1 + i
    n = 1 + len(canon)
    rows_paths = [()] + canon

    tree_indices = np.zeros(n, np.int32)
    depth = np.zeros(n, np.int32)
    parent = np.full(n, -1, np.int32)
    for p in canon:
        u = row[p]
        tree_indices[u] = 1 + (len(p) - 1) * topk + p[-1]
        depth[u] = len(p)
        parent[u] = row[p[:-1]]

    mask = np.zeros((n, n), dtype=bool)
    for u, pu in enumerate(rows_paths):
        for v, pv in enumerate(rows_paths):
            mask[u, v] = len(pv) <= len(pu) and pu[:len(pv)] == pv
    words = (n + 63) // 64
    packed = np.zeros((n, words), np.uint64)
    for u in range(n):
        for v in range(n):
            if mask[u, v]:
                packed[u, v // 64] |= np.uint64(1) << np.uint64(v % 64)

    has_child = set(parent[1:].tolist())
    leaves = [u for u in range(n) if u not in has_child]
    width = int(depth.max()) + 1
    retrieve = np.full((len(leaves), width), -1, np.int32)
    for i, u in enumerate(leaves):
        p = rows_paths[u]
        chain = [row[p[:k]] for k in range(len(p) + 1)]
        retrieve[i, :len(chain)] = chain

    out = {"paths": canon, "tree_indices": tree_indices, "depth": depth, "parent": parent,
           "mask": mask, "mask_words": words, "mask_packed": packed, "retrieve": retrieve,
           "n_nodes": n, "n_paths": len(leaves), "path_width": width, "topk": topk,
           "num_heads": num_heads}
    if rank_hit is not None:
        a = _check_rank_hit(rank_hit)
        out["node_weight"] = np.array([path_weight(a, p) for p in rows_paths], np.float64)
    return out


def compile_greedy(rank_hit, n_nodes: int) -> dict:
    """Grow ``n_nodes - 1`` paths with the frontier loop, then compile them (row count includes the root)."""
    a = _check_rank_hit(rank_hit)
    if n_nodes < 1:
        raise TreeError("EINVAL", "n_nodes counts the root and must be >= 1")
    chosen = greedy_frontier(a, n_nodes - 1)
    num_heads, topk = a.shape
    return compile_tree(chosen, num_heads, topk, rank_hit=a)


def tree_tokens(tree: dict, candidates_row) -> np.ndarray:
    """Per-row tokens: token[u] = candidates[tree_indices[u]] ([M7.2] §0x04A candidate gather)."""
    cand = np.asarray(candidates_row)
    return cand[tree["tree_indices"]].astype(np.int32)


def positions(tree: dict, prefix_len: int) -> np.ndarray:
    """Logical positions prefix_len + depth(u) ([M7.2] §0x01B)."""
    return (prefix_len + tree["depth"]).astype(np.int64)


def expected_accept_length(tree: dict) -> float:
    """The calibration objective sum over non-root nodes of w(u) ([M7.2] §0x04B)."""
    return float(tree["node_weight"][1:].sum())
