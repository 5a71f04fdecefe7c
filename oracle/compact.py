"""Oracle: commit the winning path's K/V rows with a snapshot.

TEST INFRASTRUCTURE (see the package docstring).

Follows [M7.2] §0x06A "Accepted Suffix Length Is Not Published Row Count"
(G = a + 1; u_j = retrieve[p*, j], source s_j = P + u_j, destination
d_j = P + j), §0x06B "Worked Gather-And-Compact Trace" (gather a snapshot
first because source and destination rows can overlap, then copy;
current_length = P + G) and §0x06D "Publication Invariants And Failure
Semantics" (validate before mutating; rows past the new length keep their
stale bytes).  [Chai] section "一次完整解码迭代" step 5 describes the same copy.
"""
from __future__ import annotations

import numpy as np


class CompactError(ValueError):
    pass


def commit_plan(retrieve, best_path: int, accept_len: int, prefix_len: int,
                n_nodes: int, s_max: int):
    """Validated (sources, destinations) of one sequence; raises before anything is mutated."""
    retrieve = np.asarray(retrieve)
    n_paths, width = retrieve.shape
    if not 0 <= best_path < n_paths:
        raise CompactError("best path out of range")
    if not 0 <= accept_len < width:
        raise CompactError("accept length out of range")
    G = accept_len + 1
    rows = [int(r) for r in retrieve[best_path, :G]]
    if any(r < 0 or r >= n_nodes for r in rows):
        raise CompactError("retrieve row is a sentinel or out of range")
    if prefix_len < 0 or prefix_len + n_nodes > s_max:
        raise CompactError("staged rows exceed the cache")
    src = [prefix_len + r for r in rows]
    dst = [prefix_len + j for j in range(G)]
    return src, dst


def kv_compact(caches, retrieve, best_path, accept_len, prefix_len, n_nodes: int):
    """Compact every layer's K and V cache in place; returns the new prefix lengths.

    caches: list of arrays [B, Hkv, S_max, d] (K and V of every layer).
    All sequences are validated before any cache is touched.
    """
    B = len(prefix_len)
    s_max = caches[0].shape[2]
    plans = [commit_plan(retrieve, int(best_path[b]), int(accept_len[b]),
                         int(prefix_len[b]), n_nodes, s_max) for b in range(B)]
    for cache in caches:
        for b, (src, dst) in enumerate(plans):
            snapshot = cache[b][:, src, :].copy()
            cache[b][:, dst, :] = snapshot
    return np.array([int(prefix_len[b]) + int(accept_len[b]) + 1 for b in range(B)], np.int32)
