"""Seeded synthetic inputs for one Medusa tree-verification round.

This module only draws numbers and lays them out.  It performs no step of the
method: no tree growth, no RoPE, no attention, no acceptance and no KV
compaction.  The tests, ``bench.py`` and ``__graft_entry__.smoke()`` use it to
feed the HIP library and the CPU oracle the *same* inputs; neither side
imports the other.

Every workload is synthetic.  The pages measure nothing on a public dataset
for this path; the rank-hit table below stands in for calibration statistics
and N(0, 1) logits stand in for target-model logits.

Draw order per workload (one ``numpy.random.Generator(PCG64(seed))``):
cache-K, cache-V, Q, K_new, V_new, candidates, then logits or target ids.
bf16 tensors are round-to-nearest-even conversions of float32 draws; the
values handed to both sides are those rounded values.
"""
from __future__ import annotations

import dataclasses
import itertools
from typing import Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "rank_hit_table", "cartesian_paths",
    "round_to_dtype", "draw_round", "plant_acceptance", "tree_spec", "draw_heads",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and tree recipe of one verification round."""

    name: str
    seed: int
    B: int                  # sequences in the batch
    Hq: int                 # query heads
    Hkv: int                # key/value heads
    d: int                  # head dimension d_h
    P: int                  # committed prefix rows per sequence
    dtype: str              # "f32" or "bf16" storage of Q/K/V/cache/output
    num_heads: int          # Medusa heads K (= maximum tree depth)
    topk: int               # per-head candidate pool width TOPK
    tree: str               # "cartesian" (explicit paths) or "greedy" (rank-hit growth)
    branching: Optional[tuple] = None   # Cartesian branching per depth
    n_nodes: Optional[int] = None       # greedy: rows including the root
    vocab: int = 32000
    use_logits: bool = True             # False: target next-token ids are given directly
    rope_base: float = 10000.0
    slack: int = 0                      # extra cache rows beyond P + N

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv


# The five round shapes.  "tiny" is small enough for the oracle to finish in
# well under a second; "batched" is the four-sequence, context-4096, 64-node
# tree shape used for throughput.
WORKLOADS = {
    "tiny": Workload("tiny", seed=0, B=1, Hq=1, Hkv=1, d=64, P=128, dtype="f32",
                     num_heads=2, topk=2, tree="cartesian", branching=(2, 2),
                     vocab=16, use_logits=False),
    "llama7b": Workload("llama7b", seed=1, B=1, Hq=32, Hkv=32, d=128, P=2048,
                        dtype="bf16", num_heads=4, topk=10, tree="greedy", n_nodes=64),
    "gqa8b": Workload("gqa8b", seed=2, B=1, Hq=32, Hkv=8, d=128, P=8192,
                      dtype="bf16", num_heads=4, topk=10, tree="greedy", n_nodes=64),
    "wide": Workload("wide", seed=3, B=1, Hq=32, Hkv=32, d=128, P=4096, dtype="bf16",
                     num_heads=4, topk=4, tree="cartesian", branching=(4, 4, 4, 4)),
    "batched": Workload("batched", seed=4, B=4, Hq=32, Hkv=8, d=128, P=4096,
                        dtype="bf16", num_heads=4, topk=10, tree="greedy", n_nodes=64),
}


def rank_hit_table(num_heads: int, topk: int, head_decay: float = 0.6,
                   rank_decay: float = 0.5) -> np.ndarray:
    """Synthetic exact-rank hit probabilities a_k^(i), shape [num_heads, topk].

    a_k^(i) = head_decay**k * rank_decay**i / sum_{r<topk} rank_decay**r with
    zero-based head k and rank i: the rank profile of each head is normalised
    to one and scaled by head_decay**k, so later heads hit less often and
    rank 0 beats rank 1 beats rank 2, the two asymmetries the calibration
    statistics are described to have.
    """
    ranks = np.array([rank_decay ** i for i in range(topk)], dtype=np.float64)
    norm = float(sum(rank_decay ** i for i in range(topk)))
    table = np.empty((num_heads, topk), dtype=np.float64)
    for k in range(num_heads):
        for i in range(topk):
            table[k, i] = (head_decay ** k) * ranks[i] / norm
    return table


def cartesian_paths(branching) -> list:
    """All rank tuples of a regular tree: depth i keeps ranks 0..branching[i]-1."""
    paths = []
    for depth in range(1, len(branching) + 1):
        for combo in itertools.product(*[range(b) for b in branching[:depth]]):
            paths.append(tuple(combo))
    return paths


def tree_spec(w: Workload) -> dict:
    """Arguments describing the workload's tree (explicit paths or rank-hit growth)."""
    if w.tree == "cartesian":
        return {"num_heads": w.num_heads, "topk": w.topk,
                "paths": cartesian_paths(w.branching), "rank_hit": None, "n_nodes": None}
    return {"num_heads": w.num_heads, "topk": w.topk, "paths": None,
            "rank_hit": rank_hit_table(w.num_heads, w.topk), "n_nodes": w.n_nodes}


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype; returns float32 holding exact values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype != "bf16":
        raise ValueError(dtype)
    bits = x.view(np.uint32)
    # round-to-nearest-even on the upper 16 bits; for finite inputs the sum stays below
    # 2^32 (the largest finite pattern 0xFF7FFFFF + 0x8000 = 0xFF807FFF)
    out = (bits >> 16) & np.uint32(1)
    out += np.uint32(0x7FFF)
    out += bits
    out &= np.uint32(0xFFFF0000)
    return out.view(np.float32)


def _node_count(w: Workload) -> int:
    if w.tree == "greedy":
        return w.n_nodes
    total, prod = 1, 1
    for b in w.branching:
        prod *= b
        total += prod
    return total


def draw_round(w: Workload, seed: Optional[int] = None, prefix_len=None) -> dict:
    """Draw every per-round input of workload ``w``.

    Returns float32 arrays holding dtype-exact values (bf16-representable for
    bf16 workloads) and int32 index arrays:

    k_cache, v_cache  [B, Hkv, S_max, d]  rows [0, P_b) drawn ~N(0,1), rest 0
    q                 [B, N, Hq, d]
    k_new, v_new      [B, N, Hkv, d]
    candidates        [B, 1 + K*TOPK]     slot 0 = root, slot 1+k*TOPK+r = head k rank r
    logits            [B, N, V] float32 ~N(0,1)   (when w.use_logits)
    target_ids        [B, N] int32 uniform [0,V)  (otherwise)
    prefix_len        [B] int32
    """
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    N = _node_count(w)
    P = np.full(w.B, w.P, dtype=np.int32) if prefix_len is None else np.asarray(prefix_len, np.int32)
    s_max = int(P.max()) + N + w.slack
    kc = np.zeros((w.B, w.Hkv, s_max, w.d), np.float32)
    vc = np.zeros_like(kc)
    pmax = int(P.max())
    kdraw = rng.standard_normal((w.B, w.Hkv, pmax, w.d), dtype=np.float32)
    vdraw = rng.standard_normal((w.B, w.Hkv, pmax, w.d), dtype=np.float32)
    for b in range(w.B):
        kc[b, :, :P[b]] = kdraw[b, :, :P[b]]
        vc[b, :, :P[b]] = vdraw[b, :, :P[b]]
    q = rng.standard_normal((w.B, N, w.Hq, w.d), dtype=np.float32)
    k_new = rng.standard_normal((w.B, N, w.Hkv, w.d), dtype=np.float32)
    v_new = rng.standard_normal((w.B, N, w.Hkv, w.d), dtype=np.float32)
    n_slots = 1 + w.num_heads * w.topk
    cand = np.empty((w.B, n_slots), np.int32)
    for b in range(w.B):
        cand[b, 0] = rng.integers(0, w.vocab)
        for k in range(w.num_heads):
            # a head's top-k ids are distinct; rank order = draw order
            cand[b, 1 + k * w.topk: 1 + (k + 1) * w.topk] = rng.choice(w.vocab, w.topk, replace=False)
    out = {
        "k_cache": round_to_dtype(kc, w.dtype), "v_cache": round_to_dtype(vc, w.dtype),
        "q": round_to_dtype(q, w.dtype), "k_new": round_to_dtype(k_new, w.dtype),
        "v_new": round_to_dtype(v_new, w.dtype), "candidates": cand,
        "prefix_len": P, "S_max": s_max, "N": N, "vocab": w.vocab,
    }
    if w.use_logits:
        out["logits"] = rng.standard_normal((w.B, N, w.vocab), dtype=np.float32)
        out["target_ids"] = None
    else:
        out["logits"] = None
        out["target_ids"] = rng.integers(0, w.vocab, size=(w.B, N)).astype(np.int32)
    return out


def plant_acceptance(rng: np.random.Generator, inputs: dict, tokens: np.ndarray,
                     retrieve: np.ndarray, parent: np.ndarray, b: int,
                     path: int, depth: int) -> None:
    """Edit one sequence's logits (or target ids) so that ``path`` matches to ``depth``.

    For j < depth the target's top token at row retrieve[path][j] is set to
    the token of row retrieve[path][j+1]; at the stopping row no child's token
    is the top token.  ``tokens`` are the per-row tree tokens of sequence b.
    Inputs are edited in place; this only moves values around.
    """
    rows = [int(r) for r in retrieve[path] if r >= 0]
    assert 0 <= depth < len(rows)
    children = {}
    for v, p in enumerate(parent):
        if p >= 0:
            children.setdefault(int(p), []).append(v)
    stop = rows[depth]
    child_tokens = {int(tokens[c]) for c in children.get(stop, [])}
    if inputs["logits"] is not None:
        lg = inputs["logits"][b]
        for j in range(depth):
            row = lg[rows[j]]
            row[int(tokens[rows[j + 1]])] = row.max() + np.float32(1.0)
        row = lg[stop]
        low = row.min() - np.float32(1.0)
        for t in child_tokens:
            row[t] = low
    else:
        tid = inputs["target_ids"][b]
        for j in range(depth):
            tid[rows[j]] = tokens[rows[j + 1]]
        choices = [t for t in range(int(inputs["vocab"])) if t not in child_tokens]
        tid[stop] = choices[int(rng.integers(0, len(choices)))]


def draw_heads(seed: int, B: int, K: int, hidden: int, vocab: int,
               w1_std: float = 0.002, w2_std: float = 0.02) -> dict:
    """Inputs of the Medusa head step, bf16-exact values held in float32.

    h            [B, hidden]            ~N(0, 1)            (the last hidden states)
    W1           [K, hidden, hidden]    ~N(0, w1_std^2)     (one matrix per head)
    W2           [K, vocab, hidden]     ~N(0, w2_std^2)
    root_tokens  [B] int32 uniform in [0, vocab)
    The default standard deviations are those of the batched full round (0.002 and 0.02).
    Draw order: h, then per head W1_k and W2_k (in blocks of 4096 rows), then the root
    tokens.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    h = round_to_dtype(rng.standard_normal((B, hidden), dtype=np.float32), "bf16")
    W1 = np.empty((K, hidden, hidden), np.float32)
    W2 = np.empty((K, vocab, hidden), np.float32)

    def fill(dst, std):
        for r0 in range(0, dst.shape[0], 4096):
            blk = dst[r0:r0 + 4096]
            rng.standard_normal(dtype=np.float32, out=blk)
            blk *= np.float32(std)
            blk[...] = round_to_dtype(blk, "bf16")

    for k in range(K):
        fill(W1[k], w1_std)
        fill(W2[k], w2_std)
    root = rng.integers(0, vocab, size=B).astype(np.int32)
    return {"h": h, "W1": W1, "W2": W2, "root_tokens": root}
