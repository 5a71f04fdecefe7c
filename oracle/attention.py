"""Oracle: tree attention as one ordinary causal attention per root-to-node path.

TEST INFRASTRUCTURE (see the package docstring).

What the pages fix:

* [Chai] section "Tree Attention：把一棵树压进一次并行前向": a node attends to
  the committed context, itself and its ancestors only, and the result equals
  feeding that node's root-to-node sequence to the model on its own; the
  attention is softmax(Q K^T / sqrt(d_h) + M) V with M = 0 or -inf.  Its
  engineering section "Mask、位置和 KV 必须一起验证" recommends exactly this
  per-path comparison.
* [M7.2] §0x03C "Target Verification Is A Rectangular Forward Contract":
  every prefix row is visible; staged row u is written to cache row P + u
  while its logical position is P + depth(u).
* [M7.2] §0x03A / §0x01B: position(u) = prefix_length + depth(u); siblings
  share a position.
* [Math] "Tree attention: the mask math": the same mask and position rule.

Readings where the pages are silent ("RoPE" is named, not specified):

* RoPE uses the rotate-half pairing (x[i], x[i + d/2]) with inverse
  frequency base^(-2i/d), angles in binary64.
* The committed prefix rows of the cache already hold rotated keys and are
  used as stored.
* Query head h reads key/value head h // (Hq / Hkv).
* Masked pairs are excluded from the softmax (exactly zero weight).
"""
from __future__ import annotations

import numpy as np


def rope_inv_freq(d: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/d) for i < d/2, binary64."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(base), -(2.0 * i) / d)


def rope(x, pos: int, base: float) -> np.ndarray:
    """Rotate the last axis of ``x`` to logical position ``pos`` (rotate-half pairing)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = np.float64(pos) * rope_inv_freq(d, base)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def root_path(parent, u: int) -> list:
    """Rows on the path root -> u, in depth order."""
    chain = []
    while u >= 0:
        chain.append(int(u))
        u = int(parent[u])
    return chain[::-1]


def causal_last_row(q_row, keys, values) -> np.ndarray:
    """Ordinary causal attention output of the last position of a sequence.

    The last row of a causal sequence sees every earlier row and itself:
    softmax(q . k_j / sqrt(d)) over all rows j, then the weighted sum of values.
    """
    d = q_row.shape[-1]
    s = keys @ q_row / np.sqrt(np.float64(d))
    s = s - s.max()
    p = np.exp(s)
    p = p / p.sum()
    return p @ values


def tree_attention(q, k_new, v_new, k_cache, v_cache, prefix_len, depth, parent,
                   rope_base: float, rows=None):
    """Reference output of one tree-attention layer.

    q [B,N,Hq,d]; k_new, v_new [B,N,Hkv,d]; k_cache, v_cache [B,Hkv,S,d]
    (only rows [0, P_b) are read); prefix_len [B]; depth, parent [N].
    ``rows`` optionally restricts the computed outputs to an iterable of
    (b, u, h) triples (the rest stay NaN).

    Returns (out [B,N,Hq,d], staged_k [B,Hkv,N,d], staged_v [B,Hkv,N,d]) in
    binary64; staged_k[b,g,u] = RoPE(k_new[b,u,g], P_b + depth[u]) is what
    cache row P_b + u must hold (before rounding to the storage dtype).
    """
    q = np.asarray(q, np.float64)
    k_new = np.asarray(k_new, np.float64)
    v_new = np.asarray(v_new, np.float64)
    B, N, Hq, d = q.shape
    Hkv = k_new.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv

    staged_k = np.empty((B, Hkv, N, d))
    staged_v = np.empty((B, Hkv, N, d))
    for b in range(B):
        P = int(prefix_len[b])
        for u in range(N):
            for g in range(Hkv):
                staged_k[b, g, u] = rope(k_new[b, u, g], P + int(depth[u]), rope_base)
                staged_v[b, g, u] = v_new[b, u, g]

    out = np.full((B, N, Hq, d), np.nan)
    if rows is None:
        rows = [(b, u, h) for b in range(B) for u in range(N) for h in range(Hq)]
    by_path = {}
    for b, u, h in rows:
        by_path.setdefault((b, u), []).append(h)
    for (b, u), heads in by_path.items():
        P = int(prefix_len[b])
        path = root_path(parent, u)
        for h in heads:
            g = h // group
            # the causal sequence "committed rows, then path(u)"; its last row is u
            keys = np.concatenate([np.asarray(k_cache[b, g, :P], np.float64),
                                   staged_k[b, g, path]], axis=0)
            values = np.concatenate([np.asarray(v_cache[b, g, :P], np.float64),
                                     staged_v[b, g, path]], axis=0)
            q_rot = rope(q[b, u, h], P + int(depth[u]), rope_base)
            out[b, u, h] = causal_last_row(q_rot, keys, values)
    return out, staged_k, staged_v
