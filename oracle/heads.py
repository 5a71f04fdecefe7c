"""Oracle: the Medusa head step and the candidate pool.

TEST INFRASTRUCTURE (see the package docstring).

Follows:

* [Chai] section "Medusa 的核心思路与系统位置" and [Math] section "The Medusa head:
  math and shapes": head k maps the last hidden state h to
  p^(k) = softmax(W2_k (SiLU(W1_k h) + h)), W1_k of shape [d, d], W2_k of shape [V, d],
  column-vector convention (W @ h).  [M7.2] section 0x02A writes the same residual block
  with a bias; the workload specifies none, so there is none here.
* [PartII] Part 4: each head contributes its TOPK ranked token ids (torch.topk of the head
  logits, TOPK = 10).  The ranking needs only the logits, not the softmax.
* [M7.2] section 0x01B: slot(j, r) = 1 + j * TOPK + r in the flattened candidate row, and
  [Chai] section "一次完整解码迭代": the target's own LM head decides the root token, slot 0.

Reading taken where the pages are silent: among equal logits the lower token id ranks first.
Arithmetic in binary64 on the given (already rounded) inputs.
"""
from __future__ import annotations

import numpy as np


def silu(x):
    x = np.asarray(x, np.float64)
    return x / (1.0 + np.exp(-x))


def head_logits(h, W1, W2) -> np.ndarray:
    """Logits of one head for one hidden vector: W2 (SiLU(W1 h) + h)."""
    h = np.asarray(h, np.float64)
    u = silu(np.asarray(W1, np.float64) @ h) + h
    return np.asarray(W2, np.float64) @ u


def top_ranked(logits_row, k: int) -> list:
    """The k largest entries, largest first, the lower index first among equal values (a
    stable sort by descending value)."""
    row = np.asarray(logits_row, np.float64)
    order = np.argsort(-row, kind="stable")
    return [int(i) for i in order[:k]]


def head_candidates(h, W1, W2, root_tokens, topk: int) -> dict:
    """Candidate rows [B][1 + K * topk] and the head logits [K][B][V].

    h [B][d]; W1 [K][d][d]; W2 [K][V][d]; root_tokens [B].
    """
    h = np.asarray(h, np.float64)
    K = len(W1)
    B = h.shape[0]
    V = np.asarray(W2[0]).shape[0]
    logits = np.zeros((K, B, V), np.float64)
    cand = np.zeros((B, 1 + K * topk), np.int64)
    for b in range(B):
        cand[b, 0] = int(root_tokens[b])
        for k in range(K):
            logits[k, b] = head_logits(h[b], W1[k], W2[k])
            ranked = top_ranked(logits[k, b], topk)
            for r in range(topk):
                cand[b, 1 + k * topk + r] = ranked[r]
    return {"candidates": cand, "logits": logits}
