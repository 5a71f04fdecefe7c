"""Oracle: fast typical acceptance.

TEST INFRASTRUCTURE (see the package docstring).

Follows [M7.2] §0x04E "Fast Typical Acceptance Derivation":

* p = softmax(logits / temperature) of the row that scores the next path token;
* H(p) = -sum_x p(x) log p(x), computed with the implementation's 1e-5
  guard inside the logarithm, as the page's listing shows;
* tau = min(epsilon, alpha * exp(-H)) and a pass is the strict p(c) > tau;
* a_p = sum_j prod_{r<=j} pass_{p,r};
* among paths of maximal a*, the winner maximises
  sum_{j<a*} log p_{p,j}(c_{p,j+1}); the first such path on exact ties.

[Chai] section "接受机制" gives the defaults posterior_threshold = 0.3 (epsilon)
and posterior_alpha = 0.09 (the page's delta); [M7.2] §0x04E agrees that
epsilon is the ceiling.  [Math] "Typical acceptance, not exact match" prints
the two constants the other way round; this oracle follows the first two.
"""
from __future__ import annotations

import numpy as np

EPSILON = 0.3
ALPHA = 0.09
LOG_GUARD = 1e-5


def softmax(logits_row, temperature: float) -> np.ndarray:
    z = np.asarray(logits_row, np.float64) / np.float64(temperature)
    z = z - z.max()
    e = np.exp(z)
    return e / e.sum()


def entropy(p) -> float:
    return float(-(p * np.log(p + LOG_GUARD)).sum())


def threshold(p, epsilon: float = EPSILON, alpha: float = ALPHA) -> float:
    return min(epsilon, alpha * float(np.exp(-entropy(p))))


def typical_accept(tokens, logits, retrieve, temperature: float,
                   epsilon: float = EPSILON, alpha: float = ALPHA) -> dict:
    """Winning path of one sequence under fast typical acceptance.

    tokens [N] row tokens; logits [N, V] target logits per row.
    """
    retrieve = np.asarray(retrieve)
    n_paths, width = retrieve.shape
    probs = {}

    def row_probs(r):
        if r not in probs:
            probs[r] = softmax(logits[r], temperature)
        return probs[r]

    a = np.zeros(n_paths, np.int32)
    loglik = np.zeros(n_paths, np.float64)
    for i in range(n_paths):
        for j in range(width - 1):
            nxt = int(retrieve[i, j + 1])
            if nxt < 0:
                break
            p = row_probs(int(retrieve[i, j]))
            pc = p[int(tokens[nxt])]
            if not pc > threshold(p, epsilon, alpha):
                break
            a[i] += 1
    a_star = int(a.max())
    tied = np.flatnonzero(a == a_star)
    for i in tied:
        s = 0.0
        for j in range(a_star):
            p = row_probs(int(retrieve[i, j]))
            s += float(np.log(p[int(tokens[int(retrieve[i, j + 1])])]))
        loglik[i] = s
    best = int(tied[0])
    for i in tied[1:]:
        if loglik[i] > loglik[best]:
            best = int(i)
    rows = [int(r) for r in retrieve[best, : a_star + 1]]
    return {"best_path": best, "accept_len": a_star, "rows": rows,
            "accepted_tokens": [int(tokens[r]) for r in rows], "frontier_row": rows[-1],
            "per_path": a}
