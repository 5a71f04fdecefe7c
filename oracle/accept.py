"""Oracle: greedy longest-prefix acceptance.

TEST INFRASTRUCTURE (see the package docstring).

Follows:

* [M7.2] §0x03D "Target Logits Are Shifted Along Reconstructed Paths": the
  logits of packed row u_j score the token of the next path row u_{j+1}.
* [M7.2] §0x04D "Acceptance Starts After A Target-Selected Root":
  a_p = sum_j prod_{r<=j} 1[c_{p,r+1} = argmax p_{p,r}]; the first path
  attaining max_p a_p wins, path 0 when nothing matches; G = a + 1 tokens
  are published (the root always).
* [PartII] Part 7 "Exact Greedy Verification and Rejection": the same
  cumulative-product rule; "Padded paths are not real completions".
* [M7.2] §0x06C "The Terminal Row Carries The Next Frontier": the frontier is
  row retrieve[p*, a]; the next round's target and head distributions are those
  produced at that row (conditioned on exactly the committed history), so the
  next root is the target's greedy token there and the next head step reads the
  hidden state of that row.

Readings: argmax ties go to the lowest vocabulary index; a NaN logit makes
the round invalid; a sentinel (-1) ends a path and never matches.
"""
from __future__ import annotations

import numpy as np


class AcceptError(ValueError):
    pass


def row_argmax(logits_row) -> int:
    """Index of the largest logit, lowest index on ties; NaN is an error."""
    row = np.asarray(logits_row)
    if np.isnan(row).any():
        raise AcceptError("NaN in target logits")
    best = 0
    for i in range(1, row.shape[0]):
        if row[i] > row[best]:
            best = i
    return best


def row_argmax_fast(logits_row) -> int:
    """Same definition through numpy's first-occurrence argmax (used for large vocabularies)."""
    row = np.asarray(logits_row)
    if np.isnan(row).any():
        raise AcceptError("NaN in target logits")
    return int(np.argmax(row))


def path_accept_lengths(tokens, target, retrieve) -> np.ndarray:
    """a_i for every retrieve row: leading edges whose child token equals the parent row's target."""
    retrieve = np.asarray(retrieve)
    a = np.zeros(retrieve.shape[0], np.int32)
    for i in range(retrieve.shape[0]):
        count = 0
        for j in range(retrieve.shape[1] - 1):
            nxt = int(retrieve[i, j + 1])
            if nxt < 0:
                break                       # path exhausted, not a mismatch
            if int(tokens[nxt]) != int(target[int(retrieve[i, j])]):
                break
            count += 1
        a[i] = count
    return a


def greedy_accept(tokens, target, retrieve) -> dict:
    """Select the winning path of one sequence.

    tokens [N]: row tokens (candidates[tree_indices]); target [N]: the
    target's greedy next token per row.  Returns best_path, accept_len (= a),
    accepted tokens (G = a + 1 of them) and frontier_row.
    """
    retrieve = np.asarray(retrieve)
    a = path_accept_lengths(tokens, target, retrieve)
    a_star = int(a.max()) if a.size else 0
    best = int(np.flatnonzero(a == a_star)[0]) if a.size else 0
    rows = [int(r) for r in retrieve[best, : a_star + 1]]
    return {"best_path": best, "accept_len": a_star,
            "accepted_tokens": [int(tokens[r]) for r in rows], "rows": rows,
            "frontier_row": rows[-1], "per_path": a}


def tree_walk_accept(tokens, target, parent) -> list:
    """Independent second algorithm: walk the tree along the target's greedy tokens.

    From the root, move to the child whose token equals the current row's
    target token, as long as one exists.  Returns the visited rows; their
    count minus one is the accepted length.  Requires distinct sibling tokens.
    """
    children = {}
    for v, p in enumerate(parent):
        if p >= 0:
            children.setdefault(int(p), []).append(v)
    rows = [0]
    while True:
        want = int(target[rows[-1]])
        nxt = [c for c in children.get(rows[-1], []) if int(tokens[c]) == want]
        if len(nxt) > 1:
            raise AcceptError("siblings carry equal tokens")
        if not nxt:
            return rows
        rows.append(nxt[0])


def accept_batch(tree: dict, candidates, logits=None, target_ids=None) -> dict:
    """Greedy acceptance for every sequence of a batch; exactly one of logits/target_ids."""
    cand = np.asarray(candidates)
    B = cand.shape[0]
    N = tree["n_nodes"]
    W = tree["path_width"]
    out = {"best_path": np.zeros(B, np.int32), "accept_len": np.zeros(B, np.int32),
           "accepted_tokens": np.full((B, W), -1, np.int32),
           "frontier_row": np.zeros(B, np.int32), "target": np.zeros((B, N), np.int32)}
    for b in range(B):
        tokens = cand[b][tree["tree_indices"]]
        if logits is not None:
            target = np.array([row_argmax_fast(logits[b, u]) for u in range(N)], np.int32)
        else:
            target = np.asarray(target_ids[b], np.int32)
        res = greedy_accept(tokens, target, tree["retrieve"])
        out["best_path"][b] = res["best_path"]
        out["accept_len"][b] = res["accept_len"]
        out["accepted_tokens"][b, : len(res["accepted_tokens"])] = res["accepted_tokens"]
        out["frontier_row"][b] = res["frontier_row"]
        out["target"][b] = target
    return out


def frontier_carry(result: dict, hidden=None) -> dict:
    """The state the next round starts from, for every sequence of an accept_batch result.

    next_root[b] = target[b][frontier_row[b]] (the target's greedy token after the last
    accepted input); with hidden [B][N][H], h_next[b] = hidden[b][frontier_row[b]].
    """
    B = len(result["frontier_row"])
    out = {"next_root": np.array([int(result["target"][b][int(result["frontier_row"][b])])
                                  for b in range(B)], np.int32)}
    if hidden is not None:
        hidden = np.asarray(hidden)
        out["h_next"] = np.stack([hidden[b, int(result["frontier_row"][b])] for b in range(B)])
    return out
