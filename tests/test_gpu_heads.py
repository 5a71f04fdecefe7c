"""The Medusa head step on the GPU against the oracle (through the C ABI).

Tolerance of a logit.  The library widens the bf16 inputs to fp32 and accumulates each dot
product in fp32: a lane sums its d/64 products with fused multiply-adds, then six butterfly
additions combine the 64 lanes, so every inner product carries at most n = max(d/64, 8) + 6
roundings.  Two bounds follow (u = 2^-24):

* worst case: an inner product errs by at most gamma_n = n u / (1 - n u) times its sum of
  absolute products.  For a = W1 h that gives ea = gamma_n |W1| |h|; u = SiLU(a) + h
  inherits 1.1 ea (|SiLU'| < 1.1) plus at most 8 u (|SiLU(a)| + |h|) from the exponential,
  the division and the addition; a logit carries gamma_n |W2| |u| + |W2| du.
* probabilistic (Higham and Mary, "A new approach to probabilistic rounding error analysis",
  2019: independent rounding errors of mean zero): lam times the same terms with gamma_n
  replaced by sqrt(n) u and the propagated term |W2| du by sqrt(W2^2 du^2), lam = 8, which
  one logit exceeds with probability below 1e-13.

Every logit must lie within both (twice the worst case; the probabilistic one as it is): the
worst case is what fp32 guarantees, the probabilistic one is tight enough to catch a dropped
term at hidden size 4096.

A candidate rank is compared exactly when the oracle's value at that rank is separated from
its neighbours' by more than their tolerances; every rank is also checked to hold a token
whose oracle logit lies within tolerance of the oracle's value at that rank, and the ids the
library returns must be exactly the stable descending order of the fp32 logits it returns.
"""
import numpy as np
import pytest
import torch

import medusa_tree_attention_amd as M
import workloads
from oracle import heads as HD

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_support import announce, dev  # noqa: E402

EINVAL, EUNSUPPORTED, EBUFSIZE = -1, -4, -5
U32 = 2.0 ** -24
SENTINEL = 12345


class HeadRun:
    def __init__(self, x, topk):
        self.x = x
        self.topk = topk
        self.h = dev(x["h"], torch.bfloat16)
        self.W1 = dev(x["W1"], torch.bfloat16)
        self.W2 = dev(x["W2"], torch.bfloat16)
        self.root = dev(x["root_tokens"])
        B, d = x["h"].shape
        K, V = x["W2"].shape[:2]
        self.shape = (B, K, d, V)
        self.cand = torch.full((B, 1 + K * topk), SENTINEL, dtype=torch.int32, device="cuda")
        self.logits = torch.full((K, B, V), float(SENTINEL), dtype=torch.float32, device="cuda")
        self.ws = torch.zeros(M.medusa_head_workspace_size(B, K, d, V), dtype=torch.uint8, device="cuda")
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def run(self, with_logits=True, **kw):
        args = dict(h=self.h, W1=self.W1, W2=self.W2, root_tokens=self.root, candidates=self.cand,
                    status=self.status, workspace=self.ws, topk=self.topk,
                    head_logits=self.logits if with_logits else None)
        args.update(kw)
        M.medusa_head_candidates(**args)
        torch.cuda.synchronize()
        return int(self.status.item()), self.cand.cpu().numpy(), self.logits.cpu().numpy()


def tolerance(x):
    """(worst-case, probabilistic) error bounds of every logit, [K][B][V] each."""
    h = x["h"].astype(np.float64)
    K, V, d = x["W2"].shape
    n = max(d // 64, 8) + 6
    gamma = n * U32 / (1 - n * U32)
    sig = np.sqrt(n) * U32
    worst = np.zeros((K, h.shape[0], V))
    likely = np.zeros_like(worst)
    for k in range(K):
        W1 = x["W1"][k].astype(np.float64)
        a = h @ W1.T                                             # [B][d]
        s1 = np.abs(h) @ np.abs(W1).T
        silu = HD.silu(a)
        u = np.abs(silu + h)
        own = 8 * U32 * (np.abs(silu) + np.abs(h))
        du_w = 1.1 * gamma * s1 + own
        du_p = 1.1 * sig * s1 + own                              # one standard scale
        aW2 = np.abs(x["W2"][k])                                 # float32 is enough here
        s2 = u.astype(np.float32) @ aW2.T
        worst[k] = 2.0 * (gamma * s2 + du_w.astype(np.float32) @ aW2.T)
        likely[k] = 8.0 * (sig * s2 + np.sqrt((du_p ** 2).astype(np.float32) @ (aW2 ** 2).T))
    return worst, likely


def check(x, topk, status, cand, logits, ref, tols):
    assert status == 0
    K, B, V = ref["logits"].shape
    err = np.abs(logits.astype(np.float64) - ref["logits"])
    for tol in tols:
        at = np.unravel_index(np.argmax(err / tol), err.shape)
        assert (err <= tol).all(), (at, err[at], tol[at])
    tol = tols[1]
    assert np.array_equal(cand[:, 0], x["root_tokens"])
    exact = 0
    for b in range(B):
        for k in range(K):
            got = cand[b, 1 + k * topk: 1 + (k + 1) * topk]
            row, lrow, trow = ref["logits"][k, b], logits[k, b], tol[k, b]
            # the library's own decision: stable descending order of its fp32 logits
            mine = np.argsort(-lrow, kind="stable")[:topk]
            assert np.array_equal(got, mine), (b, k)
            want = ref["candidates"][b, 1 + k * topk: 1 + (k + 1) * topk]
            order = np.argsort(-row, kind="stable")[: topk + 1]
            tmax = trow.max()
            for r in range(topk):
                assert abs(row[got[r]] - row[order[r]]) <= 2 * tmax, (b, k, r)
                lo = row[order[r + 1]] if r + 1 < len(order) else -np.inf
                hi = row[order[r - 1]] if r > 0 else np.inf
                if row[order[r]] - lo > 2 * tmax and hi - row[order[r]] > 2 * tmax:
                    assert got[r] == want[r], (b, k, r)
                    exact += 1
    return exact


CASES = [
    # (B, K, d, V, topk): ragged column group and vocab tail; one of everything; the
    # vocabulary of the batched round with a short hidden size (cached top-k at V = 32000);
    # a vocabulary longer than the register-cached top-k; topk = V = 64 (the largest
    # topk); a hidden size above 4096 (more than the default LDS per launch)
    (5, 3, 256, 3001, 10),
    (1, 1, 8, 1, 1),
    (4, 4, 64, 32000, 10),
    (4, 2, 512, 40000, 10),
    (2, 2, 64, 64, 64),
    (3, 1, 8192, 700, 5),
]


@pytest.mark.parametrize("B,K,d,V,topk", CASES)
def test_head_parity(B, K, d, V, topk):
    announce(f"head step B={B} K={K} d={d} V={V} topk={topk}")
    x = workloads.draw_heads(100 + B + K + d + V, B, K, d, V)
    ref = HD.head_candidates(x["h"], x["W1"], x["W2"], x["root_tokens"], topk)
    run = HeadRun(x, topk)
    status, cand, logits = run.run()
    exact = check(x, topk, status, cand, logits, ref, tolerance(x))
    announce(f"  {exact} of {B * K * topk} ranks compared exactly")
    assert exact >= B * K * topk * 0.8
    # without the optional logits output the candidates are the same
    run.cand.fill_(SENTINEL)
    status2, cand2, _ = run.run(with_logits=False)
    assert status2 == 0 and np.array_equal(cand, cand2)


def test_batched_round_shape():
    # four heads, hidden 4096, vocabulary 32000, four sequences, topk 10: every logit and
    # every candidate against the oracle
    B, K, d, V, topk = 4, 4, 4096, 32000, 10
    announce(f"head step full shape B={B} K={K} d={d} V={V} topk={topk} (drawing weights)")
    x = workloads.draw_heads(7, B, K, d, V)
    run = HeadRun(x, topk)
    status, cand, logits = run.run()
    announce("  oracle")
    ref = HD.head_candidates(x["h"], x["W1"], x["W2"], x["root_tokens"], topk)
    exact = check(x, topk, status, cand, logits, ref, tolerance(x))
    announce(f"  {exact} of {B * K * topk} ranks compared exactly")
    assert exact >= B * K * topk * 0.8


def test_exact_closed_forms():
    # W1 = 0 makes u = h (SiLU(0) = 0); rows of W2 that are unit vectors pick coordinates of
    # h, so every logit is exact and so is the ranking.  Rows 0..V-1 of W2 select
    # coordinate perm[v]; several rows select the same coordinate (exact ties: the lower id
    # first); the last head's W2 is zero (all logits 0: ids 0..topk-1).
    B, K, d, V, topk = 3, 3, 64, 200, 12
    rng = np.random.default_rng(5)
    x = workloads.draw_heads(9, B, K, d, V)
    x["W1"][:] = 0.0
    x["W2"][:] = 0.0
    for k in range(K - 1):
        perm = rng.integers(0, d, size=V)
        x["W2"][k, np.arange(V), perm] = 1.0
    announce("head step closed forms: W1 = 0, selection rows, a zero head")
    run = HeadRun(x, topk)
    status, cand, logits = run.run()
    assert status == 0
    for k in range(K - 1):
        perm = np.argmax(x["W2"][k], axis=1)
        for b in range(B):
            want_logits = x["h"][b][perm].astype(np.float32)
            assert np.array_equal(logits[k, b], want_logits)
            order = sorted(range(V), key=lambda v: (-float(want_logits[v]), v))[:topk]
            assert cand[b, 1 + k * topk: 1 + (k + 1) * topk].tolist() == order
    assert (logits[K - 1] == 0).all()
    for b in range(B):
        assert cand[b, 1 + (K - 1) * topk:].tolist() == list(range(topk))


def test_nan_logit_fails_the_round():
    B, K, d, V, topk = 2, 3, 64, 500, 4
    x = workloads.draw_heads(11, B, K, d, V)
    x["W2"][1, 77, 5] = np.nan  # head 1's logit 77 is NaN for every sequence
    announce("head step: NaN logit")
    run = HeadRun(x, topk)
    status, cand, _ = run.run()
    assert status == EINVAL
    # the poisoned head stored nothing
    assert (cand[:, 1 + topk: 1 + 2 * topk] == SENTINEL).all()


def test_failed_round_stores_nothing():
    B, K, d, V, topk = 2, 2, 64, 300, 4
    x = workloads.draw_heads(12, B, K, d, V)
    announce("head step: status already failed")
    run = HeadRun(x, topk)
    run.status.fill_(EINVAL)
    status, cand, logits = run.run()
    assert status == EINVAL
    assert (cand == SENTINEL).all() and (logits == SENTINEL).all()


def test_host_rejects_bad_arguments():
    B, K, d, V, topk = 2, 2, 64, 100, 4
    x = workloads.draw_heads(13, B, K, d, V)
    announce("head step: host argument checks")
    run = HeadRun(x, topk)
    for kw, code in (({"topk": 0}, EINVAL), ({"topk": 65}, EUNSUPPORTED),
                     ({"workspace": run.ws[:64]}, EBUFSIZE)):
        with pytest.raises(M.MedusaError) as e:
            run.run(**kw)
        assert e.value.code == code, kw
    # weights not 16-byte aligned
    W2 = torch.empty(K * V * d + 1, dtype=torch.bfloat16, device="cuda")[1:].view(K, V, d)
    W2.copy_(run.W2)
    with pytest.raises(M.MedusaError) as e:
        run.run(W2=W2)
    assert e.value.code == EINVAL
    # hidden sizes that are not a multiple of 8, or above 8192
    for dd in (12, 8200):
        h = torch.zeros(B, dd, dtype=torch.bfloat16, device="cuda")
        W1 = torch.zeros(K, 16, dtype=torch.bfloat16, device="cuda")
        W2 = torch.zeros(K, V, dd, dtype=torch.bfloat16, device="cuda")
        with pytest.raises(M.MedusaError) as e:
            run.run(h=h, W1=W1, W2=W2)
        assert e.value.code == EUNSUPPORTED, dd
    assert (run.cand == SENTINEL).all()
    # topk above the vocabulary
    small = HeadRun(workloads.draw_heads(14, 1, 1, 8, 30), 31)
    with pytest.raises(M.MedusaError) as e:
        small.run()
    assert e.value.code == EUNSUPPORTED
