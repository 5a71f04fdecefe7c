"""Fast typical acceptance on the GPU against the oracle (through the C ABI).

The kernel forms each row's softmax statistics in fp32, the oracle in binary64.  A pass
decision p(c) > tau whose relative margin is below 1e-4, or a log-likelihood tie-break
between equally long paths separated by less than 1e-3, may therefore go either way; such
sequences are found with the oracle and left out of the exact comparison, and each test
states how many sequences it compared.
"""
import dataclasses

import numpy as np
import pytest
import torch

import medusa_tree_attention_amd as M
import workloads
from oracle import typical as TY

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_support import announce, compile_both, dev, tree_to_device  # noqa: E402

EPS, ALPHA = TY.EPSILON, TY.ALPHA
EINVAL = -1  # MEDUSA_EINVAL
LOGIT_WORKLOADS = [n for n, w in workloads.WORKLOADS.items() if w.use_logits]


class TypicalRun:
    def __init__(self, w, x, tree):
        self.td = tree_to_device(tree)
        self.W = tree["path_width"]
        self.cand = dev(x["candidates"])
        self.logits = dev(x["logits"])
        self.out = {k: torch.full(s, 12345, dtype=torch.int32, device="cuda") for k, s in
                    [("best_path", (w.B,)), ("accept_len", (w.B,)), ("accepted_tokens", (w.B, self.W)),
                     ("frontier_row", (w.B,))]}
        self.ws = torch.zeros(M.medusa_accept_workspace_size(w.B, x["N"]), dtype=torch.uint8, device="cuda")
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def run(self, temperature, epsilon=EPS, alpha=ALPHA):
        M.medusa_accept_typical(self.cand, self.td["tree_indices"], self.td["retrieve"],
                                self.out["best_path"], self.out["accept_len"],
                                self.out["accepted_tokens"], self.out["frontier_row"], self.status,
                                self.logits, self.ws, temperature=temperature, epsilon=epsilon,
                                alpha=alpha)
        torch.cuda.synchronize()
        return int(self.status.item()), {k: v.cpu().numpy() for k, v in self.out.items()}


def robust(tokens, logits, retrieve, T):
    """False when a pass decision or the winning tie-break lies within fp32 reach."""
    cache = {}

    def stats(r):
        if r not in cache:
            p = TY.softmax(logits[r], T)
            cache[r] = (p, TY.threshold(p))
        return cache[r]

    n_paths, width = retrieve.shape
    a = np.zeros(n_paths, int)
    ll = np.zeros(n_paths)
    for i in range(n_paths):
        for j in range(width - 1):
            nxt = int(retrieve[i, j + 1])
            if nxt < 0:
                break
            p, tau = stats(int(retrieve[i, j]))
            pc = p[int(tokens[nxt])]
            if abs(pc - tau) <= 1e-4 * tau:
                return False
            if not pc > tau:
                break
            a[i] += 1
            ll[i] += np.log(pc)
    # equally long paths that accept the same rows sum the same terms on both sides: an
    # exact tie, the first index wins.  Only distinct accepted prefixes can be too close.
    best = {}
    for i in np.flatnonzero(a == a.max()):
        key = tuple(int(r) for r in retrieve[i, : a.max() + 1])
        best[key] = max(best.get(key, -np.inf), ll[i])
    top = sorted(best.values(), reverse=True)
    return len(top) < 2 or top[0] - top[1] > 1e-3 * max(1.0, abs(top[0]))


def check(w, x, ora, lib, T):
    status, got = TypicalRun(w, x, lib).run(T)
    assert status == 0
    compared = 0
    for b in range(w.B):
        tokens = x["candidates"][b][ora["tree_indices"]]
        if not robust(tokens, x["logits"][b], ora["retrieve"], T):
            continue
        ref = TY.typical_accept(tokens, x["logits"][b], ora["retrieve"], T)
        assert got["best_path"][b] == ref["best_path"], b
        assert got["accept_len"][b] == ref["accept_len"], b
        assert got["frontier_row"][b] == ref["frontier_row"], b
        G = ref["accept_len"] + 1
        assert got["accepted_tokens"][b][:G].tolist() == ref["accepted_tokens"], b
        assert (got["accepted_tokens"][b][G:] == -1).all(), b
        compared += 1
    return compared, got


def planted_round(w, ora, seed):
    x = workloads.draw_round(w, seed=seed)
    rng = np.random.default_rng(seed)
    for b in range(w.B):
        path = int(rng.integers(0, ora["n_paths"]))
        real = int((ora["retrieve"][path] >= 0).sum()) - 1
        tokens = x["candidates"][b][ora["tree_indices"]]
        workloads.plant_acceptance(rng, x, tokens, ora["retrieve"], ora["parent"], b, path,
                                   int(rng.integers(max(real - 1, 0), real + 1)))
    return x


@pytest.mark.parametrize("name", LOGIT_WORKLOADS)
@pytest.mark.parametrize("planted,T", [(False, 1.0), (True, 0.25)])
def test_workload_typical(name, planted, T):
    w = workloads.WORKLOADS[name]
    announce(f"typical accept workload={name} planted={planted} T={T}")
    lib, ora = compile_both(w)
    x = planted_round(w, ora, w.seed + 200) if planted else workloads.draw_round(w, seed=w.seed + 200)
    compared, got = check(w, x, ora, lib, T)
    announce(f"  compared {compared} of {w.B} sequences; accept_len {got['accept_len'].tolist()}")
    assert compared >= max(1, w.B - 1)


@pytest.mark.parametrize("vocab", [40000, 1001])
def test_long_and_unaligned_rows(vocab):
    # 40000 > 32768 logits: the streamed statistics; 1001: rows not a multiple of four
    w = dataclasses.replace(workloads.WORKLOADS["llama7b"], B=2, vocab=vocab)
    announce(f"typical accept vocab={vocab}")
    lib, ora = compile_both(w)
    x = workloads.draw_round(w, seed=7)
    x["candidates"] = x["candidates"] % vocab
    compared, _ = check(w, x, ora, lib, 1.0)
    assert compared >= 1


def test_low_temperature_is_greedy():
    w = dataclasses.replace(workloads.WORKLOADS["batched"], B=3)
    announce("typical accept at low temperature vs greedy")
    lib, ora = compile_both(w)
    x = planted_round(w, ora, 11)
    run = TypicalRun(w, x, lib)
    status, typ = run.run(1e-3)
    assert status == 0
    greedy = {k: torch.full_like(v, 12345) for k, v in run.out.items()}
    M.medusa_accept(run.cand, run.td["tree_indices"], run.td["retrieve"], greedy["best_path"],
                    greedy["accept_len"], greedy["accepted_tokens"], greedy["frontier_row"], run.status,
                    logits=run.logits, workspace=run.ws)
    torch.cuda.synchronize()
    assert int(run.status.item()) == 0
    assert np.array_equal(typ["accept_len"], greedy["accept_len"].cpu().numpy())
    assert np.array_equal(typ["accepted_tokens"], greedy["accepted_tokens"].cpu().numpy())
    assert typ["accept_len"].max() >= 1


def test_device_errors_store_nothing():
    w = dataclasses.replace(workloads.WORKLOADS["llama7b"], B=2, vocab=1000)
    lib, ora = compile_both(w)
    announce("typical accept: candidate outside the vocabulary, NaN logit")
    x = workloads.draw_round(w, seed=3)
    x["candidates"] = x["candidates"] % 1000
    bad = dict(x)
    bad["candidates"] = x["candidates"].copy()
    bad["candidates"][1, 3] = 1000
    status, got = TypicalRun(w, bad, lib).run(1.0)
    assert status == EINVAL and (got["accept_len"] == 12345).all()
    bad = dict(x)
    bad["logits"] = x["logits"].copy()
    bad["logits"][0, 5, 17] = np.nan
    status, got = TypicalRun(w, bad, lib).run(1.0)
    assert status == EINVAL and (got["accept_len"] == 12345).all()


def test_host_rejects_bad_arguments():
    w = dataclasses.replace(workloads.WORKLOADS["llama7b"], B=1, vocab=1000)
    lib, _ = compile_both(w)
    announce("typical accept: host argument checks")
    x = workloads.draw_round(w, seed=5)
    x["candidates"] = x["candidates"] % 1000
    run = TypicalRun(w, x, lib)
    for kw in ({"temperature": 0.0}, {"temperature": float("nan")}, {"epsilon": -0.1},
               {"alpha": float("inf")}):
        with pytest.raises(M.MedusaError):
            run.run(**{"temperature": 1.0, **kw})
    run.ws = run.ws[:8]
    with pytest.raises(M.MedusaError):
        run.run(1.0)
