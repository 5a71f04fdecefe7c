"""Greedy acceptance on the GPU: bit-exact against the oracle (through the C ABI)."""
import dataclasses

import numpy as np
import pytest
import torch

import medusa_tree_attention_amd as M
import workloads

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_support import announce, compile_both, dev, oracle_accept, tree_to_device  # noqa: E402


class AcceptRun:
    def __init__(self, w, x, tree):
        self.B, self.W = w.B, tree["path_width"]
        self.td = tree_to_device(tree)
        self.cand = dev(x["candidates"])
        self.logits = dev(x["logits"]) if x["logits"] is not None else None
        self.tids = dev(x["target_ids"]) if x["target_ids"] is not None else None
        self.out = {k: torch.full(s, 12345, dtype=torch.int32, device="cuda") for k, s in
                    [("best_path", (w.B,)), ("accept_len", (w.B,)), ("accepted_tokens", (w.B, self.W)),
                     ("frontier_row", (w.B,))]}
        self.ws = torch.zeros(M.medusa_accept_workspace_size(w.B, x["N"]), dtype=torch.uint8, device="cuda")
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def run(self):
        M.medusa_accept(self.cand, self.td["tree_indices"], self.td["retrieve"], self.out["best_path"],
                        self.out["accept_len"], self.out["accepted_tokens"], self.out["frontier_row"],
                        self.status, logits=self.logits, target_ids=self.tids, workspace=self.ws)
        torch.cuda.synchronize()
        return int(self.status.item()), {k: v.cpu().numpy() for k, v in self.out.items()}


def _compare(got, ref):
    for key in ("best_path", "accept_len", "accepted_tokens", "frontier_row"):
        assert np.array_equal(got[key], ref[key]), key


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
@pytest.mark.parametrize("planted", [False, True])
def test_workload_accept(name, planted):
    w = workloads.WORKLOADS[name]
    announce(f"accept workload={name} planted={planted}")
    lib, ora = compile_both(w)
    x = workloads.draw_round(w, seed=w.seed + (100 if planted else 0))
    if planted:
        rng = np.random.default_rng(w.seed + 100)
        for b in range(w.B):
            path = int(rng.integers(0, ora["n_paths"]))
            real = int((ora["retrieve"][path] >= 0).sum()) - 1
            tokens = x["candidates"][b][ora["tree_indices"]]
            workloads.plant_acceptance(rng, x, tokens, ora["retrieve"], ora["parent"], b, path,
                                       int(rng.integers(max(real - 1, 0), real + 1)))
    status, got = AcceptRun(w, x, lib).run()
    assert status == 0
    ref = oracle_accept(ora, x["candidates"], logits=x["logits"], target_ids=x["target_ids"])
    _compare(got, ref)
    if planted:
        assert got["accept_len"].max() >= 1


def test_argmax_ties_take_the_lowest_index():
    w = dataclasses.replace(workloads.WORKLOADS["llama7b"], B=2, vocab=1000)
    announce("accept argmax ties")
    lib, ora = compile_both(w)
    x = workloads.draw_round(w, seed=5)
    tokens = x["candidates"][0][ora["tree_indices"]]
    lg = x["logits"]
    # the root row has two equal maxima: the lower index is a rejected id, the higher one the
    # token of path row 1 -- the lowest index must win, so nothing is accepted through row 1
    low = int(min(t for t in range(1000) if t not in set(tokens.tolist())))
    lg[0, 0, :] = -1.0
    lg[0, 0, max(low, int(tokens[1]))] = 5.0
    lg[0, 0, min(low, int(tokens[1]))] = 5.0
    status, got = AcceptRun(w, x, lib).run()
    assert status == 0
    _compare(got, oracle_accept(ora, x["candidates"], logits=x["logits"]))


def test_nan_logit_voids_the_round():
    w = dataclasses.replace(workloads.WORKLOADS["llama7b"], B=2, vocab=4096)
    announce("accept NaN logit")
    lib, ora = compile_both(w)
    x = workloads.draw_round(w, seed=6)
    x["logits"][1, 17, 999] = np.nan
    status, got = AcceptRun(w, x, lib).run()
    assert status == -1
    assert all((v == 12345).all() for v in got.values())


def test_invalid_retrieve_is_rejected():
    w = workloads.WORKLOADS["tiny"]
    announce("accept invalid retrieve")
    lib, ora = compile_both(w)
    x = workloads.draw_round(w)
    bad = dict(lib)
    bad["retrieve"] = lib["retrieve"].copy()
    bad["retrieve"][1, 2] = 99
    status, got = AcceptRun(w, x, bad).run()
    assert status == -1
    assert all((v == 12345).all() for v in got.values())


def test_vocab_not_multiple_of_four():
    w = dataclasses.replace(workloads.WORKLOADS["llama7b"], B=3, vocab=1001)
    announce("accept odd vocabulary")
    lib, ora = compile_both(w)
    x = workloads.draw_round(w, seed=8)
    status, got = AcceptRun(w, x, lib).run()
    assert status == 0
    _compare(got, oracle_accept(ora, x["candidates"], logits=x["logits"]))


def test_argmax_ties_across_passes_and_threads():
    """With 16 x 64 rows a row is one piece read by 256 threads in four passes of 8 float4
    columns each (column c4 of pass p, slot k, thread t: c4 = t + 256 k + 2048 p; the last
    pass is partial).  The root rows of three sequences hold two equal maxima, the higher
    index being the token of tree row 1, the lower one read by the same thread in an earlier
    pass, by the same thread in the same pass, or by another thread: the lower index must
    win, so nothing is accepted through row 1."""
    w = dataclasses.replace(workloads.WORKLOADS["llama7b"], B=16, vocab=32000)
    announce("accept argmax ties across passes, slots and threads")
    lib, ora = compile_both(w)
    x = workloads.draw_round(w, seed=9)
    slot1 = int(ora["tree_indices"][1])
    hi = 30001                                 # float4 column 7500 = 76 + 256*5 + 2048*3, element 1
    lows = [4 * (76 + 256 * 5) + 1,            # thread 76, pass 0: an earlier pass
            4 * (6144 + 76) + 1,               # thread 76, pass 3, slot 0: the same pass
            4 * (6144 + 6) + 1]                # thread 6, pass 3: another thread
    lg = x["logits"]
    for b, lo in enumerate(lows):
        x["candidates"][b, slot1] = hi
        depth1 = [int(x["candidates"][b, s]) for s in ora["tree_indices"][1:] if s <= w.topk]
        assert lo not in depth1               # a wrong tie-break, not another child, decides
        lg[b, 0, :] = -1.0
        lg[b, 0, lo] = 5.0
        lg[b, 0, hi] = 5.0
    status, got = AcceptRun(w, x, lib).run()
    assert status == 0
    ref = oracle_accept(ora, x["candidates"], logits=x["logits"])
    _compare(got, ref)
    assert (ref["accept_len"][:3] == 0).all()
