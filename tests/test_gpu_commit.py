"""Accept, commit and carry in one call (medusa_accept_commit) on the GPU.

Bit-exact against the oracle (greedy acceptance, snapshot compaction of every layer, the
frontier carry) and against medusa_accept followed by medusa_kv_compact on copies of the
same state.
"""
import dataclasses

import numpy as np
import pytest
import torch

import medusa_tree_attention_amd as M
import workloads
from oracle import accept as AC
from oracle import compact as C

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_support import announce, compile_both, dev, tree_to_device  # noqa: E402

SENTINEL = 12345
HSENTINEL = 4096.0  # exact in bf16
EINVAL, ECAPACITY, EUNSUPPORTED = -1, -3, -4


def planted(w, ora, seed):
    x = workloads.draw_round(w, seed=seed)
    rng = np.random.default_rng(seed)
    for b in range(w.B):
        path = int(rng.integers(0, ora["n_paths"]))
        real = int((ora["retrieve"][path] >= 0).sum()) - 1
        tokens = x["candidates"][b][ora["tree_indices"]]
        workloads.plant_acceptance(rng, x, tokens, ora["retrieve"], ora["parent"], b, path,
                                   int(rng.integers(max(real - 1, 0), real + 1)))
    return x


class CommitCase:
    """A round's acceptance inputs plus n_layers random caches and the tree rows' hidden
    states, kept on the host (float32 holding dtype-exact values) for the oracle."""

    def __init__(self, w, seed, n_layers, hidden_dim=64):
        self.w = w
        self.lib, self.ora = compile_both(w)
        self.x = planted(w, self.ora, seed)
        rng = np.random.default_rng(seed + 1)
        N, S = self.x["N"], self.x["S_max"]
        self.dtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        shape = (w.B, w.Hkv, S, w.d)
        self.caches = [workloads.round_to_dtype(rng.standard_normal(shape, dtype=np.float32), w.dtype)
                       for _ in range(2 * n_layers)]
        self.hidden = workloads.round_to_dtype(
            rng.standard_normal((w.B, N, hidden_dim), dtype=np.float32), w.dtype)
        self.n_layers = n_layers

    def device_state(self, prefix=None):
        st = {"k": [dev(c, self.dtype) for c in self.caches[: self.n_layers]],
              "v": [dev(c, self.dtype) for c in self.caches[self.n_layers:]],
              "prefix": dev(np.asarray(self.x["prefix_len"] if prefix is None else prefix, np.int32)),
              "status": torch.zeros(1, dtype=torch.int32, device="cuda")}
        B, W = self.w.B, self.lib["path_width"]
        for k, s in [("best_path", (B,)), ("accept_len", (B,)), ("accepted_tokens", (B, W)),
                     ("frontier_row", (B,)), ("next_root", (B,))]:
            st[k] = torch.full(s, SENTINEL, dtype=torch.int32, device="cuda")
        st["h_next"] = torch.full((B, self.hidden.shape[-1]), HSENTINEL, dtype=self.dtype, device="cuda")
        return st

    def inputs(self):
        td = tree_to_device(self.lib)
        x = self.x
        return {"cand": dev(x["candidates"]), "td": td,
                "logits": dev(x["logits"]) if x["logits"] is not None else None,
                "tids": dev(x["target_ids"]) if x["target_ids"] is not None else None,
                "ws": torch.zeros(M.medusa_accept_workspace_size(self.w.B, x["N"]), dtype=torch.uint8,
                                  device="cuda"),
                "hidden": dev(self.hidden, self.dtype)}

    def run_fused(self, st, inp, carry=True):
        M.medusa_accept_commit(inp["cand"], inp["td"]["tree_indices"], inp["td"]["retrieve"], st["best_path"],
                               st["accept_len"], st["accepted_tokens"], st["frontier_row"], st["k"], st["v"],
                               st["prefix"], st["status"], logits=inp["logits"], target_ids=inp["tids"],
                               workspace=inp["ws"], hidden=inp["hidden"] if carry else None,
                               h_next=st["h_next"] if carry else None,
                               next_root=st["next_root"] if carry else None)
        torch.cuda.synchronize()
        return int(st["status"].item())

    def run_unfused(self, st, inp):
        M.medusa_accept(inp["cand"], inp["td"]["tree_indices"], inp["td"]["retrieve"], st["best_path"],
                        st["accept_len"], st["accepted_tokens"], st["frontier_row"], st["status"],
                        logits=inp["logits"], target_ids=inp["tids"], workspace=inp["ws"])
        M.medusa_kv_compact(st["k"], st["v"], inp["td"]["retrieve"], st["best_path"], st["accept_len"],
                            st["prefix"], self.x["N"], st["status"])
        torch.cuda.synchronize()
        return int(st["status"].item())

    def oracle(self):
        res = AC.accept_batch(self.ora, self.x["candidates"], logits=self.x["logits"],
                              target_ids=self.x["target_ids"])
        caches = [c.copy() for c in self.caches]
        new_len = C.kv_compact(caches, self.ora["retrieve"], res["best_path"], res["accept_len"],
                               self.x["prefix_len"], self.x["N"])
        carry = AC.frontier_carry(res, self.hidden)
        return res, caches, new_len, carry


def host_state(st):
    out = {k: st[k].cpu().numpy() for k in ("best_path", "accept_len", "accepted_tokens", "frontier_row",
                                             "next_root", "prefix")}
    out["caches"] = [t.float().cpu().numpy() for t in st["k"] + st["v"]]
    out["h_next"] = st["h_next"].float().cpu().numpy()
    return out


CASES = [("tiny", 1), ("llama7b", 3), ("batched", 2), ("wide", 1)]


@pytest.mark.parametrize("name,n_layers", CASES)
def test_accept_commit_matches_oracle(name, n_layers):
    w = workloads.WORKLOADS[name]
    announce(f"accept+commit workload={name} layers={n_layers}")
    case = CommitCase(w, w.seed + 300, n_layers)
    inp = case.inputs()
    st = case.device_state()
    assert case.run_fused(st, inp) == 0
    got = host_state(st)
    res, caches, new_len, carry = case.oracle()
    for k in ("best_path", "accept_len", "frontier_row"):
        assert np.array_equal(got[k], res[k]), k
    assert np.array_equal(got["accepted_tokens"], res["accepted_tokens"])
    assert np.array_equal(got["prefix"], new_len)
    for g, r in zip(got["caches"], caches):
        assert np.array_equal(g, r)
    assert np.array_equal(got["next_root"], carry["next_root"])
    assert np.array_equal(got["h_next"], carry["h_next"].astype(np.float32))
    announce(f"  accept_len {got['accept_len'].tolist()}, next roots {got['next_root'].tolist()}")
    assert got["accept_len"].max() >= 1


@pytest.mark.parametrize("name,n_layers", [("batched", 2), ("tiny", 1)])
def test_fused_equals_accept_then_compact(name, n_layers):
    w = workloads.WORKLOADS[name]
    announce(f"accept+commit vs accept then compact, workload={name}")
    case = CommitCase(w, w.seed + 301, n_layers)
    inp = case.inputs()
    a, b = case.device_state(), case.device_state()
    assert case.run_fused(a, inp, carry=False) == 0
    assert case.run_unfused(b, inp) == 0
    ga, gb = host_state(a), host_state(b)
    for k in ("best_path", "accept_len", "accepted_tokens", "frontier_row", "prefix"):
        assert np.array_equal(ga[k], gb[k]), k
    for x, y in zip(ga["caches"], gb["caches"]):
        assert np.array_equal(x, y)
    assert (ga["next_root"] == SENTINEL).all()  # no carry asked for


def test_ragged_prefixes_and_many_layers():
    w = dataclasses.replace(workloads.WORKLOADS["batched"], B=3, Hkv=2, Hq=8, P=300, slack=7)
    announce("accept+commit ragged prefixes, 32 layers")
    case = CommitCase(w, 17, 32, hidden_dim=256)
    case.x["prefix_len"] = np.array([0, 137, 300], np.int32)
    inp = case.inputs()
    st = case.device_state()
    assert case.run_fused(st, inp) == 0
    got = host_state(st)
    res, caches, new_len, carry = case.oracle()
    assert np.array_equal(got["prefix"], new_len)
    for g, r in zip(got["caches"], caches):
        assert np.array_equal(g, r)
    assert np.array_equal(got["next_root"], carry["next_root"])
    assert np.array_equal(got["h_next"], carry["h_next"].astype(np.float32))


def unchanged(case, st, prefix):
    got = host_state(st)
    assert np.array_equal(got["prefix"], np.asarray(prefix))
    for g, r in zip(got["caches"], case.caches):
        assert np.array_equal(g, r)
    for k in ("best_path", "accept_len", "accepted_tokens", "frontier_row", "next_root"):
        assert (got[k] == SENTINEL).all(), k
    assert (got["h_next"] == HSENTINEL).all()


def test_device_errors_store_nothing():
    w = dataclasses.replace(workloads.WORKLOADS["batched"], B=3, Hkv=2, Hq=8, P=200)
    case = CommitCase(w, 23, 2)
    inp = case.inputs()
    N, S = case.x["N"], case.x["S_max"]
    announce("accept+commit: one sequence without room, a failed round, a NaN logit")
    prefix = [200, S - N + 1, 100]                     # sequence 1 has no room for its staged rows
    st = case.device_state(prefix)
    assert case.run_fused(st, inp) == ECAPACITY
    unchanged(case, st, prefix)
    st = case.device_state()
    st["status"].fill_(EINVAL)                          # an earlier step failed
    assert case.run_fused(st, inp) == EINVAL
    unchanged(case, st, case.x["prefix_len"])
    bad = case.x["logits"].copy()
    bad[2, 7, 123] = np.nan
    inp_nan = dict(inp, logits=dev(bad))
    st = case.device_state()
    assert case.run_fused(st, inp_nan) == EINVAL
    unchanged(case, st, case.x["prefix_len"])


def test_host_rejects_bad_arguments():
    w = dataclasses.replace(workloads.WORKLOADS["batched"], B=2, Hkv=2, Hq=8, P=64)
    case = CommitCase(w, 29, 1)
    inp = case.inputs()
    announce("accept+commit: host argument checks")
    st = case.device_state()
    with pytest.raises(M.MedusaError) as e:        # hidden states without a destination
        M.medusa_accept_commit(inp["cand"], inp["td"]["tree_indices"], inp["td"]["retrieve"], st["best_path"],
                               st["accept_len"], st["accepted_tokens"], st["frontier_row"], st["k"], st["v"],
                               st["prefix"], st["status"], logits=inp["logits"], workspace=inp["ws"],
                               hidden=inp["hidden"])
    assert e.value.code == EINVAL
    k33 = st["k"] * 33
    with pytest.raises(M.MedusaError) as e:        # more layers than one call compacts
        M.medusa_accept_commit(inp["cand"], inp["td"]["tree_indices"], inp["td"]["retrieve"], st["best_path"],
                               st["accept_len"], st["accepted_tokens"], st["frontier_row"], k33, k33,
                               st["prefix"], st["status"], logits=inp["logits"], workspace=inp["ws"])
    assert e.value.code == EUNSUPPORTED
    with pytest.raises(M.MedusaError) as e:        # workspace too small
        M.medusa_accept_commit(inp["cand"], inp["td"]["tree_indices"], inp["td"]["retrieve"], st["best_path"],
                               st["accept_len"], st["accepted_tokens"], st["frontier_row"], st["k"], st["v"],
                               st["prefix"], st["status"], logits=inp["logits"], workspace=inp["ws"][:16])
    unchanged(case, st, case.x["prefix_len"])


def test_batch_of_more_than_64_sequences():
    """Accept, commit and carry for 70 sequences against the oracle."""
    w = dataclasses.replace(workloads.WORKLOADS["batched"], B=70, Hq=4, Hkv=1, tree="cartesian",
                            branching=(2, 2), num_heads=2, topk=2, P=120, slack=5, vocab=512)
    announce("accept+commit with 70 sequences")
    case = CommitCase(w, 47, 2)
    inp = case.inputs()
    st = case.device_state()
    assert case.run_fused(st, inp) == 0
    got = host_state(st)
    res, caches, new_len, carry = case.oracle()
    for k in ("best_path", "accept_len", "frontier_row", "accepted_tokens"):
        assert np.array_equal(got[k], res[k]), k
    assert np.array_equal(got["prefix"], new_len)
    for g, r in zip(got["caches"], caches):
        assert np.array_equal(g, r)
    assert np.array_equal(got["next_root"], carry["next_root"])
    assert np.array_equal(got["h_next"], carry["h_next"].astype(np.float32))
    announce(f"  accept lengths {np.bincount(got['accept_len']).tolist()}")
