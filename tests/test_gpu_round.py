"""A whole verification round on the GPU -- attention, acceptance, compaction on
one stream with no host synchronisation in between -- against the oracle."""
import numpy as np
import pytest
import torch

import medusa_tree_attention_amd as M
import workloads
from oracle import compact as C

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_support import (TOL, AttnRun, announce, compile_both, dev, host, oracle_accept,  # noqa: E402
                         sample_rows, staged_k_ratio)


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_round(name):
    w = workloads.WORKLOADS[name]
    announce(f"round workload={name}")
    lib, ora = compile_both(w)
    x = workloads.draw_round(w, seed=w.seed + 100)
    rng = np.random.default_rng(w.seed + 200)
    for b in range(w.B):                          # planted acceptance: G > 1 with overlapping rows
        path = int(rng.integers(0, ora["n_paths"]))
        real = int((ora["retrieve"][path] >= 0).sum()) - 1
        tokens = x["candidates"][b][ora["tree_indices"]]
        workloads.plant_acceptance(rng, x, tokens, ora["retrieve"], ora["parent"], b, path, real)

    att = AttnRun(w, x, lib, ora)
    td = att.td
    outs = {k: torch.zeros(s, dtype=torch.int32, device="cuda") for k, s in
            [("best_path", (w.B,)), ("accept_len", (w.B,)),
             ("accepted_tokens", (w.B, lib["path_width"])), ("frontier_row", (w.B,))]}
    ws = torch.zeros(M.medusa_accept_workspace_size(w.B, x["N"]), dtype=torch.uint8, device="cuda")
    cand = dev(x["candidates"])
    logits = dev(x["logits"]) if x["logits"] is not None else None
    tids = dev(x["target_ids"]) if x["target_ids"] is not None else None
    prefix = att.prefix

    # attention, then a snapshot of the staged cache for the compaction oracle
    M.medusa_tree_attn(att.q, att.kn, att.vn, att.kc, att.vc, td["depth"], td["mask"], prefix,
                       w.rope_base, att.out, att.ws, att.status)
    staged_k, staged_v = att.kc.clone(), att.vc.clone()
    M.medusa_accept(cand, td["tree_indices"], td["retrieve"], outs["best_path"], outs["accept_len"],
                    outs["accepted_tokens"], outs["frontier_row"], att.status, logits=logits,
                    target_ids=tids, workspace=ws)
    M.medusa_kv_compact([att.kc], [att.vc], td["retrieve"], outs["best_path"], outs["accept_len"],
                        prefix, x["N"], att.status)
    torch.cuda.synchronize()
    assert int(att.status.item()) == 0

    rows = sample_rows(w, x["N"], 64 if w.B * x["N"] * w.Hq > 512 else w.B * x["N"] * w.Hq, seed=2)
    out_ref, _, _ = att.oracle(rows)
    got = host(att.out)
    err = max(float(np.abs(got[r] - out_ref[r]).max()) for r in rows)
    assert err <= TOL[w.dtype]

    ref = oracle_accept(ora, x["candidates"], logits=x["logits"], target_ids=x["target_ids"])
    for key in outs:
        assert np.array_equal(outs[key].cpu().numpy(), ref[key]), key
    assert (ref["accept_len"] >= 1).all()

    caches = [host(staged_k), host(staged_v)]
    new_len = C.kv_compact(caches, ora["retrieve"], ref["best_path"], ref["accept_len"],
                           x["prefix_len"], x["N"])
    assert np.array_equal(prefix.cpu().numpy(), new_len)
    assert np.array_equal(host(att.kc), caches[0]) and np.array_equal(host(att.vc), caches[1])

    # end to end against the oracle: committed row P + j of sequence b holds node r[j] of the
    # winning path -- its staged key within one rounding of the oracle's binary64 rotation,
    # its value exactly
    _, sk, sv = att.oracle(rows[:1])
    kc_now, vc_now = host(att.kc), host(att.vc)
    for b in range(w.B):
        P, G = int(x["prefix_len"][b]), int(ref["accept_len"][b]) + 1
        path = ora["retrieve"][ref["best_path"][b]][:G]
        assert staged_k_ratio(w, x, b, kc_now[b, :, P:P + G], sk[b][:, path], path) <= 1.0
        assert np.array_equal(vc_now[b, :, P:P + G], sv[b][:, path].astype(np.float32))
