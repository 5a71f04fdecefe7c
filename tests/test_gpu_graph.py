"""A whole round captured in one HIP graph and replayed.

The round: the Medusa head step from the carried state (h, root) -> candidates; tree
attention (RoPE at P + depth, staged rows, ancestor mask); greedy acceptance, compaction
and the frontier carry into (h, root) for the next round.  Every call enqueues kernels
only (no allocation, host copy or synchronisation), so torch.cuda.graph captures it, and
each replay runs one more round from the state the last one left.  The test replays the
graph several times, with eager work and synchronisations in between, and checks the full
state after every replay against the same number of eager rounds on a copy.
"""
import numpy as np
import pytest
import torch

import medusa_tree_attention_amd as M
import workloads

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_support import announce, dev  # noqa: E402

ROUNDS = 4


def make_state(seed=5):
    B, Hq, Hkv, d, P0, K, TOPK, V, H = 2, 8, 2, 128, 256, 4, 10, 2048, 256
    spec = workloads.tree_spec(workloads.WORKLOADS["batched"])
    tree = M.medusa_tree_compile(K, TOPK, rank_hit=spec["rank_hit"], n_nodes=spec["n_nodes"])
    N, W = tree["n_nodes"], tree["path_width"]
    S = P0 + N + ROUNDS * W
    rng = np.random.default_rng(seed)
    bf = lambda shape, s=1.0: dev(workloads.round_to_dtype(
        rng.standard_normal(shape, dtype=np.float32) * np.float32(s), "bf16"), torch.bfloat16)
    heads = workloads.draw_heads(seed, B, K, H, V)
    logits = rng.standard_normal((B, N, V), dtype=np.float32)
    const = {
        "q": bf((B, N, Hq, d)), "kn": bf((B, N, Hkv, d)), "vn": bf((B, N, Hkv, d)),
        "W1": dev(heads["W1"], torch.bfloat16), "W2": dev(heads["W2"], torch.bfloat16),
        "hidden": bf((B, N, H)), "logits": dev(logits),
        "depth": dev(tree["depth"]), "mask": dev(tree["tree_mask"].view(np.int64)),
        "tidx": dev(tree["tree_indices"]), "retrieve": dev(tree["retrieve"]),
        "attn_ws": torch.zeros(M.medusa_tree_attn_workspace_size(M.BF16, B, Hq, Hkv, d, N, S),
                               dtype=torch.uint8, device="cuda"),
        "acc_ws": torch.zeros(M.medusa_accept_workspace_size(B, N), dtype=torch.uint8, device="cuda"),
        "head_ws": torch.zeros(M.medusa_head_workspace_size(B, K, H, V), dtype=torch.uint8, device="cuda"),
        "topk": TOPK, "N": N, "W": W,
    }
    kc = np.zeros((B, Hkv, S, d), np.float32)
    vc = np.zeros_like(kc)
    kc[:, :, :P0] = rng.standard_normal((B, Hkv, P0, d), dtype=np.float32)
    vc[:, :, :P0] = rng.standard_normal((B, Hkv, P0, d), dtype=np.float32)
    state = {
        "kc": dev(workloads.round_to_dtype(kc, "bf16"), torch.bfloat16),
        "vc": dev(workloads.round_to_dtype(vc, "bf16"), torch.bfloat16),
        "prefix": dev(np.full(B, P0, np.int32)),
        "h": dev(heads["h"], torch.bfloat16), "root": dev(heads["root_tokens"]),
        "cand": torch.zeros((B, 1 + K * TOPK), dtype=torch.int32, device="cuda"),
        "out": torch.zeros((B, N, Hq, d), dtype=torch.bfloat16, device="cuda"),
        "best": torch.zeros(B, dtype=torch.int32, device="cuda"),
        "alen": torch.zeros(B, dtype=torch.int32, device="cuda"),
        "tokens": torch.zeros((B, W), dtype=torch.int32, device="cuda"),
        "frontier": torch.zeros(B, dtype=torch.int32, device="cuda"),
        "status": torch.zeros(1, dtype=torch.int32, device="cuda"),
    }
    return const, state


def one_round(c, s):
    M.medusa_head_candidates(s["h"], c["W1"], c["W2"], s["root"], s["cand"], s["status"], c["head_ws"],
                             c["topk"])
    M.medusa_tree_attn(c["q"], c["kn"], c["vn"], s["kc"], s["vc"], c["depth"], c["mask"], s["prefix"],
                       10000.0, s["out"], c["attn_ws"], s["status"])
    M.medusa_accept_commit(s["cand"], c["tidx"], c["retrieve"], s["best"], s["alen"], s["tokens"],
                           s["frontier"], [s["kc"]], [s["vc"]], s["prefix"], s["status"],
                           logits=c["logits"], workspace=c["acc_ws"], hidden=c["hidden"],
                           h_next=s["h"], next_root=s["root"])


def snapshot(s):
    return {k: v.clone() for k, v in s.items()}


def test_round_graph_replays_match_eager_rounds():
    announce("graph: capture one round (head step, attention, accept+commit+carry), replay")
    const, eager = make_state()
    graph_state = snapshot(eager)
    # eager reference rounds
    ref = []
    for _ in range(ROUNDS):
        one_round(const, eager)
        torch.cuda.synchronize()
        ref.append(snapshot(eager))
    assert int(eager["status"].item()) == 0
    lens = [int(r["prefix"][0].item()) for r in ref]
    announce(f"  eager prefix lengths of sequence 0 over the rounds: {lens}")
    # capture on the graph state (the capture itself runs nothing)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        one_round(const, graph_state)
    torch.cuda.synchronize()
    for r in range(ROUNDS):
        g.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 16, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for k, v in ref[r].items():
            assert torch.equal(graph_state[k], v), (r, k)
    announce(f"  {ROUNDS} replays equal the eager rounds")
