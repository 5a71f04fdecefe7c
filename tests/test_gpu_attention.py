"""Tree attention on the GPU against the binary64 oracle (through the C ABI)."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from gpu_support import TOL, AttnRun, announce, compile_both, host  # noqa: E402


def _all_rows(w, N):
    return [(b, u, h) for b in range(w.B) for u in range(N) for h in range(w.Hq)]


@pytest.mark.parametrize("name", ["tiny", "llama7b", "gqa8b", "wide", "batched"])
def test_workload_attention(name):
    """Every output row of every workload, in the launch configuration the benchmark
    times, against the binary64 per-path oracle."""
    w = workloads.WORKLOADS[name]
    announce(f"attention workload={name}")
    lib, ora = compile_both(w)
    x = workloads.draw_round(w)
    N = x["N"]
    run = AttnRun(w, x, lib, ora)
    assert run.run() == 0
    rows = _all_rows(w, N)
    announce(f"  oracle over all {len(rows)} rows")
    err, staged = run.check(rows)
    announce(f"  max abs err {err:.3e}, staged-row error {staged:.3f} of its bound")
    assert err <= TOL[w.dtype]
    assert staged <= 1.0


EDGE = {
    # root-only tree, an empty prefix next to a ragged one
    "root_only_f32": (dataclasses.replace(workloads.WORKLOADS["tiny"], B=2, tree="greedy",
                                          n_nodes=1, d=64), [0, 77]),
    "root_only_bf16": (dataclasses.replace(workloads.WORKLOADS["llama7b"], B=2, Hq=4, Hkv=2,
                                           n_nodes=1), [0, 130]),
    # ragged prefixes not multiple of 64, GQA group 4, small tree
    "ragged_gqa": (dataclasses.replace(workloads.WORKLOADS["batched"], B=3, Hq=8, Hkv=2,
                                       tree="cartesian", branching=(2, 2), num_heads=2, topk=2,
                                       slack=5), [1, 64, 200]),
    # d_h = 64 in bf16, mask spanning two words (N = 100)
    "d64_two_words": (dataclasses.replace(workloads.WORKLOADS["llama7b"], B=2, Hq=4, Hkv=1, d=64,
                                          n_nodes=100), [37, 300]),
    # matrix-core path with many prefix splits, an empty prefix, splits with no keys,
    # a split count that breaks the XCD grouping, and two staged tiles
    "mfma_splits_ragged": (dataclasses.replace(workloads.WORKLOADS["batched"], B=3, Hq=8, Hkv=2),
                           [0, 700, 3001]),
    # matrix-core path with a query block that is not a multiple of 64 rows (N * group = 20)
    "mfma_partial_qtile": (dataclasses.replace(workloads.WORKLOADS["batched"], B=2, Hq=4, Hkv=1,
                                               n_nodes=5), [257, 31]),
    # d_h = 64 in bf16 on the matrix-core path (padded to the 128-wide layout): the
    # benchmark's launch shape (four key-range splits and their merge), one split (the
    # output stored directly), and a 20-deep chain (RoPE frequencies of the shorter head)
    "mfma_d64_batched": (dataclasses.replace(workloads.WORKLOADS["batched"], d=64), [4096, 4096, 4096, 4096]),
    "mfma_d64_single_split": (dataclasses.replace(workloads.WORKLOADS["batched"], B=2, Hq=8, Hkv=2, d=64,
                                                  slack=3), [40, 200]),
    "mfma_d64_chain": (dataclasses.replace(workloads.WORKLOADS["batched"], B=2, Hq=8, Hkv=2, d=64,
                                           tree="cartesian", branching=(1,) * 20, num_heads=20, topk=1),
                       [300, 1000]),
    # matrix-core path with GQA groups that are not powers of two (query rows split into
    # node and head by a run-time divisor): 3 over two query blocks, 5 with d_h = 64 over
    # three, 7 over four with a single sequence
    "mfma_group3": (dataclasses.replace(workloads.WORKLOADS["batched"], B=3, Hq=6, Hkv=2), [900, 2500, 17]),
    "mfma_group5_d64": (dataclasses.replace(workloads.WORKLOADS["batched"], B=2, Hq=10, Hkv=2, d=64),
                        [1234, 640]),
    "mfma_group7": (dataclasses.replace(workloads.WORKLOADS["batched"], B=1, Hq=7, Hkv=1), [3000]),
    # matrix-core path with more tree nodes than threads in a workgroup (600: the node depths
    # are checked and cached in a second pass) and ragged prefixes
    "mfma_600_nodes": (dataclasses.replace(workloads.WORKLOADS["batched"], B=2, Hq=2, Hkv=1, n_nodes=600,
                                           use_logits=False, vocab=16), [100, 333]),
    # matrix-core path with more tree rows than the LDS depth cache holds (4161 > 4096: the
    # staged-row fixes read the depths from memory), 66 visibility words per row
    "mfma_4161_rows": (dataclasses.replace(workloads.WORKLOADS["batched"], B=1, Hq=1, Hkv=1, tree="cartesian",
                                           branching=(64, 64), num_heads=2, topk=64, use_logits=False,
                                           vocab=128), [77]),
    # a chain: ordinary causal attention over prefix + path
    "chain_f32": (dataclasses.replace(workloads.WORKLOADS["tiny"], Hq=2, Hkv=1, d=128,
                                      branching=(1, 1, 1, 1), num_heads=4, topk=1), [65]),
}


@pytest.mark.parametrize("case", list(EDGE))
def test_edge_cases(case):
    w, P = EDGE[case]
    announce(f"attention edge case={case}")
    lib, ora = compile_both(w)
    x = workloads.draw_round(w, seed=11, prefix_len=P)
    run = AttnRun(w, x, lib, ora)
    assert run.run() == 0
    err, staged = run.check(_all_rows(w, x["N"]))
    assert err <= TOL[w.dtype] and staged <= 1.0


def test_capacity_violation_stores_nothing():
    w = dataclasses.replace(workloads.WORKLOADS["tiny"], B=2)
    announce("attention capacity violation")
    lib, ora = compile_both(w)
    x = workloads.draw_round(w, seed=3, prefix_len=[10, 128])
    x["prefix_len"] = np.array([10, 129], np.int32)   # 129 + 7 > S_max = 135
    run = AttnRun(w, x, lib, ora)
    kc0, out0 = host(run.kc).copy(), host(run.out).copy()
    assert run.run() == -3
    assert np.array_equal(host(run.kc), kc0) and np.array_equal(host(run.out), out0)


def test_sticky_status_skips_the_call():
    w = workloads.WORKLOADS["tiny"]
    announce("attention with a failed round")
    lib, ora = compile_both(w)
    x = workloads.draw_round(w)
    run = AttnRun(w, x, lib, ora, status_init=-1)
    kc0, out0 = host(run.kc).copy(), host(run.out).copy()
    assert run.run() == -1
    assert np.array_equal(host(run.kc), kc0) and np.array_equal(host(run.out), out0)


def test_host_rejects_bad_shapes():
    import medusa_tree_attention_amd as M
    w = workloads.WORKLOADS["tiny"]
    lib, ora = compile_both(w)
    x = workloads.draw_round(w)
    run = AttnRun(w, x, lib, ora)
    bad_q = torch.zeros((1, 7, 1, 96), device="cuda")
    with pytest.raises(M.MedusaError) as e:
        M.medusa_tree_attn(bad_q, run.kn, run.vn, run.kc, run.vc, run.td["depth"], run.td["mask"],
                           run.prefix, 1e4, bad_q, run.ws, run.status)
    assert e.value.name == "MEDUSA_EUNSUPPORTED"


def test_repeated_calls_reuse_the_workspace():
    """A second call on the same workspace (holding the first call's split partials)
    gives the same output bit for bit."""
    w = workloads.WORKLOADS["batched"]
    announce("attention twice on one workspace")
    lib, ora = compile_both(w)
    x = workloads.draw_round(w, seed=21)
    run = AttnRun(w, x, lib, ora)
    assert run.run() == 0
    first = run.out.clone()
    run.out.fill_(3.0)
    run.kc.copy_(torch.from_numpy(x["k_cache"]).to("cuda", torch.bfloat16))
    assert run.run() == 0
    assert torch.equal(first, run.out)


@pytest.mark.parametrize("amp", [6, 16])
def test_running_maximum_moves_inside_the_key_stream(amp):
    """Committed keys whose scale climbs from 1 to `amp` along each quarter of the context (a
    sawtooth), values at unit scale: the largest score of a key range grows by far more than
    the 2^8 slack (about 3 to 70 in log2 units), so the running maximum moves, with O and l
    rescaled, in the middle of every workgroup's key stream, and the softmax is peaked.  A
    tile mishandled around a move is off by a factor of at least 2^8 and shows as an error
    of order |v|.

    Precision: a score is q~ . k with |q~||k| up to about 16 sqrt(d_h) here.  The kernel
    carries q~ as a hi/lo pair of bf16 operands (exact to about 2^-17), so the score error is
    far below what a peaked softmax would pass on; what remains is the bf16 rounding of the
    output (half an ulp, 2^-9 of |o| up to 2^-8) and of the probabilities.  Every row is
    compared."""
    w = dataclasses.replace(workloads.WORKLOADS["batched"], B=2, Hq=8, Hkv=2)
    announce(f"attention with a climbing score scale to {amp} (running-maximum moves), unit-scale V")
    lib, ora = compile_both(w)
    x = workloads.draw_round(w, seed=31, prefix_len=[4096, 3001])
    scale = 1.0 + (amp - 1.0) * (np.arange(x["S_max"]) % 1024) / 1024
    x["k_cache"] = workloads.round_to_dtype(
        x["k_cache"] * scale[None, None, :, None].astype(np.float32), w.dtype)
    run = AttnRun(w, x, lib, ora)
    assert run.run() == 0
    err, staged = run.check(_all_rows(w, x["N"]))
    announce(f"  max abs err {err:.3e}")
    assert err <= TOL[w.dtype] and staged <= 1.0


def test_deepest_supported_chain_and_the_first_unsupported_depth():
    """The matrix-core path keeps RoPE phases for depths 0..31.  A chain 31 deep (32 rows,
    positions P .. P + 31) must verify like causal attention over the prefix and the path;
    a chain 32 deep must fail the round on the device with MEDUSA_EUNSUPPORTED and store
    nothing to the cache or the output."""
    base = dataclasses.replace(workloads.WORKLOADS["batched"], B=2, Hq=8, Hkv=2, tree="cartesian", topk=1)
    w = dataclasses.replace(base, branching=(1,) * 31, num_heads=31)
    announce("attention: a 31-deep chain (the deepest RoPE phase kept)")
    lib, ora = compile_both(w)
    x = workloads.draw_round(w, seed=41, prefix_len=[300, 1000])
    run = AttnRun(w, x, lib, ora)
    assert run.run() == 0
    err, staged = run.check(_all_rows(w, x["N"]))
    announce(f"  max abs err {err:.3e}")
    assert err <= TOL[w.dtype] and staged <= 1.0

    w = dataclasses.replace(base, branching=(1,) * 32, num_heads=32)
    announce("attention: a 32-deep chain is rejected on the device")
    lib, ora = compile_both(w)
    x = workloads.draw_round(w, seed=42, prefix_len=[300, 1000])
    run = AttnRun(w, x, lib, ora)
    kc0, vc0, out0 = host(run.kc).copy(), host(run.vc).copy(), host(run.out).copy()
    assert run.run() == -4  # MEDUSA_EUNSUPPORTED
    assert np.array_equal(host(run.kc), kc0) and np.array_equal(host(run.vc), vc0)
    assert np.array_equal(host(run.out), out0)


def test_batch_of_more_than_64_sequences():
    """70 sequences on the matrix-core path: the prefix lengths are checked 64 per pass, so a
    sequence past the first 64 that does not fit must fail the round (no stores), and a
    fitting batch must match the oracle on every row of every sequence."""
    w = dataclasses.replace(workloads.WORKLOADS["batched"], B=70, Hq=4, Hkv=1, tree="cartesian",
                            branching=(2, 2), num_heads=2, topk=2, slack=3)
    announce("attention with 70 sequences")
    lib, ora = compile_both(w)
    rng = np.random.default_rng(43)
    prefix = [int(p) for p in rng.integers(0, 250, size=w.B)]
    x = workloads.draw_round(w, seed=43, prefix_len=prefix)
    run = AttnRun(w, x, lib, ora)
    assert run.run() == 0
    N = x["N"]
    err, staged = run.check(_all_rows(w, N))
    announce(f"  max abs err {err:.3e}")
    assert err <= TOL[w.dtype] and staged <= 1.0

    x["prefix_len"] = x["prefix_len"].copy()
    x["prefix_len"][67] = x["S_max"] - N + 1  # sequence 67 has no room for its staged rows
    run = AttnRun(w, x, lib, ora)
    kc0, out0 = host(run.kc).copy(), host(run.out).copy()
    assert run.run() == -3  # MEDUSA_ECAPACITY
    assert np.array_equal(host(run.kc), kc0) and np.array_equal(host(run.out), out0)
