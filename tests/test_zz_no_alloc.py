"""medusa_tree_attn_noalloc against medusa_tree_attn, through the C ABI: the same inputs
give the same output and cache rows, call after call, with the partials in the library's
own device array instead of a caller workspace."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import medusa_tree_attention_amd as M  # noqa: E402
from gpu_support import AttnRun, announce, compile_both, host  # noqa: E402


def _same_as_workspace_call(w, seed, prefix=None):
    lib, ora = compile_both(w)
    x = workloads.draw_round(w, seed=seed, prefix_len=prefix)
    ref = AttnRun(w, x, lib, ora)  # medusa_tree_attn with a caller workspace
    got = AttnRun(w, x, lib, ora)  # medusa_tree_attn_noalloc (its workspace stays unused)
    assert ref.run() == 0
    M.medusa_tree_attn_noalloc(got.q, got.kn, got.vn, got.kc, got.vc, got.td["depth"], got.td["mask"],
                               got.prefix, w.rope_base, got.out, got.status)
    torch.cuda.synchronize()
    assert int(got.status.item()) == 0
    assert torch.equal(ref.out, got.out), "outputs differ"
    assert torch.equal(ref.kc, got.kc) and torch.equal(ref.vc, got.vc), "staged cache rows differ"
    # and the output is the attention the oracle defines, on a sample of rows
    rows = [(b, u, h) for b in range(w.B) for u in (0, x["N"] - 1) for h in (0, w.Hq - 1)]
    out_ref, _, _ = got.oracle(rows)
    err = max(float(np.abs(host(got.out)[r] - out_ref[r]).max()) for r in rows)
    assert err <= (2e-2 if w.dtype == "bf16" else 1e-5)


def test_noalloc_matches_the_workspace_call_on_consecutive_calls():
    """Three calls in a row on one GPU: the batched workload (the largest split partials the
    array holds, four splits of two query blocks), then a smaller bf16 call with ragged
    prefixes and more splits per block, then the fp32 path (no partials)."""
    big = workloads.WORKLOADS["batched"]
    announce("no-allocation attention: batched workload")
    _same_as_workspace_call(big, seed=51)
    small = dataclasses.replace(big, B=2, Hq=8, Hkv=2)
    announce("no-allocation attention: smaller call after it")
    _same_as_workspace_call(small, seed=52, prefix=[3001, 777])
    announce("no-allocation attention: fp32 call")
    _same_as_workspace_call(workloads.WORKLOADS["tiny"], seed=53)


def test_scratch_bound_covers_the_largest_workspace():
    """Every shape's workspace fits the array: partials exist only for grids of at most
    256 workgroups of 128 rows."""
    bound = 256 * 128 * (16 + 128 * 2)
    for B, Hq, Hkv, N, P in [(4, 32, 8, 64, 4096), (1, 32, 8, 64, 8192), (1, 32, 32, 341, 4096),
                             (3, 8, 2, 64, 20000), (1, 4, 1, 5, 100000), (2, 64, 1, 64, 1000)]:
        assert M.medusa_tree_attn_workspace_size(M.BF16, B, Hq, Hkv, 128, N, P + N) <= bound
