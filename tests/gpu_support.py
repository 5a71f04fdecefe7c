"""Shared set-up for the GPU parity tests: the same seeded inputs go to the
HIP library (through its C ABI) and to the CPU oracle."""
import numpy as np
import torch

import medusa_tree_attention_amd as M
import workloads
from oracle import accept as AC
from oracle import attention as A
from oracle import tree as T

DT = {"f32": torch.float32, "bf16": torch.bfloat16}
# max-abs error of attention outputs against the binary64 oracle
TOL = {"f32": 1e-5, "bf16": 2e-2}


def announce(msg):
    print(f"[gpu] {msg}", flush=True)


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device="cuda", dtype=dtype) if dtype is not None else t.to("cuda")


def host(t):
    return t.detach().to("cpu").float().numpy() if t.is_floating_point() else t.detach().cpu().numpy()


def compile_both(w):
    """The library's tree and the oracle's tree for a workload; they must be identical."""
    spec = workloads.tree_spec(w)
    if spec["paths"] is not None:
        lib = M.medusa_tree_compile(w.num_heads, w.topk, paths=spec["paths"])
        ora = T.compile_tree(spec["paths"], w.num_heads, w.topk)
    else:
        lib = M.medusa_tree_compile(w.num_heads, w.topk, rank_hit=spec["rank_hit"], n_nodes=spec["n_nodes"])
        ora = T.compile_greedy(spec["rank_hit"], spec["n_nodes"])
    assert np.array_equal(lib["tree_mask"], ora["mask_packed"])
    assert np.array_equal(lib["retrieve"], ora["retrieve"])
    return lib, ora


def tree_to_device(tree):
    return {"depth": dev(tree["depth"]), "mask": dev(tree["tree_mask"].view(np.int64)),
            "tree_indices": dev(tree["tree_indices"]), "retrieve": dev(tree["retrieve"])}


class AttnRun:
    """One medusa_tree_attn call on a workload's inputs, plus the oracle for chosen rows."""

    def __init__(self, w, x, lib_tree, ora_tree, status_init=0):
        """lib_tree feeds the device (library buffers); ora_tree feeds the oracle."""
        self.w, self.x, self.tree = w, x, ora_tree
        dt = DT[w.dtype]
        self.q, self.kn, self.vn = dev(x["q"], dt), dev(x["k_new"], dt), dev(x["v_new"], dt)
        self.kc, self.vc = dev(x["k_cache"], dt), dev(x["v_cache"], dt)
        self.td = tree_to_device(lib_tree)
        self.prefix = dev(x["prefix_len"])
        self.out = torch.full_like(self.q, 7.0)
        nbytes = M.medusa_tree_attn_workspace_size(
            M.F32 if w.dtype == "f32" else M.BF16, w.B, w.Hq, w.Hkv, w.d, x["N"], x["S_max"])
        self.ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device="cuda")
        self.status = torch.full((1,), status_init, dtype=torch.int32, device="cuda")

    def run(self):
        M.medusa_tree_attn(self.q, self.kn, self.vn, self.kc, self.vc, self.td["depth"],
                           self.td["mask"], self.prefix, self.w.rope_base, self.out, self.ws,
                           self.status)
        torch.cuda.synchronize()
        return int(self.status.item())

    def oracle(self, rows):
        x = self.x
        return A.tree_attention(x["q"], x["k_new"], x["v_new"], x["k_cache"], x["v_cache"],
                                x["prefix_len"], self.tree["depth"], self.tree["parent"],
                                self.w.rope_base, rows=rows)

    def check(self, rows):
        """Max-abs error of the chosen output rows, and the staged cache rows' error as a
        fraction of the bound their arithmetic allows (at most 1 passes)."""
        out_ref, sk, sv = self.oracle(rows)
        got = host(self.out)
        err = max(float(np.abs(got[b, u, h] - out_ref[b, u, h]).max()) for b, u, h in rows)
        kc, vc = host(self.kc), host(self.vc)
        N = self.x["N"]
        staged_err = 0.0
        for b in range(self.w.B):
            P = int(self.x["prefix_len"][b])
            gk, gv = kc[b, :, P:P + N], vc[b, :, P:P + N]
            staged_err = max(staged_err, staged_k_ratio(self.w, self.x, b, gk, sk[b], np.arange(N)))
            assert np.array_equal(gv, sv[b].astype(np.float32)), "staged V rows differ"
            # rows outside the staged block are untouched
            assert np.array_equal(kc[b, :, :P], self.x["k_cache"][b, :, :P])
            assert np.array_equal(kc[b, :, P + N:], self.x["k_cache"][b, :, P + N:])
        return err, staged_err


def staged_k_ratio(w, x, b, got, exact, nodes):
    """Largest error of staged key rows (of the given nodes, [Hkv][len(nodes)][d]) against the
    oracle's binary64 rotation, as a fraction of the bound the kernel's arithmetic allows."""
    d = w.d
    # |x1| + |x2| of the rotate-half pair each staged element is formed from
    kn = np.abs(x["k_new"][b].transpose(1, 0, 2).astype(np.float64))[:, nodes]
    pair = kn + np.roll(kn, d // 2, axis=-1)
    if w.dtype == "bf16":
        # rotated in fp32 (the phase angle is reduced in binary64 and rounded to fp32, about
        # pi 2^-24 rad, then sincosf; with two products and a sum the value is within
        # 2^-20 (|x1| + |x2|)), then rounded once to bf16 (unit roundoff 2^-8)
        bound = 2.0 ** -8 * np.abs(exact) + 2.0 ** -20 * pair
    else:
        # rotated in binary64 and rounded once to fp32 (unit roundoff 2^-24); each side's
        # binary64 angle at positions below ~8300 is within 3e-12 rad
        bound = 2.0 ** -24 * np.abs(exact) + 1e-11 * pair
    return float((np.abs(got - exact) / bound).max())


def sample_rows(w, N, n, seed=0, must=()):
    rng = np.random.default_rng(seed)
    rows = set(must)
    while len(rows) < n:
        rows.add((int(rng.integers(0, w.B)), int(rng.integers(0, N)), int(rng.integers(0, w.Hq))))
    return sorted(rows)


def oracle_accept(tree, candidates, logits=None, target_ids=None):
    return AC.accept_batch(tree, candidates, logits=logits, target_ids=target_ids)
