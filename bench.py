#!/usr/bin/env python3
"""Throughput of one Medusa tree-verification round on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload batched]

A step is one whole round over one batch of synthetic inputs already resident
in HBM.  By default (``--round verify``) that is ``medusa_tree_attn`` (RoPE at P + depth, staged K/V rows, tree
attention) and ``medusa_accept_commit`` (greedy acceptance over fp32 target logits and the
winning-path K/V gather in one call; ``--commit separate`` uses ``medusa_accept`` then
``medusa_kv_compact``), on one stream with no host synchronisation.  ``--round full`` runs the batched full round: the Medusa head
step ``medusa_head_candidates`` (W2 (SiLU(W1 h) + h) for four heads, top-10 of
each, candidate rows written on the device) comes first in every step and
fills the candidates that the acceptance reads.  The tree itself is compiled once on the host before the
timed region (the buffers are static for a tree shape) and its compile time
is reported separately.

Each step uses the next of several independent buffer sets (cache, Q, K/V,
logits, outputs), together larger than the 256 MB Infinity Cache, so the KV
stream is served from HBM.  Compaction advances the prefix lengths, so every
step gets its own prefix-length and status block, filled before timing: every
round runs at the same context length and the timed loop holds library calls
only.

Printed on stdout: one JSON line.  ``value`` = verified tree nodes per second
over the timed steps (B * N per step).  ``roofline`` rates the attention call
(the dominant kernels: attention and split merge): algorithmic bytes per call /
mean call time from HIP events recorded by the two dispatches, against 8 TB/s.  ``cpu_baseline`` times the CPU
oracle on one round of the same workload.  With ``--round full`` the head call
is the dominant one and ``roofline`` rates it (weights, h and candidate rows per
call); the attention figures move to ``attention_roofline``.
"""
import argparse
import ctypes
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
EVENT_EVERY = 4  # timed steps per attention (and head) call that records timing events
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix rate (published)
ATTN_SOURCES = ["attn.hip", "attn_mfma.hip", "attn_common.h", "common.h"]
HEAD_SOURCES = ["heads.hip", "common.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_traffic_batched.md")
HEAD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "head_step_traffic_batched.md")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "medusa_tree_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def attn_source_hash():
    return source_hash(ATTN_SOURCES)


def head_source_hash():
    return source_hash(HEAD_SOURCES)


def algorithmic_flops(w, N):
    """Matrix FLOPs of the attention call: Q K^T and P V over every committed and staged key,
    4 d_h Hq N (P + N) B (the masked staged pairs included, as the matrix cores compute them)."""
    return 4 * w.d * w.Hq * N * (w.P + N) * w.B


def algorithmic_bytes(w, N, esize):
    """Bytes the attention call must move: prefix K/V once, Q, K_new/V_new, staged K/V, O."""
    prefix_kv = 2 * w.B * w.Hkv * w.P * w.d * esize
    q = o = w.B * N * w.Hq * w.d * esize
    new_kv = staged = 2 * w.B * N * w.Hkv * w.d * esize
    return prefix_kv + q + new_kv + staged + o


def head_algorithmic_bytes(B, K, hidden, V, topk):
    """Bytes the head step must move: both weight sets of every head once, h, the root
    tokens and the candidate rows (the u vectors and the logits are intermediates)."""
    return 2 * K * (hidden * hidden + V * hidden) + 2 * B * hidden + 4 * B + 4 * B * (1 + K * topk)


def measured_traffic(src_hash, path=TRAFFIC_FILE):
    """HBM bytes per call from a committed rocprofv3 counter summary, if it was taken on the
    current kernel sources."""
    if not os.path.exists(path):
        return None
    text = open(path, encoding="utf-8").read()
    m_hash = re.search(r"kernel source hash:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"scaled HBM bytes per launch:\s*([0-9]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != src_hash:
        return None
    return int(m_bytes.group(1))


class HipEvents:
    """hipEvent_t handles through the HIP runtime torch has loaded."""

    def __init__(self):
        import torch  # noqa: F401  (loads the runtime first)
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        assert self.hip.hipEventCreateWithFlags(ctypes.byref(ev), 0) == 0
        return ev.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, ev):
        self.hip.hipEventDestroy(ev)


def build_sets(w, x, tree, n_sets, torch, M):
    import numpy as np
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dcode = M.BF16 if w.dtype == "bf16" else M.F32
    N = x["N"]
    dev = lambda a, d=None: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", d)
    shared = {"depth": dev(tree["depth"]), "mask": dev(tree["tree_mask"].view(np.int64)),
              "tidx": dev(tree["tree_indices"]), "retrieve": dev(tree["retrieve"])}
    pristine = dev(np.concatenate([x["prefix_len"], [0]]).astype(np.int32))
    attn_ws = M.medusa_tree_attn_workspace_size(dcode, w.B, w.Hq, w.Hkv, w.d, N, x["S_max"])
    acc_ws = M.medusa_accept_workspace_size(w.B, N)
    sets = []
    for _ in range(n_sets):
        s = {"q": dev(x["q"], dt), "kn": dev(x["k_new"], dt), "vn": dev(x["v_new"], dt),
             "kc": dev(x["k_cache"], dt), "vc": dev(x["v_cache"], dt),
             "logits": dev(x["logits"]) if x["logits"] is not None else None,
             "tids": dev(x["target_ids"]) if x["target_ids"] is not None else None,
             "cand": dev(x["candidates"])}
        s["out"] = torch.empty_like(s["q"])
        s["attn_ws"] = torch.zeros(max(attn_ws, 16), dtype=torch.uint8, device="cuda")
        s["acc_ws"] = torch.zeros(acc_ws, dtype=torch.uint8, device="cuda")
        s["best"] = torch.zeros(w.B, dtype=torch.int32, device="cuda")
        s["alen"] = torch.zeros(w.B, dtype=torch.int32, device="cuda")
        s["frontier"] = torch.zeros(w.B, dtype=torch.int32, device="cuda")
        s["tokens"] = torch.zeros((w.B, tree["path_width"]), dtype=torch.int32, device="cuda")
        sets.append(s)
    return shared, pristine, sets


def set_bytes(s):
    return sum(t.numel() * t.element_size() for t in s.values() if hasattr(t, "numel") and t is not None)


def cpu_model():
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.machine()


def read_ceiling_gbs(torch, M):
    """Practical read bandwidth of this GPU: the library's streaming-read probe over 1 GiB
    (four times the Infinity Cache), timed with events on torch's stream, where it runs."""
    x = torch.ones(2 ** 28, dtype=torch.float32, device="cuda")
    sink = torch.zeros(M.medusa_read_probe_sink_size() // 4, dtype=torch.int32, device="cuda")
    for _ in range(3):
        M.medusa_read_probe(x, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        M.medusa_read_probe(x, sink)
    e1.record()
    e1.synchronize()
    sec = e0.elapsed_time(e1) / 10 * 1e-3
    del x
    return 2 ** 30 / sec / 1e9


# The CPU oracle runs in a child process started before this process makes any HIP call (a
# process that has initialised the GPU is never forked or replaced); the child spreads the
# per-path attention over a pool of forked workers, one BLAS thread each.
_CPU_CTX = {}


def _oracle_rows(rows):
    """Worker: the oracle's attention outputs for a chunk of (b, u, h) rows."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as A
    x, ora, base = _CPU_CTX["x"], _CPU_CTX["ora"], _CPU_CTX["rope_base"]
    with threadpool_limits(limits=1):
        out, _, _ = A.tree_attention(x["q"], x["k_new"], x["v_new"], x["k_cache"], x["v_cache"],
                                     x["prefix_len"], ora["depth"], ora["parent"], base, rows=rows)
    return [(r, out[r]) for r in rows]


def _oracle_round(w, x, xh, pool, n_chunks):
    """One round through the oracle: the head step (given its inputs), tree compile, every
    row's per-path attention (over the pool, or in this process), greedy acceptance and
    the compaction of the staged rows."""
    import numpy as np

    import workloads
    from oracle import accept as AC
    from oracle import attention as A
    from oracle import compact as C
    from oracle import heads as HD
    from oracle import tree as T

    spec = workloads.tree_spec(w)
    cand = x["candidates"]
    if xh is not None:
        cand = HD.head_candidates(xh["h"], xh["W1"], xh["W2"], xh["root_tokens"], w.topk)["candidates"]
    ora = (T.compile_tree(spec["paths"], w.num_heads, w.topk) if spec["paths"] is not None
           else T.compile_greedy(spec["rank_hit"], spec["n_nodes"]))
    rows = [(b, u, h) for b in range(w.B) for u in range(x["N"]) for h in range(w.Hq)]
    if pool is None:
        _, sk, sv = A.tree_attention(x["q"], x["k_new"], x["v_new"], x["k_cache"], x["v_cache"],
                                     x["prefix_len"], ora["depth"], ora["parent"], w.rope_base)
    else:
        # the workers were forked with the inputs and this same tree in _CPU_CTX
        chunks = [rows[i::n_chunks] for i in range(n_chunks)]
        out = np.full((w.B, x["N"], w.Hq, w.d), np.nan)
        for part in pool.map(_oracle_rows, chunks):
            for r, v in part:
                out[r] = v
        # the staged K/V rows (no attention rows) for the compaction
        _, sk, sv = A.tree_attention(x["q"], x["k_new"], x["v_new"], x["k_cache"], x["v_cache"],
                                     x["prefix_len"], ora["depth"], ora["parent"], w.rope_base, rows=[])
    res = AC.accept_batch(ora, cand, logits=x["logits"], target_ids=x["target_ids"])
    cache = [np.array(x["k_cache"], np.float64), np.array(x["v_cache"], np.float64)]
    for b in range(w.B):
        P = int(x["prefix_len"][b])
        for c, st in zip(cache, (sk, sv)):
            c[b, :, P:P + x["N"]] = st[b]
    C.kv_compact(cache, ora["retrieve"], res["best_path"], res["accept_len"], x["prefix_len"], x["N"])


def cpu_baseline_child(w, full_round):
    """The CPU oracle, as it stands, on one full round of the workload: on every core this
    process may use (a pool of forked workers, capped at 16, the machine's CPU share per GPU),
    and on one thread."""
    import multiprocessing

    from threadpoolctl import threadpool_info, threadpool_limits

    import workloads
    x = workloads.draw_round(w)
    xh = workloads.draw_heads(w.seed + 300, w.B, w.num_heads, w.Hq * w.d, w.vocab) if full_round else None
    affinity = len(os.sched_getaffinity(0))
    workers = max(1, min(affinity, 16))
    from oracle import tree as T
    spec = workloads.tree_spec(w)
    _CPU_CTX.update(x=x, rope_base=w.rope_base,
                    ora=(T.compile_tree(spec["paths"], w.num_heads, w.topk) if spec["paths"] is not None
                         else T.compile_greedy(spec["rank_hit"], spec["n_nodes"])))
    with multiprocessing.get_context("fork").Pool(workers) as pool:
        pool.map(abs, range(workers))  # workers started before the timed region
        with threadpool_limits(limits=workers):  # the head step's matrix products in this process
            t0 = time.perf_counter()
            _oracle_round(w, x, xh, pool, 4 * workers)
            dt_all = time.perf_counter() - t0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        _oracle_round(w, x, xh, None, 1)
        dt_one = time.perf_counter() - t0
    blas = sorted({i.get("internal_api", "?") + ":" + str(i.get("num_threads")) for i in threadpool_info()})
    nodes = w.B * x["N"]
    return {"value": nodes / dt_all, "unit": "nodes/s", "cores": workers, "kind": "oracle",
            "affinity_cores": affinity, "blas_threads_per_worker": 1, "blas": blas,
            "cpu_model": cpu_model(), "seconds": dt_all,
            "single_thread": {"value": nodes / dt_one, "seconds": dt_one},
            "sample": (f"one full round of the workload ({w.B} sequences x {x['N']} nodes x {w.Hq} heads at "
                       f"P={w.P}): " + ("binary64 head step (4 heads, top-k), " if full_round else "")
                       + f"tree compile, per-path binary64 attention of every row over {workers} forked "
                       f"workers (one BLAS thread each), greedy accept, compaction; {dt_all:.2f} s "
                       f"({dt_one:.1f} s on one thread) on {cpu_model()}")}


def run_cpu_baseline(args):
    """Start the oracle baseline as a child process (before any HIP call here) and return its
    JSON record, or None if it failed."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--cpu-baseline-child", "--workload", args.workload,
           "--prefix", str(args.prefix), "--round", args.round]
    log("[bench] timing the CPU oracle on one round (child process) ...")
    r = subprocess.run(cmd, capture_output=True, text=True)
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    if r.returncode != 0 or not lines:
        log(f"[bench] CPU baseline failed ({r.returncode}): {r.stderr[-500:]}")
        return None
    return json.loads(lines[-1])


def budget_sweep(args, np, torch, M, workloads):
    """Per-layer attention cost of the greedy trees T_N at several contexts P, and the node
    budget medusa_tree_budget picks from it for each P.  The per-round fixed cost is the
    backbone weight stream (--backbone-gb) at the read ceiling measured in the same run."""
    import dataclasses
    base = workloads.WORKLOADS[args.workload]
    spec = workloads.tree_spec(base)
    if spec["rank_hit"] is None:
        raise SystemExit("--budget needs a workload whose tree grows from a rank-hit table")
    nodes = [8, 16, 24, 32, 48, 64, 96, 128]
    contexts = [1024, 4096, 16384]
    layers = 32
    ceiling = read_ceiling_gbs(torch, M)
    fixed_us = args.backbone_gb * 1e9 / (ceiling * 1e9) * 1e6
    ev = HipEvents()
    e0, e1 = ev.create(), ev.create()
    sptr = torch.cuda.current_stream().cuda_stream
    dt = torch.bfloat16 if base.dtype == "bf16" else torch.float32
    dcode = M.BF16 if base.dtype == "bf16" else M.F32
    out = {}
    for P in contexts:
        w = dataclasses.replace(base, P=P, n_nodes=max(nodes))
        x = workloads.draw_round(w, seed=w.seed + 500)
        S = x["S_max"]
        per_set = 2 * w.B * w.Hkv * S * w.d * (2 if dt == torch.bfloat16 else 4)
        n_sets = max(2, -(-512 * 2 ** 20 // per_set))
        kc = [torch.from_numpy(x["k_cache"]).to("cuda", dt) for _ in range(n_sets)]
        vc = [torch.from_numpy(x["v_cache"]).to("cuda", dt) for _ in range(n_sets)]
        times = []
        for N in nodes:
            tree = M.medusa_tree_compile(w.num_heads, w.topk, rank_hit=spec["rank_hit"], n_nodes=N)
            q = torch.from_numpy(np.ascontiguousarray(x["q"][:, :N])).to("cuda", dt)
            kn = torch.from_numpy(np.ascontiguousarray(x["k_new"][:, :N])).to("cuda", dt)
            vn = torch.from_numpy(np.ascontiguousarray(x["v_new"][:, :N])).to("cuda", dt)
            depth = torch.from_numpy(tree["depth"]).to("cuda")
            mask = torch.from_numpy(tree["tree_mask"].view(np.int64)).to("cuda")
            o = torch.empty_like(q)
            ws = torch.zeros(max(M.medusa_tree_attn_workspace_size(dcode, w.B, w.Hq, w.Hkv, w.d, N, S), 16),
                             dtype=torch.uint8, device="cuda")
            ctl = torch.from_numpy(np.concatenate([x["prefix_len"], [0]]).astype(np.int32)).to("cuda")
            lib = M.load()
            reps, warm = 30, 5
            ms = []
            for r in range(warm + reps):
                k, v = kc[r % n_sets], vc[r % n_sets]
                rc = lib.medusa_tree_attn(sptr, dcode, w.B, w.Hq, w.Hkv, w.d, N, depth.data_ptr(),
                                          mask.data_ptr(), tree["mask_words"], ctl.data_ptr(), q.data_ptr(),
                                          kn.data_ptr(), vn.data_ptr(), k.data_ptr(), v.data_ptr(), S,
                                          float(w.rope_base), o.data_ptr(), ws.data_ptr(), ws.numel(),
                                          ctl[w.B:].data_ptr(), e0, e1)
                if rc:
                    raise RuntimeError(f"medusa_tree_attn failed ({rc}) at P={P} N={N}")
                torch.cuda.synchronize()
                if r >= warm:
                    ms.append(ev.elapsed_ms(e0, e1))
            if int(ctl[w.B].item()) != 0:
                raise RuntimeError(f"device status {int(ctl[w.B].item())} at P={P} N={N}")
            times.append(float(np.median(ms)) * 1e3)
            log(f"[bench] budget sweep P={P} N={N}: attention {times[-1]:.2f} us")
        best, et, rt = M.medusa_tree_budget(spec["rank_hit"], nodes, times, fixed_us, layers)
        out[str(P)] = {"attention_us": dict(zip(map(str, nodes), times)), "best_n": best,
                       "expected_tokens": float(et[best]),
                       "tokens_per_s_per_sequence": float(rt[best]) * 1e6,
                       "tokens_per_s_at_64": float(rt[64]) * 1e6 if len(rt) > 64 else None}
        log(f"[bench] budget P={P}: best N={best} ({et[best]:.3f} tokens per round, "
            f"{rt[best] * 1e6:.1f} tokens/s per sequence; N=64: {rt[64] * 1e6:.1f})")
        del kc, vc
        torch.cuda.empty_cache()
    ev.destroy(e0)
    ev.destroy(e1)
    print(json.dumps({"metric": "node budget per context (medusa_tree_budget over measured attention cost)",
                      "workload": f"{base.name}: B={base.B}, Hq={base.Hq}, Hkv={base.Hkv}, d_h={base.d}, "
                                  f"greedy trees from the K={base.num_heads}, TOPK={base.topk} rank table",
                      "layers": layers, "backbone_gb": args.backbone_gb, "read_ceiling_gbs": ceiling,
                      "fixed_us": fixed_us, "nodes": nodes, "contexts": out}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # untimed steps first: on MI355X the attention call settles about 2.5 us lower only after
    # some hundreds of steps of sustained work (measured over the timed steps after 20 warm-up
    # steps: 44.6 us, after 300: 42.4 us, after 1000: 42.0 us), so the default warm-up runs 500
    # (about 30 ms)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", default="batched")
    ap.add_argument("--prefix", type=int, default=0,
                    help="override the workload's context length P (secondary runs, e.g. llama7b at 4096)")
    ap.add_argument("--accept", choices=["greedy", "typical"], default="greedy",
                    help="acceptance rule of the round (typical: temperature 1, epsilon 0.3, alpha 0.09)")
    ap.add_argument("--commit", choices=["fused", "separate"], default="fused",
                    help="greedy rounds: accept and compact in one call (fused) or two")
    ap.add_argument("--graph", action=argparse.BooleanOptionalAction, default=True,
                    help="also time the same number of steps replayed from one captured HIP graph "
                         "(reported beside the eager figure, which stays the value)")
    ap.add_argument("--budget", action="store_true",
                    help="sweep the attention call over tree sizes and contexts and choose the node "
                         "budget per context (medusa_tree_budget); prints its own JSON line")
    ap.add_argument("--backbone-gb", type=float, default=16.0,
                    help="--budget: backbone weight bytes streamed once per round (GB)")
    ap.add_argument("--round", choices=["verify", "full"], default="verify",
                    help="full: the Medusa head step fills the candidates first in every step")
    ap.add_argument("--sets", type=int, default=0, help="buffer sets to rotate (0: enough for > 512 MB)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (for HBM counter scaling)")
    ap.add_argument("--cpu-baseline-child", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.cpu_baseline_child:  # the oracle baseline in a process that never touches the GPU
        import dataclasses

        import workloads
        w = workloads.WORKLOADS[args.workload]
        if args.prefix:
            w = dataclasses.replace(w, P=args.prefix)
        print(json.dumps(cpu_baseline_child(w, args.round == "full")), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the round is measured per GPU; see DESIGN.md for how it would shard)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import medusa_tree_attention_amd as M
    import workloads

    if args.budget:
        budget_sweep(args, np, torch, M, workloads)
        return
    w = workloads.WORKLOADS[args.workload]
    if args.prefix:
        import dataclasses
        w = dataclasses.replace(w, P=args.prefix)
    spec = workloads.tree_spec(w)
    # the CPU oracle first, in a child process, before this process makes any HIP call
    cpu_record = None if args.no_cpu else run_cpu_baseline(args)
    M.load()  # the library's first load is not part of the compile time
    t0 = time.perf_counter()
    tree = (M.medusa_tree_compile(w.num_heads, w.topk, paths=spec["paths"]) if spec["paths"] is not None
            else M.medusa_tree_compile(w.num_heads, w.topk, rank_hit=spec["rank_hit"], n_nodes=spec["n_nodes"]))
    compile_us = (time.perf_counter() - t0) * 1e6
    x = workloads.draw_round(w)
    N = x["N"]
    torch.cuda.init()
    shared, pristine, sets = build_sets(w, x, tree, 1, torch, M)
    per_set = set_bytes(sets[0])
    n_sets = args.sets or max(2, -(-512 * 2 ** 20 // per_set))
    shared, pristine, sets = build_sets(w, x, tree, n_sets, torch, M)
    log(f"[bench] workload={w.name} N={N} sets={n_sets} x {per_set / 2**20:.1f} MiB")
    xh = heads = None
    hidden = w.Hq * w.d
    if args.round == "full":
        # one copy of the head weights (1.18 GB at hidden 4096, V 32000: four times the
        # Infinity Cache, so every step reads them from HBM)
        xh = workloads.draw_heads(w.seed + 300, w.B, w.num_heads, hidden, w.vocab)
        hb = M.medusa_head_workspace_size(w.B, w.num_heads, hidden, w.vocab)
        heads = {"h": torch.from_numpy(xh["h"]).to("cuda", torch.bfloat16),
                 "W1": torch.from_numpy(xh["W1"]).to("cuda", torch.bfloat16),
                 "W2": torch.from_numpy(xh["W2"]).to("cuda", torch.bfloat16),
                 "root": torch.from_numpy(xh["root_tokens"]).to("cuda"),
                 "ws": torch.zeros(hb, dtype=torch.uint8, device="cuda")}
        log(f"[bench] head step: K={w.num_heads} hidden={hidden} V={w.vocab} topk={w.topk}")

    lib = M.load()
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    dcode = M.BF16 if w.dtype == "bf16" else M.F32
    nn = tree["n_paths"]
    width = tree["path_width"]
    p = lambda t: None if t is None else t.data_ptr()

    # Every step gets its own control block (prefix lengths P_b, then the status word),
    # filled with the round's initial values before timing: compaction advances P_b by the
    # accepted count, and a fresh block per step keeps every step at the same P without a
    # reset copy inside the timed loop.  Argument tuples are built up front as well, so the
    # timed loop only calls into the library.
    total = args.warmup + args.steps
    fused = args.accept == "greedy" and args.commit == "fused"
    kc_arrs = [(ctypes.c_void_p * 1)(s["kc"].data_ptr()) for s in sets]
    vc_arrs = [(ctypes.c_void_p * 1)(s["vc"].data_ptr()) for s in sets]
    hidden_rows = None
    if heads is not None and fused:
        # the tree rows' hidden states: the frontier carry feeds the next head step from them
        hidden_rows = torch.randn((w.B, N, hidden), device="cuda").to(torch.bfloat16)

    def build_calls(sptr, ctl, n):
        calls = []
        for i in range(n):
            s, kc_arr, vc_arr = sets[i % n_sets], kc_arrs[i % n_sets], vc_arrs[i % n_sets]
            prefix, status = p(ctl[i]), p(ctl[i, w.B:])
            attn = (sptr, dcode, w.B, w.Hq, w.Hkv, w.d, N, p(shared["depth"]), p(shared["mask"]),
                    tree["mask_words"], prefix, p(s["q"]), p(s["kn"]), p(s["vn"]), p(s["kc"]),
                    p(s["vc"]), x["S_max"], float(w.rope_base), p(s["out"]), p(s["attn_ws"]),
                    s["attn_ws"].numel(), status)
            V = w.vocab if x["logits"] is not None else 0
            n_slots = x["candidates"].shape[1]
            cmp_ = None
            if args.accept == "typical":
                acc = (sptr, w.B, N, w.vocab, p(s["logits"]), 1.0, 0.3, 0.09, p(s["cand"]), n_slots,
                       p(shared["tidx"]), p(shared["retrieve"]), nn, width, p(s["best"]), p(s["alen"]),
                       p(s["tokens"]), p(s["frontier"]), p(s["acc_ws"]), s["acc_ws"].numel(), status)
                # typical rounds commit with the separate compaction call
                cmp_ = (sptr, dcode, 1, w.B, w.Hkv, w.d, x["S_max"], N, ctypes.cast(kc_arr, ctypes.c_void_p),
                        ctypes.cast(vc_arr, ctypes.c_void_p), p(shared["retrieve"]), nn, width, p(s["best"]),
                        p(s["alen"]), prefix, status)
            elif fused:
                carry = ((hidden, p(hidden_rows), p(heads["h"]), p(heads["root"])) if hidden_rows is not None
                         else (0, None, None, None))
                acc = (sptr, w.B, N, V, p(s["logits"]), p(s["tids"]), p(s["cand"]), n_slots, p(shared["tidx"]),
                       p(shared["retrieve"]), nn, width, p(s["best"]), p(s["alen"]), p(s["tokens"]),
                       p(s["frontier"]), dcode, 1, w.Hkv, w.d, x["S_max"], ctypes.cast(kc_arr, ctypes.c_void_p),
                       ctypes.cast(vc_arr, ctypes.c_void_p), prefix) + carry + (
                           p(s["acc_ws"]), s["acc_ws"].numel(), status)
            else:
                acc = (sptr, w.B, N, V, p(s["logits"]), p(s["tids"]), p(s["cand"]), n_slots, p(shared["tidx"]),
                       p(shared["retrieve"]), nn, width, p(s["best"]), p(s["alen"]), p(s["tokens"]),
                       p(s["frontier"]), p(s["acc_ws"]), s["acc_ws"].numel(), status)
                cmp_ = (sptr, dcode, 1, w.B, w.Hkv, w.d, x["S_max"], N, ctypes.cast(kc_arr, ctypes.c_void_p),
                        ctypes.cast(vc_arr, ctypes.c_void_p), p(shared["retrieve"]), nn, width, p(s["best"]),
                        p(s["alen"]), prefix, status)
            head = None
            if heads is not None:
                head = (sptr, w.B, w.num_heads, hidden, w.vocab, w.topk, p(heads["h"]), p(heads["W1"]),
                        p(heads["W2"]), p(heads["root"]), p(s["cand"]), None, p(heads["ws"]),
                        heads["ws"].numel(), status)
            calls.append((attn, acc, cmp_, head))
        return calls

    accept_fn = (lib.medusa_accept_typical if args.accept == "typical"
                 else lib.medusa_accept_commit if fused else lib.medusa_accept)
    ev = HipEvents()
    events = [(ev.create(), ev.create()) for _ in range(total)]
    head_events = [(ev.create(), ev.create()) for _ in range(total)] if heads is not None else []
    acc_events = [(ev.create(), ev.create()) for _ in range(total)]
    no_events = (None, None)

    def step(call, evs, hevs, aevs=no_events):
        attn, acc, cmp_, head = call
        rc = 0
        if head is not None:
            rc |= lib.medusa_head_candidates(*head, *hevs)
        rc |= lib.medusa_tree_attn(*attn, *evs)
        rc |= accept_fn(*acc, *aevs)
        if cmp_ is not None:
            rc |= lib.medusa_kv_compact(*cmp_, None, None)
        if rc:
            raise RuntimeError("library call failed")

    ctl = pristine.repeat(total, 1).contiguous()   # [steps][B + 1]
    calls = build_calls(sptr, ctl, total)
    hev = lambda i: head_events[i] if head_events else no_events
    for i in range(args.warmup):
        step(calls[i], events[i], hev(i), acc_events[i])
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    # Timing events cost host launch time (the extended launch that records them): around every
    # call they stretched the eager step by about 4 us, beyond what the GPU spends.  The
    # attention and head calls are therefore timed on every EVENT_EVERY-th timed step, the
    # acceptance call in the warm-up steps only.
    timed = lambda i: (i - args.warmup) % EVENT_EVERY == 0
    for i in range(args.warmup, total):
        step(calls[i], events[i] if timed(i) else no_events, hev(i) if timed(i) else no_events)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start

    graph_info = None
    if args.graph:
        # the same number of steps, captured once on a stream of their own (no timing
        # events) and replayed as one graph, with fresh control blocks
        ctl_g = pristine.repeat(args.steps, 1).contiguous()
        cap = torch.cuda.Stream()
        gcalls = build_calls(cap.cuda_stream, ctl_g, args.steps)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap):
            for c in gcalls:
                step(c, no_events, no_events)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        g_el = time.perf_counter() - t0
        g_status = ctl_g[:, w.B].cpu().numpy()
        if g_status.any():
            raise RuntimeError(f"graph replay status words {sorted(set(g_status.tolist()))}")
        graph_info = {"ms_per_step": g_el / args.steps * 1e3, "value": w.B * N * args.steps / g_el,
                      "library_calls_per_step": (3 if heads is not None else 2) + (0 if fused else 1)}
        log(f"[bench] graph replay: {g_el / args.steps * 1e6:.1f} us per step")

    statuses = ctl[:, w.B].cpu().numpy()
    if statuses.any():
        raise RuntimeError(f"device status words {sorted(set(statuses.tolist()))}: the round failed")
    attn_ms = np.array([ev.elapsed_ms(*events[i]) for i in range(args.warmup, total) if timed(i)])
    head_ms = np.array([ev.elapsed_ms(*head_events[i]) for i in range(args.warmup, total) if timed(i)]
                       if head_events else [])
    # the acceptance call's events add host launch cost, so they are recorded in the untimed
    # warm-up steps only
    acc_ms = np.array([ev.elapsed_ms(a, b) for a, b in acc_events[:args.warmup]] or [float("nan")])
    # tokens each timed step committed per sequence: the compaction advanced P_b by G_b
    committed = ctl[args.warmup:, :w.B].cpu().numpy().astype(np.int64) - x["prefix_len"][None, :].astype(np.int64)
    for a, b in events + head_events + acc_events:
        ev.destroy(a)
        ev.destroy(b)

    copy_info = None
    if args.copy_calibration:
        src = torch.randn(2 ** 26, device="cuda")      # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        copy_info = "torch.neg over 2^26 fp32 (256 MiB read + 256 MiB written) x5"

    ceiling_gbs = read_ceiling_gbs(torch, M)
    esize = 2 if w.dtype == "bf16" else 4
    alg = algorithmic_bytes(w, N, esize)
    mean_s = float(attn_ms.mean()) * 1e-3
    achieved = alg / mean_s / 1e9
    src_hash = attn_source_hash()
    result = {
        "metric": "tree-verify attention nodes/s and % HBM peak, 64-node tree @ ctx 4096",
        "value": w.B * N * args.steps / elapsed,
        "unit": "nodes/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": (f"{w.name}: B={w.B}, Hq={w.Hq}, Hkv={w.Hkv}, d_h={w.d}, P={w.P}, "
                                f"N={N} ({w.tree} tree), V={w.vocab}"),
                   "global_batch": w.B, "seq_len": w.P, "tree_nodes": N, "buffer_sets": n_sets,
                   "accept": args.accept, "round": args.round,
                   "commit": "fused" if fused else "separate"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(src_hash),
                     "kernel": "medusa_tree_attn", "algorithmic_bytes": alg,
                     "mean_us": mean_s * 1e6, "median_us": float(np.median(attn_ms)) * 1e3,
                     "p10_us": float(np.percentile(attn_ms, 10)) * 1e3,
                     "p90_us": float(np.percentile(attn_ms, 90)) * 1e3,
                     "timed_calls": int(attn_ms.size), "event_every": EVENT_EVERY,
                     "source_hash": src_hash,
                     "read_ceiling_gbs": ceiling_gbs, "frac_of_read_ceiling": achieved / ceiling_gbs},
        "attention_nodes_per_s": w.B * N / mean_s,
        "tree_compile_us": compile_us,
        # what [Chai]'s engineering notes ask a round to record: the tree's shape, the
        # committed-token distribution G, and per-stage latency
        "round_metrics": {
            "nodes": N, "nodes_per_depth": np.bincount(tree["depth"]).tolist(),
            "n_paths": tree["n_paths"], "path_width": tree["path_width"],
            "committed_tokens_G": {
                "mean": float(committed.mean()),
                "per_sequence_mean": committed.mean(axis=0).tolist(),
                "histogram": {str(int(g)): int(c) for g, c in zip(*np.unique(committed, return_counts=True))}},
            "stage_us": {"attention": float(attn_ms.mean()) * 1e3,
                         "accept" + ("_commit" if fused else ""): float(acc_ms.mean()) * 1e3,
                         **({"head": float(head_ms.mean()) * 1e3} if heads is not None else {}),
                         "round_step": elapsed / args.steps * 1e6},
        },
    }
    if w.dtype == "bf16":  # the matrix-core path; its peak is the dense bf16 MFMA rate
        flops = algorithmic_flops(w, N)
        result["mfma"] = {"achieved": flops / mean_s / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
                          "unit": "TFLOP/s", "frac": flops / mean_s / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                          "flops": flops, "kernel": "medusa_tree_attn"}
    if heads is not None:
        h_alg = head_algorithmic_bytes(w.B, w.num_heads, hidden, w.vocab, w.topk)
        h_mean = float(head_ms.mean()) * 1e-3
        h_ach = h_alg / h_mean / 1e9
        h_hash = head_source_hash()
        result["attention_roofline"] = result.pop("roofline")
        result["roofline"] = {
            "bound": "hbm", "achieved": h_ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": h_ach / HBM_PEAK_GBS, "traffic": measured_traffic(h_hash, HEAD_TRAFFIC_FILE),
            "kernel": "medusa_head_candidates", "algorithmic_bytes": h_alg,
            "mean_us": h_mean * 1e6, "median_us": float(np.median(head_ms)) * 1e3,
            "p10_us": float(np.percentile(head_ms, 10)) * 1e3,
            "p90_us": float(np.percentile(head_ms, 90)) * 1e3,
            "source_hash": h_hash, "read_ceiling_gbs": ceiling_gbs,
            "frac_of_read_ceiling": h_ach / ceiling_gbs}
        result["config"]["workload"] += f"; head step K={w.num_heads}, hidden={hidden}, topk={w.topk}"
        log(f"[bench] head step mean {h_mean * 1e6:.2f} us -> {h_ach:.0f} GB/s "
            f"({h_ach / HBM_PEAK_GBS:.1%} of HBM peak, {h_ach / ceiling_gbs:.1%} of the read ceiling)")
    if graph_info:
        result["graph"] = graph_info
    if copy_info:
        result["copy_calibration"] = copy_info
    log(f"[bench] attention mean {mean_s * 1e6:.2f} us -> {achieved:.0f} GB/s "
        f"({achieved / HBM_PEAK_GBS:.1%} of HBM peak, {achieved / ceiling_gbs:.1%} of the "
        f"{ceiling_gbs:.0f} GB/s read ceiling); step {elapsed / args.steps * 1e6:.1f} us")
    if cpu_record is not None:
        result["cpu_baseline"] = cpu_record
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
