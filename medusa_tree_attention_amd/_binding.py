"""ctypes binding of libmedusa.so: argument marshalling only.

Each function has the name of the C entry point it calls (include/medusa.h),
converts torch tensors / numpy arrays to pointers and sizes, and raises
``MedusaError`` on a negative status.  Every step of the round runs in the
library; nothing here computes any part of it.  The library must be built
(``__graft_entry__.build()``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_PKG, "libmedusa.so")

STATUS = {0: "MEDUSA_OK", -1: "MEDUSA_EINVAL", -2: "MEDUSA_ENOT_PREFIX_CLOSED",
          -3: "MEDUSA_ECAPACITY", -4: "MEDUSA_EUNSUPPORTED", -5: "MEDUSA_EBUFSIZE",
          -6: "MEDUSA_EHIP"}
F32, BF16 = 0, 1


class MedusaError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)}")
        self.code = code
        self.name = STATUS.get(code, str(code))


class TreeSpec(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("n_paths", ctypes.c_int32), ("path_len", ctypes.POINTER(ctypes.c_int32)),
                ("path_ranks", ctypes.POINTER(ctypes.c_int32)),
                ("rank_hit", ctypes.POINTER(ctypes.c_double)), ("n_nodes", ctypes.c_int32)]


class Tree(ctypes.Structure):
    _fields_ = [("n_nodes", ctypes.c_int32), ("n_paths", ctypes.c_int32),
                ("path_width", ctypes.c_int32), ("mask_words", ctypes.c_int32),
                ("tree_indices", ctypes.POINTER(ctypes.c_int32)),
                ("depth", ctypes.POINTER(ctypes.c_int32)),
                ("parent", ctypes.POINTER(ctypes.c_int32)),
                ("tree_mask", ctypes.POINTER(ctypes.c_uint64)),
                ("retrieve_indices", ctypes.POINTER(ctypes.c_int32)),
                ("node_weight", ctypes.POINTER(ctypes.c_double))]


_lib = None
_P, _I32, _SZ, _D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_double
_SIGNATURES = {
    "medusa_tree_compile": (_I32, [ctypes.POINTER(TreeSpec), ctypes.POINTER(Tree)]),
    "medusa_tree_attn_workspace_size": (_SZ, [_I32] * 7),
    "medusa_tree_attn": (_I32, [_P, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _I32, _P, _P, _P,
                                _P, _P, _P, _I32, _D, _P, _P, _SZ, _P, _P, _P]),
    "medusa_tree_attn_noalloc": (_I32, [_P, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _I32, _P, _P, _P,
                                        _P, _P, _P, _I32, _D, _P, _P, _P, _P]),
    "medusa_accept_workspace_size": (_SZ, [_I32, _I32]),
    "medusa_accept": (_I32, [_P, _I32, _I32, _I32, _P, _P, _P, _I32, _P, _P, _I32, _I32, _P, _P,
                             _P, _P, _P, _SZ, _P, _P, _P]),
    "medusa_accept_typical": (_I32, [_P, _I32, _I32, _I32, _P, _D, _D, _D, _P, _I32, _P, _P, _I32,
                                     _I32, _P, _P, _P, _P, _P, _SZ, _P, _P, _P]),
    "medusa_head_workspace_size": (_SZ, [_I32] * 4),
    "medusa_head_candidates": (_I32, [_P, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P,
                                      _SZ, _P, _P, _P]),
    "medusa_kv_compact": (_I32, [_P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _I32,
                                 _I32, _P, _P, _P, _P, _P, _P]),
    "medusa_tree_budget": (_I32, [_P, _I32, _I32, _I32, _P, _P, _D, _I32, _P, _P, _P]),
    "medusa_read_probe_sink_size": (_SZ, []),
    "medusa_read_probe": (_I32, [_P, _P, _SZ, _P, _P, _P]),
    "medusa_accept_commit": (_I32, [_P, _I32, _I32, _I32, _P, _P, _P, _I32, _P, _P, _I32, _I32, _P,
                                    _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _I32, _P,
                                    _P, _P, _P, _SZ, _P, _P, _P]),
}


def load():
    """Load libmedusa.so (built in-tree); raises if it is missing.

    torch is imported first: its wheel carries its own HIP runtime with the
    same soname, and loading it before libmedusa makes both share that one
    runtime (device pointers and streams are runtime objects).
    """
    global _lib
    if _lib is None:
        import torch  # noqa: F401
        if not os.path.exists(LIBRARY):
            raise ImportError(f"{LIBRARY} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(LIBRARY)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


def _check(fn, code):
    if code != 0:
        raise MedusaError(fn, code)


VALIDATE_ENV = "MEDUSA_VALIDATE"


def validating():
    """True when MEDUSA_VALIDATE is set to a non-empty value other than 0: every device entry
    point then waits for its work and checks the round's status word (a debugging mode; the
    library itself never synchronises)."""
    return os.environ.get(VALIDATE_ENV, "0") not in ("", "0")


def _validate(fn, status):
    """In validation mode: synchronise the status word's device and raise MedusaError if
    the word holds an error code."""
    if not validating():
        return
    if getattr(status, "is_cuda", False):
        import torch
        torch.cuda.synchronize(status.device)
    code = int(status.reshape(-1)[0].item())
    if code != 0:
        raise MedusaError(fn + " (device status word)", code)


def _ptr(t):
    """Device pointer of a torch tensor (or None)."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmedusa must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def _arr(a, dtype, ctype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.POINTER(ctype))


# ------------------------------------------------------------------ tree compile

def medusa_tree_compile(num_heads, topk, paths=None, rank_hit=None, n_nodes=0):
    """Compile a tree (explicit ``paths`` or greedy growth from ``rank_hit``) into host arrays."""
    lib = load()
    spec = TreeSpec(num_heads=num_heads, topk=topk, n_paths=0, n_nodes=int(n_nodes or 0))
    keep = []
    if paths is not None:
        lens, plen = _arr([len(p) for p in paths] or [0], np.int32, ctypes.c_int32)
        flat, pranks = _arr([r for p in paths for r in p] or [0], np.int32, ctypes.c_int32)
        spec.n_paths, spec.path_len, spec.path_ranks = len(paths), plen, pranks
        keep += [lens, flat]
    if rank_hit is not None:
        rh, prh = _arr(np.asarray(rank_hit, np.float64).reshape(-1), np.float64, ctypes.c_double)
        spec.rank_hit = prh
        keep.append(rh)
    sizes = Tree()
    _check("medusa_tree_compile", lib.medusa_tree_compile(ctypes.byref(spec), ctypes.byref(sizes)))
    n, npaths, w, words = sizes.n_nodes, sizes.n_paths, sizes.path_width, sizes.mask_words
    out = {"tree_indices": np.zeros(n, np.int32), "depth": np.zeros(n, np.int32),
           "parent": np.zeros(n, np.int32), "tree_mask": np.zeros((n, words), np.uint64),
           "retrieve": np.zeros((npaths, w), np.int32)}
    tree = Tree(n_nodes=n, n_paths=npaths, path_width=w, mask_words=words)
    tree.tree_indices = out["tree_indices"].ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    tree.depth = out["depth"].ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    tree.parent = out["parent"].ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    tree.tree_mask = out["tree_mask"].ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))
    tree.retrieve_indices = out["retrieve"].ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    if rank_hit is not None:
        out["node_weight"] = np.zeros(n, np.float64)
        tree.node_weight = out["node_weight"].ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    _check("medusa_tree_compile", lib.medusa_tree_compile(ctypes.byref(spec), ctypes.byref(tree)))
    out.update(n_nodes=n, n_paths=npaths, path_width=w, mask_words=words)
    return out


def medusa_tree_budget(rank_hit, cost_nodes, cost_us, fixed_us, n_layers):
    """Best node count for measured per-layer costs; returns (best_n, expected_tokens, rate),
    the arrays indexed by the node count."""
    lib = load()
    a, pa = _arr(np.asarray(rank_hit, np.float64).reshape(-1), np.float64, ctypes.c_double)
    K, TOPK = np.asarray(rank_hit).shape
    nodes, pn = _arr(cost_nodes, np.int32, ctypes.c_int32)
    us, pu = _arr(cost_us, np.float64, ctypes.c_double)
    hi = int(nodes[-1])
    et = np.zeros(hi + 1, np.float64)
    rt = np.zeros(hi + 1, np.float64)
    best = ctypes.c_int32(0)
    code = lib.medusa_tree_budget(pa, K, TOPK, len(nodes), pn, pu, float(fixed_us), int(n_layers),
                                  ctypes.byref(best), et.ctypes.data_as(ctypes.c_void_p),
                                  rt.ctypes.data_as(ctypes.c_void_p))
    _check("medusa_tree_budget", code)
    return int(best.value), et, rt


# ------------------------------------------------------------------ tree attention

def medusa_tree_attn_workspace_size(dt, B, Hq, Hkv, d_h, N, S_max):
    return int(load().medusa_tree_attn_workspace_size(dt, B, Hq, Hkv, d_h, N, S_max))


def medusa_tree_attn(q, k_new, v_new, k_cache, v_cache, depth, tree_mask, prefix_len, rope_base,
                     out, workspace, status, stream=None, ev_start=None, ev_stop=None):
    """One tree-attention layer; shapes are read from the tensors (see include/medusa.h)."""
    B, N, Hq, d = q.shape
    Hkv, S_max = k_new.shape[2], k_cache.shape[2]
    code = load().medusa_tree_attn(
        _stream(stream), _dtype_code(q), B, Hq, Hkv, d, N, _ptr(depth), _ptr(tree_mask),
        tree_mask.shape[1], _ptr(prefix_len), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
        _ptr(v_cache), S_max, float(rope_base), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _ptr(status), ev_start, ev_stop)
    _check("medusa_tree_attn", code)
    _validate("medusa_tree_attn", status)


def medusa_tree_attn_noalloc(q, k_new, v_new, k_cache, v_cache, depth, tree_mask, prefix_len, rope_base,
                             out, status, stream=None, ev_start=None, ev_stop=None):
    """medusa_tree_attn with the split partials in the library's own device array."""
    B, N, Hq, d = q.shape
    Hkv, S_max = k_new.shape[2], k_cache.shape[2]
    code = load().medusa_tree_attn_noalloc(
        _stream(stream), _dtype_code(q), B, Hq, Hkv, d, N, _ptr(depth), _ptr(tree_mask),
        tree_mask.shape[1], _ptr(prefix_len), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
        _ptr(v_cache), S_max, float(rope_base), _ptr(out), _ptr(status), ev_start, ev_stop)
    _check("medusa_tree_attn_noalloc", code)
    _validate("medusa_tree_attn_noalloc", status)


# ------------------------------------------------------------------ acceptance

def medusa_accept_workspace_size(B, N):
    return int(load().medusa_accept_workspace_size(B, N))


def medusa_accept(candidates, tree_indices, retrieve, best_path, accept_len, accepted_tokens,
                  frontier_row, status, logits=None, target_ids=None, workspace=None,
                  stream=None, ev_start=None, ev_stop=None):
    B, n_slots = candidates.shape
    N = tree_indices.shape[0]
    V = logits.shape[2] if logits is not None else 0
    n_paths, width = retrieve.shape
    code = load().medusa_accept(
        _stream(stream), B, N, V, _ptr(logits), _ptr(target_ids), _ptr(candidates), n_slots,
        _ptr(tree_indices), _ptr(retrieve), n_paths, width, _ptr(best_path), _ptr(accept_len),
        _ptr(accepted_tokens), _ptr(frontier_row), _ptr(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _ptr(status), ev_start, ev_stop)
    _check("medusa_accept", code)
    _validate("medusa_accept", status)


def medusa_accept_typical(candidates, tree_indices, retrieve, best_path, accept_len, accepted_tokens,
                          frontier_row, status, logits, workspace, temperature=1.0, epsilon=0.3,
                          alpha=0.09, stream=None, ev_start=None, ev_stop=None):
    B, n_slots = candidates.shape
    N = tree_indices.shape[0]
    V = logits.shape[2]
    n_paths, width = retrieve.shape
    code = load().medusa_accept_typical(
        _stream(stream), B, N, V, _ptr(logits), float(temperature), float(epsilon), float(alpha),
        _ptr(candidates), n_slots, _ptr(tree_indices), _ptr(retrieve), n_paths, width,
        _ptr(best_path), _ptr(accept_len), _ptr(accepted_tokens), _ptr(frontier_row),
        _ptr(workspace), workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _ptr(status), ev_start, ev_stop)
    _check("medusa_accept_typical", code)
    _validate("medusa_accept_typical", status)


def medusa_accept_commit(candidates, tree_indices, retrieve, best_path, accept_len, accepted_tokens,
                         frontier_row, k_caches, v_caches, prefix_len, status, logits=None,
                         target_ids=None, workspace=None, hidden=None, h_next=None, next_root=None,
                         stream=None, ev_start=None, ev_stop=None):
    """Greedy acceptance, compaction of every layer in ``k_caches``/``v_caches`` (lists of
    [B,Hkv,S_max,d] tensors) and the frontier carry (``hidden`` [B,N,H] -> ``h_next`` [B,H],
    ``next_root`` [B]) in one call."""
    B, n_slots = candidates.shape
    N = tree_indices.shape[0]
    V = logits.shape[2] if logits is not None else 0
    n_paths, width = retrieve.shape
    n_layers = len(k_caches)
    _, Hkv, S_max, d = k_caches[0].shape
    karr = (ctypes.c_void_p * max(n_layers, 1))(*[_ptr(t) for t in k_caches])
    varr = (ctypes.c_void_p * max(n_layers, 1))(*[_ptr(t) for t in v_caches])
    hidden_dim = hidden.shape[-1] if hidden is not None else 0
    code = load().medusa_accept_commit(
        _stream(stream), B, N, V, _ptr(logits), _ptr(target_ids), _ptr(candidates), n_slots,
        _ptr(tree_indices), _ptr(retrieve), n_paths, width, _ptr(best_path), _ptr(accept_len),
        _ptr(accepted_tokens), _ptr(frontier_row), _dtype_code(k_caches[0]), n_layers, Hkv, d, S_max,
        ctypes.cast(karr, ctypes.c_void_p), ctypes.cast(varr, ctypes.c_void_p), _ptr(prefix_len),
        hidden_dim, _ptr(hidden), _ptr(h_next), _ptr(next_root), _ptr(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _ptr(status), ev_start, ev_stop)
    _check("medusa_accept_commit", code)
    _validate("medusa_accept_commit", status)


# ------------------------------------------------------------------ head step

def medusa_head_workspace_size(B, K, d, V):
    return int(load().medusa_head_workspace_size(B, K, d, V))


def medusa_head_candidates(h, W1, W2, root_tokens, candidates, status, workspace, topk,
                           head_logits=None, stream=None, ev_start=None, ev_stop=None):
    B, d = h.shape
    K, V = W2.shape[0], W2.shape[1]
    code = load().medusa_head_candidates(
        _stream(stream), B, K, d, V, topk, _ptr(h), _ptr(W1), _ptr(W2), _ptr(root_tokens),
        _ptr(candidates), _ptr(head_logits), _ptr(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _ptr(status), ev_start, ev_stop)
    _check("medusa_head_candidates", code)
    _validate("medusa_head_candidates", status)


# ------------------------------------------------------------------ compaction

def medusa_kv_compact(k_caches, v_caches, retrieve, best_path, accept_len, prefix_len, n_nodes,
                      status, stream=None, ev_start=None, ev_stop=None):
    """Compact every layer's cache; ``k_caches``/``v_caches`` are lists of [B,Hkv,S_max,d] tensors."""
    n_layers = len(k_caches)
    B, Hkv, S_max, d = k_caches[0].shape
    karr = (ctypes.c_void_p * max(n_layers, 1))(*[_ptr(t) for t in k_caches])
    varr = (ctypes.c_void_p * max(n_layers, 1))(*[_ptr(t) for t in v_caches])
    n_paths, width = retrieve.shape
    code = load().medusa_kv_compact(
        _stream(stream), _dtype_code(k_caches[0]), n_layers, B, Hkv, d, S_max, n_nodes,
        ctypes.cast(karr, ctypes.c_void_p), ctypes.cast(varr, ctypes.c_void_p), _ptr(retrieve),
        n_paths, width, _ptr(best_path), _ptr(accept_len), _ptr(prefix_len), _ptr(status),
        ev_start, ev_stop)
    _check("medusa_kv_compact", code)
    _validate("medusa_kv_compact", status)


# ------------------------------------------------------------------ measurement utility

def medusa_read_probe_sink_size():
    return int(load().medusa_read_probe_sink_size())


def medusa_read_probe(src, sink, stream=None, ev_start=None, ev_stop=None):
    """Stream ``src`` (a contiguous device tensor) once; ``sink`` receives one word per workgroup."""
    code = load().medusa_read_probe(_stream(stream), _ptr(src), src.numel() * src.element_size(),
                                    _ptr(sink), ev_start, ev_stop)
    _check("medusa_read_probe", code)
