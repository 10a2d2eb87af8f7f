"""UNO decode-cycle sampling on MI355X (gfx950).

Thin ctypes binding of ``libuno.so`` (C ABI in ``include/uno.h``).  Every step
of the sampling path runs in the library's HIP kernels; this module only
allocates output tensors and the workspace with PyTorch and passes device
pointers and the current HIP stream.  If the library is missing, every call
raises -- there is no fallback.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading

import numpy as np
import torch

__all__ = [
    "UnoError", "Sampling", "library_path", "load_library", "workspace_bytes", "filter_rows",
    "sample_linear", "build_tree", "verify_tree", "tree_attention", "OP_FILTER", "OP_SAMPLE_LINEAR",
    "OP_BUILD_TREE", "OP_VERIFY_TREE", "MAX_TOP_K", "ORDER_TOPK_FIRST", "ORDER_JOINT",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# UNO_LIBRARY names another build of the library (for instance the
# sanitizer build of the host code); by default the in-tree libuno.so.
_LIB_PATH = os.environ.get("UNO_LIBRARY") or os.path.join(_HERE, "libuno.so")
_lock = threading.Lock()
_lib = None

OP_FILTER, OP_SAMPLE_LINEAR, OP_BUILD_TREE, OP_VERIFY_TREE = 0, 1, 2, 3
MAX_TOP_K = 256
ORDER_TOPK_FIRST, ORDER_JOINT = 0, 1     # uno_order_t
_STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported configuration",
           -3: "workspace missing, too small or misaligned", -4: "HIP launch failure",
           -5: "workspace exceeds the allocation-free entry point's fixed scratch"}
NOALLOC_SCRATCH_BYTES = 32 << 20       # UNO_NOALLOC_SCRATCH_BYTES


class UnoError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_STATUS.get(status, 'unknown status')} (status {status})")


class Sampling(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("top_k", ctypes.c_int32),
                ("top_p", ctypes.c_float), ("order", ctypes.c_int32)]


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libuno.so; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() first")
        lib = ctypes.CDLL(_LIB_PATH)
        P, i32, i64, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
        SP = ctypes.POINTER(Sampling)
        sz = ctypes.POINTER(ctypes.c_size_t)
        lib.uno_workspace_bytes.argtypes = [i32, i64, i32, i32, i32, i64, i32, SP, sz]
        lib.uno_filter.argtypes = [P, i32, i64, i64, SP, i32, P, P, P, P, P, ctypes.c_size_t, P]
        lib.uno_sample_linear.argtypes = [P, P, i32, i32, i32, i64, SP, u64, u64, P, P, P, P, P, P,
                                          ctypes.c_size_t, P]
        lib.uno_build_tree.argtypes = [P, i32, i32, i32, i32, i32, i64, SP, P, P, P, P, P, P,
                                       ctypes.c_size_t, P]
        lib.uno_verify_tree.argtypes = [P, i32, i32, i32, i32, i64, SP, u64, u64, P, P, P, P, P, P,
                                        P, P, P, ctypes.c_size_t, P]
        lib.uno_workspace_bytes_ex.argtypes = [i32, i64, i32, i32, i32, i64, i32, SP, i32, sz]
        lib.uno_filter_ex.argtypes = [P, i32, i64, i64, SP, i32, i32, P, P, P, P, P, ctypes.c_size_t, P]
        lib.uno_sample_linear_ex.argtypes = [P, P, i32, i32, i32, i64, SP, i32, u64, u64, P, P, P, P, P, P,
                                             ctypes.c_size_t, P]
        lib.uno_build_tree_ex.argtypes = [P, i32, i32, i32, i32, i32, i64, SP, i32, P, P, P, P, P, P,
                                          ctypes.c_size_t, P]
        lib.uno_verify_tree_ex.argtypes = [P, i32, i32, i32, i32, i64, SP, i32, u64, u64, P, P, P, P, P, P,
                                           P, P, P, ctypes.c_size_t, P]
        lib.uno_tree_attention.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, ctypes.c_float,
                                           P, P, P]
        lib.uno_sample_linear_noalloc.argtypes = [P, P, i32, i32, i32, i64, SP, u64, u64, P, P, P, P, P, P]
        lib.uno_stream_read.argtypes = [P, i64, i64, P, P]
        for f in ("uno_workspace_bytes", "uno_filter", "uno_sample_linear", "uno_build_tree",
                  "uno_verify_tree", "uno_tree_attention", "uno_last_hip_error", "uno_workspace_bytes_ex",
                  "uno_filter_ex", "uno_sample_linear_ex", "uno_build_tree_ex", "uno_verify_tree_ex",
                  "uno_sample_linear_noalloc", "uno_stream_read"):
            getattr(lib, f).restype = ctypes.c_int
        lib.uno_status_string.argtypes = [ctypes.c_int]
        lib.uno_status_string.restype = ctypes.c_char_p
        lib.uno_version.restype = ctypes.c_char_p
        _lib = lib
        return lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return 0
    if t.dtype == torch.bfloat16:
        return 1
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Context in which a call allocates its outputs, workspace and temporaries
    and converts its arguments: the call's own stream, so the caching allocator
    orders their reuse after the kernels that read them.  The caller orders the
    inputs it passes against that stream."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _check(status: int, where: str):
    if status != 0:
        raise UnoError(status, where)


def _sp(temperature, top_k, top_p, order=ORDER_TOPK_FIRST) -> Sampling:
    return Sampling(float(temperature), int(top_k), float(top_p), int(order))


def _sp_set(n, temperature, top_k, top_p, order):
    """(array of Sampling, count): one set when every parameter is a scalar,
    else one per request (or row), each parameter broadcast to n."""
    vals = [np.asarray(x.cpu() if isinstance(x, torch.Tensor) else x) for x in (temperature, top_k, top_p, order)]
    if all(v.ndim == 0 for v in vals):
        return (Sampling * 1)(_sp(*[v.item() for v in vals])), 1
    T, K, P, O = (np.broadcast_to(v, (n,)) for v in vals)
    return (Sampling * n)(*[Sampling(float(T[i]), int(K[i]), float(P[i]), int(O[i])) for i in range(n)]), n


def workspace_bytes(op, batch_or_rows, B, K, V, vocab, dtype_code, temperature, top_k, top_p,
                    order=ORDER_TOPK_FIRST) -> int:
    lib = load_library()
    out = ctypes.c_size_t(0)
    sps, n = _sp_set(batch_or_rows, temperature, top_k, top_p, order)
    _check(lib.uno_workspace_bytes_ex(op, batch_or_rows, B, K, V, vocab, dtype_code, sps, n, ctypes.byref(out)),
           "uno_workspace_bytes_ex")
    return int(out.value)


def _workspace(nbytes, device, ws):
    if nbytes == 0:
        return None
    if ws is not None and ws.numel() >= nbytes:
        return ws
    return torch.empty(nbytes + 256, dtype=torch.uint8, device=device)


def _aligned_ptr(ws):
    if ws is None:
        return None, 0
    p = ws.data_ptr()
    a = (p + 255) // 256 * 256
    return ctypes.c_void_p(a), ws.numel() - (a - p)


def _as_u32_ids(request_ids, batch, device):
    if request_ids is None:
        return None
    r = torch.as_tensor(request_ids, device=device)
    if r.dtype != torch.int32:
        r = r.to(torch.int64).to(torch.int32)   # uint32 ids carried in int32 storage
    assert r.shape == (batch,)
    return r.contiguous()


def _filter_rows_impl(logits, temperature, top_k, top_p, cap=None, workspace=None, stream=None,
                order=ORDER_TOPK_FIRST):
    """uno_filter over logits [rows, vocab].  Returns dict of device tensors:
    ids/probs [rows, cap] (sparse modes), count [rows], stats [rows, 2]."""
    lib = load_library()
    assert logits.is_cuda and logits.dim() == 2 and logits.is_contiguous()
    rows, vocab = logits.shape
    dt = _dtype_code(logits)
    dev = logits.device
    sps, nsp = _sp_set(rows, temperature, top_k, top_p, order)
    # rows on the top-k path get supports of the largest k among them; rows
    # over the full vocabulary report only their count and statistics
    sparse, k_eff = False, 1
    for i in range(nsp):
        greedy = sps[i].temperature == 0.0
        topk_on = 0 < sps[i].top_k < vocab
        if greedy or topk_on or vocab <= MAX_TOP_K:
            sparse = True
            k_eff = max(k_eff, 1 if greedy else (sps[i].top_k if topk_on else vocab))
    cap = (k_eff if sparse else 0) if cap is None else int(cap)
    nb = workspace_bytes(OP_FILTER, rows, 0, 0, 0, vocab, dt, temperature, top_k, top_p, order)
    ws = _workspace(nb, dev, workspace)
    wsp, wsn = _aligned_ptr(ws)
    ids = torch.empty((rows, max(cap, 1)), dtype=torch.int32, device=dev) if sparse else None
    probs = torch.empty((rows, max(cap, 1)), dtype=torch.float64, device=dev) if sparse else None
    count = torch.empty(rows, dtype=torch.int32, device=dev)
    stats = torch.empty((rows, 2), dtype=torch.float64, device=dev)
    _check(lib.uno_filter_ex(_ptr(logits), dt, rows, vocab, sps, nsp, cap, _ptr(ids),
                             _ptr(probs), _ptr(count), _ptr(stats), wsp, wsn, _stream(stream)),
           "uno_filter_ex")
    return dict(ids=ids, probs=probs, count=count, stats=stats, workspace=ws)


def _sample_linear_impl(draft, target, temperature, top_k, top_p, seed, offset, request_ids=None,
                  out=None, workspace=None, stream=None, order=ORDER_TOPK_FIRST):
    """uno_sample_linear: draft [batch, B, vocab], target [batch, B+1, vocab]."""
    lib = load_library()
    assert draft.is_cuda and target.is_cuda and draft.dtype == target.dtype
    assert draft.is_contiguous() and target.is_contiguous()
    batch, B, vocab = draft.shape
    assert target.shape == (batch, B + 1, vocab)
    dt = _dtype_code(draft)
    dev = draft.device
    if out is None:
        out = dict(tokens=torch.empty((batch, B + 1), dtype=torch.int32, device=dev),
                   accept_len=torch.empty(batch, dtype=torch.int32, device=dev),
                   proposals=torch.empty((batch, B), dtype=torch.int32, device=dev),
                   flags=torch.empty(batch, dtype=torch.int32, device=dev))
    if workspace is None:
        nb = workspace_bytes(OP_SAMPLE_LINEAR, batch, B, 1, B, vocab, dt, temperature, top_k, top_p, order)
        workspace = _workspace(nb, dev, None)
    wsp, wsn = _aligned_ptr(workspace)
    rid = _as_u32_ids(request_ids, batch, dev)
    sps, nsp = _sp_set(batch, temperature, top_k, top_p, order)
    _check(lib.uno_sample_linear_ex(_ptr(draft), _ptr(target), dt, batch, B, vocab, sps, nsp,
                                 int(seed), int(offset), _ptr(rid), _ptr(out["tokens"]),
                                 _ptr(out["accept_len"]), _ptr(out.get("proposals")),
                                 _ptr(out.get("flags")), wsp, wsn, _stream(stream)),
           "uno_sample_linear_ex")
    out["workspace"] = workspace
    return out


def _build_tree_impl(draft, K, V, temperature, top_k, top_p, out=None, workspace=None, stream=None,
               order=ORDER_TOPK_FIRST):
    """uno_build_tree: draft [batch, B, vocab] -> node arrays [batch, V+1], num_nodes [batch]."""
    lib = load_library()
    assert draft.is_cuda and draft.is_contiguous()
    batch, B, vocab = draft.shape
    dt = _dtype_code(draft)
    dev = draft.device
    if out is None:
        out = dict(node_token=torch.empty((batch, V + 1), dtype=torch.int32, device=dev),
                   node_parent=torch.empty((batch, V + 1), dtype=torch.int32, device=dev),
                   node_depth=torch.empty((batch, V + 1), dtype=torch.int32, device=dev),
                   node_score=torch.empty((batch, V + 1), dtype=torch.float64, device=dev),
                   num_nodes=torch.empty(batch, dtype=torch.int32, device=dev))
    if workspace is None:
        nb = workspace_bytes(OP_BUILD_TREE, batch, B, K, V, vocab, dt, temperature, top_k, top_p, order)
        workspace = _workspace(nb, dev, None)
    wsp, wsn = _aligned_ptr(workspace)
    sps, nsp = _sp_set(batch, temperature, top_k, top_p, order)
    _check(lib.uno_build_tree_ex(_ptr(draft), dt, batch, B, int(K), int(V), vocab, sps, nsp,
                              _ptr(out["node_token"]), _ptr(out["node_parent"]),
                              _ptr(out["node_depth"]), _ptr(out.get("node_score")),
                              _ptr(out["num_nodes"]), wsp, wsn, _stream(stream)), "uno_build_tree_ex")
    out["workspace"] = workspace
    return out


def _verify_tree_impl(target, B, node_token, node_parent, num_nodes, temperature, top_k, top_p, seed,
                offset, request_ids=None, out=None, workspace=None, stream=None, order=ORDER_TOPK_FIRST):
    """uno_verify_tree: target [batch, V+1, vocab] and a tree from build_tree."""
    lib = load_library()
    assert target.is_cuda and target.is_contiguous()
    batch, V1, vocab = target.shape
    V = V1 - 1
    dt = _dtype_code(target)
    dev = target.device
    for t in (node_token, node_parent):
        assert t.dtype == torch.int32 and t.shape == (batch, V1) and t.is_contiguous()
    assert num_nodes.dtype == torch.int32 and num_nodes.shape == (batch,)
    if out is None:
        out = dict(tokens=torch.empty((batch, B + 1), dtype=torch.int32, device=dev),
                   path=torch.empty((batch, B + 1), dtype=torch.int32, device=dev),
                   accept_len=torch.empty(batch, dtype=torch.int32, device=dev),
                   flags=torch.empty(batch, dtype=torch.int32, device=dev))
    if workspace is None:
        nb = workspace_bytes(OP_VERIFY_TREE, batch, B, 1, V, vocab, dt, temperature, top_k, top_p, order)
        workspace = _workspace(nb, dev, None)
    wsp, wsn = _aligned_ptr(workspace)
    rid = _as_u32_ids(request_ids, batch, dev)
    sps, nsp = _sp_set(batch, temperature, top_k, top_p, order)
    _check(lib.uno_verify_tree_ex(_ptr(target), dt, batch, int(B), V, vocab, sps, nsp,
                               int(seed), int(offset), _ptr(rid), _ptr(node_token),
                               _ptr(node_parent), _ptr(num_nodes), _ptr(out["tokens"]),
                               _ptr(out["path"]), _ptr(out["accept_len"]), _ptr(out.get("flags")),
                               wsp, wsn, _stream(stream)), "uno_verify_tree_ex")
    out["workspace"] = workspace
    return out


def _tree_attention_impl(q, k, v, o_prefix, lse_prefix, node_parent, num_nodes, scale, out=None, stream=None):
    """uno_tree_attention: q, o_prefix [batch, n, Hq, D], k, v [batch, n, Hkv, D] (bf16),
    lse_prefix [batch, n, Hq] (fp32), node_parent [batch, n], num_nodes [batch] or None.
    Returns dict(o [batch, n, Hq, D] bf16, lse [batch, n, Hq] fp32)."""
    lib = load_library()
    batch, n, Hq, D = q.shape
    Hkv = k.shape[2]
    for t in (q, k, v, o_prefix):
        assert t.is_cuda and t.is_contiguous() and t.dtype == torch.bfloat16
    assert k.shape == (batch, n, Hkv, D) and v.shape == k.shape and o_prefix.shape == q.shape
    assert lse_prefix.dtype == torch.float32 and lse_prefix.shape == (batch, n, Hq) and lse_prefix.is_contiguous()
    assert node_parent.dtype == torch.int32 and node_parent.shape == (batch, n) and node_parent.is_contiguous()
    if num_nodes is not None:
        assert num_nodes.dtype == torch.int32 and num_nodes.shape == (batch,)
    if out is None:
        out = dict(o=torch.empty_like(q), lse=torch.empty_like(lse_prefix))
    _check(lib.uno_tree_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(o_prefix), _ptr(lse_prefix), _ptr(node_parent),
                                  _ptr(num_nodes), 1, batch, n, Hq, Hkv, D, float(scale), _ptr(out["o"]),
                                  _ptr(out["lse"]), _stream(stream)), "uno_tree_attention")
    return out


def filter_rows(logits, temperature, top_k, top_p, cap=None, workspace=None, stream=None,
                order=ORDER_TOPK_FIRST):
    """uno_filter over logits [rows, vocab].  Returns dict of device tensors:
    ids/probs [rows, cap] (sparse modes), count [rows], stats [rows, 2]."""
    with _on(stream):
        return _filter_rows_impl(logits, temperature, top_k, top_p, cap, workspace, stream, order)


def sample_linear(draft, target, temperature, top_k, top_p, seed, offset, request_ids=None,
                  out=None, workspace=None, stream=None, order=ORDER_TOPK_FIRST):
    """uno_sample_linear: draft [batch, B, vocab], target [batch, B+1, vocab]."""
    with _on(stream):
        return _sample_linear_impl(draft, target, temperature, top_k, top_p, seed, offset, request_ids, out,
                                   workspace, stream, order)


def build_tree(draft, K, V, temperature, top_k, top_p, out=None, workspace=None, stream=None,
               order=ORDER_TOPK_FIRST):
    """uno_build_tree: draft [batch, B, vocab] -> node arrays [batch, V+1], num_nodes [batch]."""
    with _on(stream):
        return _build_tree_impl(draft, K, V, temperature, top_k, top_p, out, workspace, stream, order)


def verify_tree(target, B, node_token, node_parent, num_nodes, temperature, top_k, top_p, seed,
                offset, request_ids=None, out=None, workspace=None, stream=None, order=ORDER_TOPK_FIRST):
    """uno_verify_tree: target [batch, V+1, vocab] and a tree from build_tree."""
    with _on(stream):
        return _verify_tree_impl(target, B, node_token, node_parent, num_nodes, temperature, top_k, top_p, seed,
                                 offset, request_ids, out, workspace, stream, order)


def tree_attention(q, k, v, o_prefix, lse_prefix, node_parent, num_nodes, scale, out=None, stream=None):
    """uno_tree_attention: q, o_prefix [batch, n, Hq, D], k, v [batch, n, Hkv, D] (bf16),
    lse_prefix [batch, n, Hq] (fp32), node_parent [batch, n], num_nodes [batch] or None.
    Returns dict(o [batch, n, Hq, D] bf16, lse [batch, n, Hq] fp32)."""
    with _on(stream):
        return _tree_attention_impl(q, k, v, o_prefix, lse_prefix, node_parent, num_nodes, scale, out, stream)
