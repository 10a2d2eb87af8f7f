"""Plain fp64 CPU oracle for the UNO decode-cycle sampling path (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: only the tests, ``__graft_entry__.smoke()`` and the
bench's ``cpu_baseline`` leg may import this package.  The GPU product path
never imports it and shares no code with it.

Every function here marshals numpy arrays into ``uno_oracle.c``; the method's
arithmetic lives there, each step commented with the passage it follows
(SGLang PR #37667 "native SGLang serving support for UNO": Motivation,
Modifications, filter-order review thread; the run_math_eval walk-through:
B/K/V mapping, startup constraints, TPF accounting).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "uno_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

# Filter orders: top-k, renormalise, then top-p (the default), or joint (the
# top-p cut taken on the full-vocabulary softmax, within the top-k set).
ORDER_TOPK_FIRST = 0
ORDER_JOINT = 1


# UNO_ORACLE_SANITIZE=1 builds and loads an AddressSanitizer + UBSan build
# instead (liboracle_san.so); the process must then start with gcc's libasan
# preloaded (LD_PRELOAD=$(gcc -print-file-name=libasan.so)).
_SANITIZE = os.environ.get("UNO_ORACLE_SANITIZE", "") == "1"
if _SANITIZE:
    _LIB = os.path.join(_HERE, "liboracle_san.so")


def build(force: bool = False) -> str:
    """Compile ``uno_oracle.c`` into ``liboracle.so`` (gcc, -O2, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        opt = (["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                "-fno-sanitize-recover=undefined"] if _SANITIZE else ["-O2"])
        cmd = ["gcc"] + opt + ["-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
                               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, u32, u64, f64 = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                                   ctypes.c_uint64, ctypes.c_double)
        lib.oracle_philox4x32_10.argtypes = [P, P, P]
        lib.oracle_philox4x32_10.restype = None
        lib.oracle_uniform.argtypes = [u64, u32, u32, u64, ctypes.c_int]
        lib.oracle_uniform.restype = f64
        lib.oracle_filter.argtypes = [P, i64, i64, f64, i32, f64, i32, P, P, P, P, i32, P, P]
        lib.oracle_filter.restype = ctypes.c_int
        lib.oracle_sample.argtypes = [P, i64, f64, P]
        lib.oracle_sample.restype = i32
        lib.oracle_linear.argtypes = [P, P, i32, i32, i64, i64, i64, f64, i32, f64, i32, u64, u64, P, P,
                                      P, P, P, P]
        lib.oracle_linear.restype = None
        lib.oracle_build_tree.argtypes = [P, i32, i32, i32, i32, i64, i64, f64, i32, f64, i32,
                                          P, P, P, P, P, P]
        lib.oracle_build_tree.restype = None
        lib.oracle_verify_tree.argtypes = [P, i32, i32, i32, i64, i64, f64, i32, f64, i32, u64, u64, P, P,
                                           P, P, P, P, P, P, P]
        lib.oracle_verify_tree.restype = None
        lib.oracle_tree_attention.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32, f64, P, P]
        lib.oracle_tree_attention.restype = None
        lib.oracle_tpf.argtypes = [P, i64]
        lib.oracle_tpf.restype = f64
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
        return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(x):
    """Logits as contiguous float32 (bf16 inputs must already be widened)."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    return a


def _param(x):
    """Sampling scalars cross the boundary as float32; widen exactly."""
    return float(np.float32(x))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def philox4x32_10(ctr, key):
    lib = _load()
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib.oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def uniform(seed, req, pos, offset, lane):
    return float(_load().oracle_uniform(seed, req, pos, offset, lane))


def filter_rows(z, temperature, top_k, top_p, cap=None, dense=True, order=ORDER_TOPK_FIRST):
    """Filter each row of ``z`` [rows, N].

    Returns dict(dense [rows,N] f64 or None, ids [rows,cap], probs [rows,cap]
    (support in filter order, -1 / 0 padded), n [rows] (-1 = invalid row),
    stats [rows,2] (m, S), margin [rows])."""
    lib = _load()
    z = _f32(z)
    if z.ndim == 1:
        z = z[None, :]
    rows, N = z.shape
    cap = N if cap is None else int(cap)
    d = np.zeros((rows, N), dtype=np.float64) if dense else None
    ids = np.full((rows, cap), -1, dtype=np.int32)
    probs = np.zeros((rows, cap), dtype=np.float64)
    n = np.zeros(rows, dtype=np.int32)
    stats = np.zeros((rows, 2), dtype=np.float64)
    margin = np.zeros(rows, dtype=np.float64)
    rc = lib.oracle_filter(_ptr(z), rows, N, _param(temperature), int(top_k), _param(top_p), int(order),
                           _ptr(d), _ptr(ids), _ptr(probs), _ptr(n), cap, _ptr(stats), _ptr(margin))
    if rc != 0:
        raise MemoryError("oracle_filter: allocation failed")
    return dict(dense=d, ids=ids, probs=probs, n=n, stats=stats, margin=margin)


def sample(w, u):
    lib = _load()
    w = np.ascontiguousarray(w, dtype=np.float64)
    m = np.zeros(1, dtype=np.float64)
    s = lib.oracle_sample(_ptr(w), w.shape[0], float(u), _ptr(m))
    return int(s), float(m[0])


def _req_ids(request_ids, batch):
    if request_ids is None:
        return None
    r = np.ascontiguousarray(request_ids, dtype=np.uint32)
    assert r.shape == (batch,)
    return r


def _offsets(offsets, batch):
    if offsets is None:
        return None
    r = np.ascontiguousarray(offsets, dtype=np.uint64)
    assert r.shape == (batch,)
    return r


def linear(draft, target, temperature, top_k, top_p, seed, offset, request_ids=None,
           batch=None, order=ORDER_TOPK_FIRST, offsets=None):
    """One linear UNO cycle per request.

    draft [batch, B, N] and target [batch, B+1, N]; with ``batch`` given and
    2-D inputs ([B, N], [B+1, N]) all requests share the same rows.
    ``offsets`` [batch] (optional): request b's cycle index instead of ``offset``.
    Returns dict(tokens [batch, B+1], accept_len [batch], proposals [batch, B],
    margin [batch])."""
    lib = _load()
    draft = _f32(draft)
    target = _f32(target)
    if draft.ndim == 2:
        assert batch is not None
        B, N = draft.shape
        ds = ts = 0
    else:
        batch, B, N = draft.shape
        ds, ts = B * N, (B + 1) * N
    assert target.shape[-2:] == (B + 1, N)
    tokens = np.zeros((batch, B + 1), dtype=np.int32)
    acc = np.zeros(batch, dtype=np.int32)
    prop = np.zeros((batch, B), dtype=np.int32)
    mg = np.zeros(batch, dtype=np.float64)
    rid = _req_ids(request_ids, batch)
    offs = _offsets(offsets, batch)
    lib.oracle_linear(_ptr(draft), _ptr(target), batch, B, N, ds, ts, _param(temperature),
                      int(top_k), _param(top_p), int(order), int(seed), int(offset), _ptr(rid), _ptr(offs),
                      _ptr(tokens), _ptr(acc), _ptr(prop), _ptr(mg))
    return dict(tokens=tokens, accept_len=acc, proposals=prop, margin=mg)


def build_tree(draft, K, V, temperature, top_k, top_p, order=ORDER_TOPK_FIRST):
    """Best-first candidate tree per request from draft [batch, B, N]."""
    lib = _load()
    draft = _f32(draft)
    batch, B, N = draft.shape
    tok = np.zeros((batch, V + 1), dtype=np.int32)
    par = np.zeros((batch, V + 1), dtype=np.int32)
    dep = np.zeros((batch, V + 1), dtype=np.int32)
    sc = np.zeros((batch, V + 1), dtype=np.float64)
    nn = np.zeros(batch, dtype=np.int32)
    gap = np.zeros(batch, dtype=np.float64)
    lib.oracle_build_tree(_ptr(draft), batch, B, int(K), int(V), N, B * N, _param(temperature),
                          int(top_k), _param(top_p), int(order), _ptr(tok), _ptr(par), _ptr(dep), _ptr(sc),
                          _ptr(nn), _ptr(gap))
    return dict(node_token=tok, node_parent=par, node_depth=dep, node_score=sc, num_nodes=nn,
                min_gap=gap)


def verify_tree(target, B, node_token, node_parent, num_nodes, temperature, top_k, top_p,
                seed, offset, request_ids=None, batch=None, order=ORDER_TOPK_FIRST, offsets=None):
    """Target-sampled tree walk per request over target [batch, V+1, N].

    With ``batch`` given and a 2-D target [V+1, N] plus one tree ([V+1], [V+1],
    scalar), every request shares those rows and that tree.  ``offsets``
    [batch] (optional): request b's cycle index instead of ``offset``."""
    lib = _load()
    target = _f32(target)
    if target.ndim == 2:
        assert batch is not None
        V1, N = target.shape
        stride = 0
        node_token = np.tile(np.asarray(node_token, dtype=np.int32).reshape(1, V1), (batch, 1))
        node_parent = np.tile(np.asarray(node_parent, dtype=np.int32).reshape(1, V1), (batch, 1))
        num_nodes = np.full(batch, int(np.asarray(num_nodes).ravel()[0]), dtype=np.int32)
    else:
        batch, V1, N = target.shape
        stride = V1 * N
    V = V1 - 1
    tk = np.ascontiguousarray(node_token, dtype=np.int32)
    pa = np.ascontiguousarray(node_parent, dtype=np.int32)
    nn = np.ascontiguousarray(num_nodes, dtype=np.int32)
    assert tk.shape == (batch, V + 1) and pa.shape == (batch, V + 1) and nn.shape == (batch,)
    tokens = np.zeros((batch, B + 1), dtype=np.int32)
    path = np.zeros((batch, B + 1), dtype=np.int32)
    acc = np.zeros(batch, dtype=np.int32)
    mg = np.zeros(batch, dtype=np.float64)
    rid = _req_ids(request_ids, batch)
    offs = _offsets(offsets, batch)
    lib.oracle_verify_tree(_ptr(target), batch, int(B), V, N, stride, _param(temperature),
                           int(top_k), _param(top_p), int(order), int(seed), int(offset), _ptr(rid), _ptr(offs),
                           _ptr(tk), _ptr(pa), _ptr(nn), _ptr(tokens), _ptr(path), _ptr(acc),
                           _ptr(mg))
    return dict(tokens=tokens, path=path, accept_len=acc, margin=mg)


def tpf(accept_len):
    a = np.ascontiguousarray(accept_len, dtype=np.int32).ravel()
    return float(_load().oracle_tpf(_ptr(a), a.shape[0]))


def tree_attention(q, k, v, o_prefix, lse_prefix, node_parent, num_nodes, scale):
    """Tree-suffix attention merged with the prefix state, per request.

    q, o_prefix [batch, n, Hq, D]; k, v [batch, n, Hkv, D]; lse_prefix [batch, n, Hq];
    node_parent [batch, n]; num_nodes [batch].  Returns dict(o [batch, n, Hq, D],
    lse [batch, n, Hq]) in float64 (rows at or past num_nodes are zero)."""
    lib = _load()
    q, k, v, op = _f32(q), _f32(k), _f32(v), _f32(o_prefix)
    lp = _f32(lse_prefix)
    batch, n, Hq, D = q.shape
    Hkv = k.shape[2]
    assert k.shape == (batch, n, Hkv, D) and v.shape == k.shape and op.shape == q.shape
    assert lp.shape == (batch, n, Hq) and Hq % Hkv == 0
    par = np.ascontiguousarray(node_parent, dtype=np.int32)
    nn = np.ascontiguousarray(num_nodes, dtype=np.int32)
    o = np.zeros((batch, n, Hq, D), dtype=np.float64)
    lse = np.zeros((batch, n, Hq), dtype=np.float64)
    lib.oracle_tree_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(op), _ptr(lp), _ptr(par), _ptr(nn),
                              batch, n, Hq, Hkv, D, float(scale), _ptr(o), _ptr(lse))
    return dict(o=o, lse=lse)
