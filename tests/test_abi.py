"""C ABI checks that need no GPU: every declared symbol is exported, status
strings, workspace sizing, and every invalid argument is rejected on the host
before anything is launched (all calls here fail validation, so no HIP call
is made)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import lossless_draft_verify_amd as uno
from lossless_draft_verify_amd import build as hip_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "uno.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
F32, BF16 = 0, 1
FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: validation fails first
FAKE_ODD = ctypes.c_void_p(0x10002)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hip_build.LIB):
        hip_build.build()
    return uno.load_library()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*|size_t)\s+(uno_\w+)\s*\(", text, re.M)))


def sp(T=1.0, k=50, p=0.95, order=0):
    return ctypes.byref(uno.Sampling(T, k, p, order))


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert set(names) >= {"uno_filter", "uno_sample_linear", "uno_build_tree", "uno_verify_tree",
                          "uno_workspace_bytes", "uno_status_string", "uno_last_hip_error",
                          "uno_version"}
    out = subprocess.run(["nm", "-D", "--defined-only", hip_build.LIB], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(uno_\w+)$", out, re.M))
    for n in names:
        assert n in exported, n
        getattr(lib, n)


def test_status_strings_and_version(lib):
    assert lib.uno_status_string(OK) == b"ok"
    for s in (INVALID, UNSUPPORTED, WORKSPACE, -4):
        assert lib.uno_status_string(s) not in (b"ok", b"unknown status")
    assert lib.uno_status_string(12345) == b"unknown status"
    assert b"gfx950" in lib.uno_version()
    assert lib.uno_last_hip_error() == 0


def _ws(lib, op, batch, B, K, V, vocab, dtype, s):
    n = ctypes.c_size_t(0)
    st = lib.uno_workspace_bytes(op, batch, B, K, V, vocab, dtype, s, ctypes.byref(n))
    return st, n.value


def test_workspace_sizes(lib):
    N = 151936
    # linear 8/1/8 b64 sparse: supports only (k = 50) for 1088 rows, no segment partials
    st, n = _ws(lib, uno.OP_SAMPLE_LINEAR, 64, 8, 1, 8, N, F32, sp())
    assert st == OK and n >= 1088 * 50 * (4 + 8) + 1088 * 4
    # dense linear: chunk statistics (max and sum, no finite counts: the
    # samplers never read them) for every row dominate
    st, nd = _ws(lib, uno.OP_SAMPLE_LINEAR, 256, 16, 1, 16, N, BF16, sp(0.7, 0, 1.0))
    nch = math.ceil(N / 2048)
    assert st == OK and nd >= 256 * 33 * nch * (4 + 8)
    # dense filter: the counts too (each row's support size)
    st, ndf = _ws(lib, uno.OP_FILTER, 1000, 0, 0, 0, N, BF16, sp(0.7, 0, 1.0))
    assert st == OK and ndf >= 1000 * nch * (4 + 8 + 4)
    # few rows -> segmented rows need partial lists
    st, nt = _ws(lib, uno.OP_BUILD_TREE, 1, 16, 32, 32, N, F32, sp())
    assert st == OK and nt > 16 * 50 * 12
    st, nv = _ws(lib, uno.OP_VERIFY_TREE, 1, 16, 1, 32, N, F32, sp())
    assert st == OK and nv > 33 * 50 * 12
    # dense tree: exact chunk statistics of every row; the build also keeps
    # K-entry supports with their row statistics
    st, nbd = _ws(lib, uno.OP_BUILD_TREE, 1, 16, 32, 32, N, F32, sp(1.0, 0, 1.0))
    assert st == OK and nbd >= 16 * nch * (4 + 8) + 16 * 32 * (4 + 8) + 16 * 16
    st, nvd = _ws(lib, uno.OP_VERIFY_TREE, 1, 16, 1, 32, N, F32, sp(1.0, 0, 1.0))
    assert st == OK and nvd >= 33 * nch * (4 + 8) + 33 * 4      # and one draw per node row
    # joint order: exact chunk statistics of every filtered row on top of the supports
    st, nj = _ws(lib, uno.OP_SAMPLE_LINEAR, 64, 8, 1, 8, N, F32, sp(order=uno.ORDER_JOINT))
    assert st == OK and nj >= n + 1088 * nch * (4 + 8)
    st, nfj = _ws(lib, uno.OP_FILTER, 4096, 0, 0, 0, N, F32, sp(order=uno.ORDER_JOINT))
    assert st == OK and nfj >= 4096 * nch * (4 + 8)
    # ... which the orders share when only one filter is on
    st, n1 = _ws(lib, uno.OP_SAMPLE_LINEAR, 64, 8, 1, 8, N, F32, sp(1.0, 50, 1.0, uno.ORDER_JOINT))
    assert st == OK and n1 == _ws(lib, uno.OP_SAMPLE_LINEAR, 64, 8, 1, 8, N, F32, sp(1.0, 50, 1.0))[1]
    # nucleus: chunk statistics and a keep threshold per row
    st, nn = _ws(lib, uno.OP_SAMPLE_LINEAR, 256, 16, 1, 16, N, BF16, sp(0.7, 0, 0.9))
    assert st == OK and nn >= nd + 256 * 33 * 8
    st, nfn = _ws(lib, uno.OP_FILTER, 1000, 0, 0, 0, N, BF16, sp(0.7, 0, 0.9))
    assert st == OK and nfn >= 1000 * (nch * (4 + 8) + 8)
    # filter with many rows needs nothing beyond the caller's outputs
    st, nf = _ws(lib, uno.OP_FILTER, 4096, 0, 0, 0, N, F32, sp())
    assert st == OK and nf == 0
    st, _ = _ws(lib, 9, 1, 1, 1, 1, N, F32, sp())
    assert st == INVALID
    assert lib.uno_workspace_bytes(0, 1, 1, 1, 1, N, F32, sp(), None) == INVALID


@pytest.mark.parametrize("T,k,p,expect", [
    (-1.0, 50, 0.95, INVALID), (float("nan"), 50, 0.95, INVALID), (float("inf"), 50, 0.95, INVALID),
    (1.0, 50, 0.0, INVALID), (1.0, 50, 1.5, INVALID), (1.0, 50, float("nan"), INVALID),
    (1.0, 257, 1.0, UNSUPPORTED), (1.0, 300, 0.95, UNSUPPORTED),
])
def test_sampling_parameter_checks(lib, T, k, p, expect):
    st, _ = _ws(lib, uno.OP_SAMPLE_LINEAR, 2, 4, 1, 4, 1000, F32, sp(T, k, p))
    assert st == expect
    ids = ctypes.c_void_p(0x20000)
    assert lib.uno_filter(FAKE, F32, 4, 1000, sp(T, k, p), 256, ids, ids, ids, ids, None, 0, None) == expect


def test_filter_argument_checks(lib):
    out = ctypes.c_void_p(0x20000)
    f = lib.uno_filter
    assert f(FAKE, 2, 4, 1000, sp(), 64, out, out, out, out, None, 0, None) == UNSUPPORTED
    assert f(FAKE, F32, -1, 1000, sp(), 64, out, out, out, out, None, 0, None) == INVALID
    assert f(FAKE, F32, 4, 0, sp(), 64, out, out, out, out, None, 0, None) == INVALID
    assert f(FAKE, F32, 4, 1 << 31, sp(), 64, out, out, out, out, None, 0, None) == INVALID
    assert f(FAKE, F32, 4, 1000, None, 64, out, out, out, out, None, 0, None) == INVALID
    assert f(FAKE, F32, 4, 1000, sp(), 49, out, out, out, out, None, 0, None) == INVALID   # cap < k
    assert f(None, F32, 4, 1000, sp(), 64, out, out, out, out, None, 0, None) == INVALID
    assert f(FAKE, F32, 4, 1000, sp(), 64, None, out, out, out, None, 0, None) == INVALID
    assert f(FAKE, F32, 4, 1000, sp(), 64, out, out, None, out, None, 0, None) == INVALID
    assert f(FAKE_ODD, F32, 4, 1000, sp(), 64, out, out, out, out, None, 0, None) == INVALID
    # dense mode needs stats and a workspace
    assert f(FAKE, F32, 4, 1000, sp(1.0, 0, 1.0), 0, None, None, out, None, None, 0, None) == INVALID
    assert f(FAKE, F32, 4, 1000, sp(1.0, 0, 1.0), 0, None, None, out, out, None, 0, None) == WORKSPACE
    # the full-vocabulary nucleus (top-k off, top_p < 1) is a dense mode too
    assert f(FAKE, F32, 4, 1000, sp(1.0, 0, 0.9), 0, None, None, out, None, None, 0, None) == INVALID
    assert f(FAKE, F32, 4, 1000, sp(1.0, 0, 0.9), 0, None, None, out, out, None, 0, None) == WORKSPACE
    # zero rows is a no-op
    assert f(None, F32, 0, 1000, sp(), 0, None, None, None, None, None, 0, None) == OK


def test_linear_argument_checks(lib):
    f = lib.uno_sample_linear
    o = ctypes.c_void_p(0x30000)
    args = lambda batch=2, B=4, vocab=1000, d=FAKE, t=FAKE, s=None, dt=F32, ws=None, wsn=0, tok=o, acc=o: \
        f(d, t, dt, batch, B, vocab, s or sp(), 1, 0, None, tok, acc, None, None, ws, wsn, None)
    assert args(B=0) == INVALID
    assert args(B=129) == INVALID
    assert args(batch=-1) == INVALID
    assert args(dt=7) == UNSUPPORTED
    assert args(d=None) == INVALID
    assert args(tok=None) == INVALID
    assert args(acc=None) == INVALID
    assert args(d=FAKE_ODD) == INVALID
    assert args() == WORKSPACE                                       # sparse supports need ws
    assert args(s=sp(1.0, 0, 1.0)) == WORKSPACE                      # dense chunk stats need ws
    assert args(ws=ctypes.c_void_p(0x40001), wsn=1 << 30) == WORKSPACE   # misaligned
    assert args(ws=ctypes.c_void_p(0x40000), wsn=16) == WORKSPACE        # too small
    assert args(s=sp(1.0, 0, 0.5)) == WORKSPACE                      # the full-vocabulary nucleus too
    assert args(batch=0, d=None, t=None, tok=None, acc=None) == OK


def test_tree_argument_checks(lib):
    o = ctypes.c_void_p(0x30000)
    bt = lambda B=4, K=4, V=8, s=None, d=FAKE: lib.uno_build_tree(
        d, F32, 2, B, K, V, 1000, s or sp(), o, o, o, None, o, None, 0, None)
    assert bt(V=3) == INVALID              # V < B
    assert bt(V=129, B=4, K=1) == INVALID  # V > 128
    assert bt(K=0) == INVALID
    assert bt(K=300, V=8) == INVALID       # V * K > 2048
    assert bt(B=0) == INVALID
    # full-vocabulary filters: the build picks its K candidates with the top-k path
    assert bt(s=sp(1.0, 0, 1.0)) == WORKSPACE
    assert bt(s=sp(1.0, 0, 1.0), K=257, V=4) == UNSUPPORTED
    assert bt(s=sp(1.0, 0, 0.9)) == WORKSPACE       # full-vocabulary nucleus
    assert bt(d=None) == INVALID
    assert bt() == WORKSPACE
    assert bt(K=256, V=8) == WORKSPACE     # V * K == 2048 is allowed
    vt = lambda B=4, V=8, s=None: lib.uno_verify_tree(
        FAKE, F32, 2, B, V, 1000, s or sp(), 1, 0, None, o, o, o, o, o, o, None, None, 0, None)
    assert vt(V=3) == INVALID
    assert vt(V=200) == INVALID
    assert vt(s=sp(0.5, 0, 1.0)) == WORKSPACE        # dense walk
    assert vt(s=sp(0.5, 0, 0.9)) == WORKSPACE         # full-vocabulary nucleus
    assert vt() == WORKSPACE
    # greedy decoding is a sparse (k = 1) mode
    assert vt(s=sp(0.0, 0, 1.0)) == WORKSPACE


@pytest.mark.parametrize("order", [-1, 2, 7])
def test_unknown_filter_order_is_rejected(lib, order):
    o = ctypes.c_void_p(0x30000)
    n = ctypes.c_size_t(0)
    assert lib.uno_workspace_bytes(uno.OP_FILTER, 4, 0, 0, 0, 1000, F32, sp(order=order),
                                   ctypes.byref(n)) == INVALID
    assert lib.uno_filter(FAKE, F32, 4, 1000, sp(order=order), 64, o, o, o, o, None, 0, None) == INVALID
    assert lib.uno_sample_linear(FAKE, FAKE, F32, 2, 4, 1000, sp(order=order), 1, 0, None, o, o, None,
                                 None, None, 0, None) == INVALID


def test_tree_attention_argument_checks(lib):
    P = ctypes.c_void_p(0x50000)
    f = lambda dt=BF16, batch=2, n=9, Hq=32, Hkv=8, D=128, scale=0.088, q=P, out=P: lib.uno_tree_attention(
        q, P, P, P, P, P, None, dt, batch, n, Hq, Hkv, D, ctypes.c_float(scale), out, P, None)
    assert f(dt=F32) == UNSUPPORTED
    assert f(D=64) == UNSUPPORTED
    assert f(n=0) == INVALID
    assert f(n=131) == INVALID                # more than V + 1 nodes
    assert f(Hq=30) == INVALID                # Hq % Hkv != 0
    assert f(scale=0.0) == INVALID
    assert f(scale=float("nan")) == INVALID
    assert f(q=None) == INVALID
    assert f(out=None) == INVALID
    assert f(batch=0, q=None, out=None) == OK
    odd = ctypes.c_void_p(0x50008)            # k and v must be 16-byte aligned
    assert lib.uno_tree_attention(P, odd, P, P, P, P, None, BF16, 2, 9, 32, 8, 128, ctypes.c_float(0.1), P, P,
                                  None) == INVALID


def _sp_array(*sets):
    arr = (uno.Sampling * len(sets))(*[uno.Sampling(*s) for s in sets])
    return arr, len(sets)


def test_per_request_parameter_checks(lib):
    N = 151936
    n = ctypes.c_size_t(0)
    ws = lambda op, batch, sets: (lib.uno_workspace_bytes_ex(op, batch, 8, 16, 8, N, F32, sets[0], sets[1],
                                                             ctypes.byref(n)), n.value)
    mixed = _sp_array((0.0, 0, 1.0, 0), (1.0, 50, 0.95, 0), (0.7, 20, 1.0, 1), (1.3, 256, 0.9, 0))
    st, nmix = ws(uno.OP_SAMPLE_LINEAR, 4, mixed)
    assert st == OK
    # supports sized for the largest k (256), plus one parameter set per row
    assert nmix >= 4 * 17 * 256 * 12 + 4 * 17 * 40
    assert ws(uno.OP_SAMPLE_LINEAR, 3, mixed)[0] == INVALID            # one set per request
    # top-k sets beside full-softmax and nucleus sets: the call also holds
    # chunk statistics of every row (max fp32 + sum fp64 per 2048-logit chunk)
    # and the dense samplers' scratch
    dense = _sp_array((1.0, 50, 0.95, 0), (1.0, 0, 1.0, 0))
    st, nd = ws(uno.OP_SAMPLE_LINEAR, 2, dense)
    assert st == OK and nd >= 2 * 17 * 75 * 12
    nuc = _sp_array((0.7, 0, 0.9, 0), (1.3, 0, 1.0, 0))
    assert ws(uno.OP_SAMPLE_LINEAR, 2, nuc)[0] == OK
    joint_t = _sp_array((1.0, 50, 0.9, 1), (0.5, 50, 0.9, 1))
    assert ws(uno.OP_SAMPLE_LINEAR, 2, joint_t)[0] == OK               # joint sets, each at its own temperature
    # a full-vocabulary build takes its K candidates from the top-k stream
    st, _ = (lib.uno_workspace_bytes_ex(uno.OP_BUILD_TREE, 2, 2, 300, 2, N, F32, dense[0], dense[1],
                                        ctypes.byref(n)), 0)
    assert st == UNSUPPORTED
    bad = _sp_array((1.0, 50, 0.95, 0), (-1.0, 50, 0.95, 0))
    assert ws(uno.OP_SAMPLE_LINEAR, 2, bad)[0] == INVALID
    assert ws(uno.OP_BUILD_TREE, 4, mixed)[0] == OK
    assert ws(uno.OP_VERIFY_TREE, 4, mixed)[0] == OK
    assert ws(uno.OP_FILTER, 4, mixed)[0] == OK


def test_noalloc_rejects_workspace_beyond_its_scratch(lib):
    # the size check runs on the host before anything else: a dense linear call
    # whose chunk statistics alone exceed the fixed scratch is refused
    N = 151936
    need = _ws(lib, uno.OP_SAMPLE_LINEAR, 1200, 16, 1, 16, N, BF16, sp(0.7, 0, 1.0))[1]
    assert need > uno.NOALLOC_SCRATCH_BYTES
    f = lib.uno_sample_linear_noalloc
    o = ctypes.c_void_p(0x30000)
    assert f(FAKE, FAKE, BF16, 1200, 16, N, sp(0.7, 0, 1.0), 1, 0, None, o, o, None, None, None) == -5
    assert lib.uno_status_string(-5) not in (b"ok", b"unknown status")
    # argument errors come first, as for uno_sample_linear
    assert f(FAKE, FAKE, F32, 2, 0, 1000, sp(), 1, 0, None, o, o, None, None, None) == INVALID
    assert f(FAKE, FAKE, F32, 2, 4, 1000, None, 1, 0, None, o, o, None, None, None) == INVALID


def test_stream_read_argument_checks(lib):
    o = ctypes.c_void_p(0x30000)
    f = lib.uno_stream_read
    assert f(FAKE, 1000, 16, o, None) == INVALID          # bytes not a multiple of 16
    assert f(FAKE, 1024, 24, o, None) == INVALID          # range not a multiple of 16
    assert f(FAKE, 1024, 0, o, None) == INVALID
    assert f(FAKE_ODD, 1024, 16, o, None) == INVALID      # misaligned buffer
    assert f(FAKE, 1024, 16, None, None) == INVALID
    assert f(None, 0, 16, None, None) == OK               # nothing to read
