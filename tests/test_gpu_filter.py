"""GPU parity of uno_filter against the oracle (sparse supports and dense statistics)."""
import numpy as np
import pytest
import torch

import lossless_draft_verify_amd as uno
import oracle
from gpu_util import device, np_of, say

pytestmark = pytest.mark.gpu


def _rows(rng, rows, N, scale=2.0):
    return (rng.standard_normal((rows, N)) * scale).astype(np.float32)


def _check_sparse(z32, dtype, T, k, p, label, order=uno.ORDER_TOPK_FIRST):
    dev = device()
    zt = torch.from_numpy(z32).to(dev).to(dtype).contiguous()
    zh = zt.float().cpu().numpy()                     # exact values the GPU sees
    g = uno.filter_rows(zt, T, k, p, order=order)
    torch.cuda.synchronize()
    cap = g["ids"].shape[1]
    o = oracle.filter_rows(zh, T, k, p, cap=cap, dense=False, order=order)
    gn, gi, gp = np_of(g["count"]), np_of(g["ids"]), np_of(g["probs"])
    # rows whose top-p cut sits within rounding of the threshold may cut differently
    near = o["margin"] < 1e-9
    worst = 0.0
    for r in range(zh.shape[0]):
        if near[r]:
            continue
        n = int(o["n"][r])
        assert gn[r] == n, (label, r, gn[r], n)
        if n <= 0:
            continue
        assert np.array_equal(gi[r, :n], o["ids"][r, :n]), (label, r)
        assert np.all(gi[r, n:] == -1) and np.all(gp[r, n:] == 0.0)
        rel = np.abs(gp[r, :n] - o["probs"][r, :n]) / o["probs"][r, :n]
        worst = max(worst, float(rel.max()))
    assert worst <= 1e-5, (label, worst)          # parity bar on filtered probabilities
    assert worst <= 1e-12, (label, worst)         # same fp64 operations; only exp may differ by an ulp
    if order == uno.ORDER_JOINT and T > 0:
        # the statistics carry the full-vocabulary normaliser, summed in another
        # order: within the error bound of a recursive sum of N positive terms
        ok = o["n"] > 0
        gs = np_of(g["stats"])
        assert np.array_equal(gs[ok, 0], o["stats"][ok, 0]), label
        np.testing.assert_allclose(gs[ok, 1], o["stats"][ok, 1], rtol=2 * zh.shape[1] * 2.0**-53, atol=0)
    say(f"{label}: rows {zh.shape[0]} max rel err {worst:.2e} near-cut rows {int(near.sum())}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("T,k,p", [(1.0, 50, 0.95), (0.7, 50, 1.0), (1.0, 1, 1.0), (0.0, 0, 1.0),
                                   (1.3, 256, 0.9), (1.0, 7, 0.5), (1.0, 128, 0.97), (1.0, 129, 0.97)])
def test_sparse_many_rows_ragged_vocab(dtype, T, k, p):
    # 1100 rows of a 1003-logit vocabulary: one workgroup per row, rows that start
    # off 16-byte boundaries (scalar head and tail), several tiles per row
    rng = np.random.default_rng(100 + k)
    z = _rows(rng, 1100, 1003)
    _check_sparse(z, dtype, T, k, p, f"ragged {dtype} T{T} k{k} p{p}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("T,k,p", [(1.0, 50, 0.95), (0.0, 0, 1.0), (1.0, 256, 1.0)])
def test_sparse_full_vocab_segmented(dtype, T, k, p):
    # few rows of the full 151936 vocabulary: rows split over segments + merge kernel
    rng = np.random.default_rng(7)
    N = 151936
    rank = np.argsort(rng.random((6, N)), axis=1).astype(np.float32)
    z = (-1.2 * np.log1p(rank) + rng.standard_normal((6, N))).astype(np.float32)
    _check_sparse(z, dtype, T, k, p, f"full-vocab {dtype} T{T} k{k} p{p}")


def test_sparse_full_vocab_one_workgroup_per_row():
    rng = np.random.default_rng(8)
    N, rows = 151936, 1040
    z = (rng.standard_normal((rows, N)) * 1.5).astype(np.float32)
    _check_sparse(z, torch.float32, 1.0, 50, 0.95, "full-vocab 1040 rows f32")


def test_sparse_edge_rows():
    N = 777
    rng = np.random.default_rng(9)
    z = _rows(rng, 12, N)
    z[0, :] = 3.0                            # all tied: smallest ids win
    z[1, ::3] = np.nan                       # NaN counts as -inf
    z[2, 5] = np.inf                         # +inf: invalid row
    z[3, :] = -np.inf                        # no finite logit: invalid row
    z[4, :] = -np.inf
    z[4, [700, 3, 50]] = [1.0, 1.0, 0.5]     # fewer finite logits than k
    z[5, :] = np.round(z[5, :] * 2) / 2      # many ties
    z[6, :] = -0.0
    z[6, ::2] = 0.0                          # signed zeros tie
    z[7, :] = np.linspace(-5, 5, N)          # ascending: every logit beats the running top-k
    z[8, :] = np.linspace(5, -5, N)          # descending
    z[9, :] = 1e-40                          # denormals
    z[9, 17] = 2e-40
    z[10, :] = -3e38
    z[10, 100] = 3e38
    for (T, k, p) in [(1.0, 50, 0.95), (1.0, 5, 1.0), (0.0, 0, 1.0), (2.0, 256, 0.99)]:
        _check_sparse(z, torch.float32, T, k, p, f"edge T{T} k{k} p{p}")
        _check_sparse(z, torch.bfloat16, T, k, p, f"edge-bf16 T{T} k{k} p{p}")


@pytest.mark.parametrize("N", [1, 5, 63, 64, 65, 1000, 4096, 151936])
def test_sparse_small_and_boundary_vocab(N):
    rng = np.random.default_rng(N)
    z = _rows(rng, 5, N)
    _check_sparse(z, torch.float32, 1.0, min(50, max(1, N - 1)), 0.95, f"N={N}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("N,T", [(1000, 1.0), (1003, 0.7), (151936, 0.7), (2049, 2.5)])
def test_dense_statistics(dtype, N, T):
    dev = device()
    rng = np.random.default_rng(N)
    z = _rows(rng, 9, N, scale=3.0)
    z[1, ::7] = -np.inf
    z[2, :] = -np.inf
    z[3, 11] = np.inf
    z[4, ::5] = np.nan
    zt = torch.from_numpy(z).to(dev).to(dtype).contiguous()
    zh = zt.float().cpu().numpy()
    g = uno.filter_rows(zt, T, 0, 1.0)
    torch.cuda.synchronize()
    o = oracle.filter_rows(zh, T, 0, 1.0, dense=False)
    gc, gs = np_of(g["count"]), np_of(g["stats"])
    for r in range(zh.shape[0]):
        if o["n"][r] < 0:
            assert gc[r] == -1, r
            continue
        assert gc[r] == int(np.sum(np.isfinite(zh[r]))), r
        assert gs[r, 0] == o["stats"][r, 0]
        assert abs(gs[r, 1] - o["stats"][r, 1]) <= 1e-13 * o["stats"][r, 1], (r, gs[r, 1], o["stats"][r, 1])
    say(f"dense {dtype} N={N} T={T} ok")


def test_filter_is_deterministic():
    dev = device()
    rng = np.random.default_rng(10)
    z = torch.from_numpy(_rows(rng, 300, 151936)).to(dev)
    a = uno.filter_rows(z, 1.0, 50, 0.95)
    b = uno.filter_rows(z, 1.0, 50, 0.95)
    torch.cuda.synchronize()
    for key in ("ids", "probs", "count"):
        assert torch.equal(a[key], b[key])


# ---- joint filter order: the top-p cut on the full-vocabulary softmax ------------------

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("T,k,p", [(1.0, 50, 0.95), (0.7, 20, 0.8), (1.3, 256, 0.9), (1.0, 7, 0.5),
                                   (0.0, 50, 0.9), (1.0, 50, 1.0)])
def test_joint_order_ragged_vocab(dtype, T, k, p):
    rng = np.random.default_rng(300 + k)
    z = _rows(rng, 1100, 1003)
    _check_sparse(z, dtype, T, k, p, f"joint ragged {dtype} T{T} k{k} p{p}", order=uno.ORDER_JOINT)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows", [6, 1040])
def test_joint_order_full_vocab(dtype, rows):
    # 6 rows: segments and the merge kernel; 1040 rows: one workgroup per row
    rng = np.random.default_rng(9)
    N = 151936
    rank = np.argsort(rng.random((rows, N)), axis=1).astype(np.float32)
    z = (-1.2 * np.log1p(rank) + rng.standard_normal((rows, N))).astype(np.float32)
    _check_sparse(z, dtype, 1.0, 50, 0.95, f"joint full-vocab {rows} rows {dtype}", order=uno.ORDER_JOINT)


def test_joint_order_keeps_at_least_the_default_support():
    dev = device()
    rng = np.random.default_rng(13)
    z = torch.from_numpy(_rows(rng, 500, 4000)).to(dev)
    a = uno.filter_rows(z, 1.0, 40, 0.9)
    b = uno.filter_rows(z, 1.0, 40, 0.9, order=uno.ORDER_JOINT)
    torch.cuda.synchronize()
    na, nb = np_of(a["count"]), np_of(b["count"])
    assert np.all(nb >= na) and np.all(nb <= 40) and np.any(nb > na)


# ---- full-vocabulary nucleus (top-p without top-k) ---------------------------------------

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("N,T,p", [(1003, 1.0, 0.9), (3001, 0.7, 0.5), (5000, 1.5, 0.99), (151936, 1.0, 0.95),
                                   (600000, 1.0, 0.9)])
def test_nucleus_support_size_and_stats(dtype, N, T, p):
    # (600000 logits: more chunks than the one-pass finish tracks, so the
    # first level counts too and the key-bin levels finish every row)
    dev = device()
    rng = np.random.default_rng(N + int(100 * p))
    rows = 12 if N > 100000 else 40
    z = _rows(rng, rows, N, scale=3.0)
    rank = np.argsort(rng.random((4, N)), axis=1).astype(np.float32)
    z[:4] = -1.2 * np.log1p(rank) + rng.standard_normal((4, N)).astype(np.float32)   # long tails
    z[4] = np.round(z[4] * 2) / 2                  # coarse values: ties at the cut
    z[5, ::3] = np.nan                             # NaN counts as -inf
    z[6, ::2] = -np.inf
    z[7] = 0.25                                    # one value everywhere: the cut falls inside a tie
    z[8, 17] = np.inf                              # invalid row
    z[9] = -np.inf                                 # invalid row
    zt = torch.from_numpy(z).to(dev).to(dtype).contiguous()
    zh = zt.float().cpu().numpy()
    g = uno.filter_rows(zt, T, 0, p)
    torch.cuda.synchronize()
    o = oracle.filter_rows(zh, T, 0, p, cap=1, dense=False)
    gc, gs = np_of(g["count"]), np_of(g["stats"])
    near = o["margin"] < 1e-9
    for r in range(rows):
        if o["n"][r] < 0:
            assert gc[r] == -1, r
            continue
        if not near[r]:
            assert gc[r] == o["n"][r], (r, gc[r], o["n"][r])
        assert gs[r, 0] == o["stats"][r, 0], r
        assert abs(gs[r, 1] - o["stats"][r, 1]) <= 2 * N * 2.0**-53 * o["stats"][r, 1], r
    say(f"nucleus {dtype} N={N} T={T} p={p}: sizes {sorted(gc.tolist())[-3:]}, near-cut rows {int(near.sum())}")
