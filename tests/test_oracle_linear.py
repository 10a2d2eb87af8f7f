"""Pins for the oracle's sampling primitive and linear UNO cycle.

Losslessness is checked by chi-square over many Philox streams (requests that
share one set of rows), the acceptance rate against its closed form, and the
special cases q = p, disjoint supports and greedy decoding.
"""
import numpy as np
import pytest

import oracle
from stats_util import chisq_pvalue, mean_zscore

P_MIN = 1e-4     # fixed seeds: these are deterministic outcomes, not flaky draws


def test_sample_boundaries_brute_force():
    w = np.array([0.0, 1.0, 0.0, 3.0])       # cumulative 0, 1, 1, 4
    assert oracle.sample(w, 0.0)[0] == 1
    assert oracle.sample(w, 0.2499)[0] == 1
    assert oracle.sample(w, 0.25)[0] == 3     # t = 1.0 is not > cumulative 1 -> next
    assert oracle.sample(w, 0.9999)[0] == 3
    assert oracle.sample(np.zeros(4), 0.3)[0] == -1
    # unnormalised weights pick the same ids as normalised ones
    rng = np.random.default_rng(1)
    v = rng.random(50) * (rng.random(50) < 0.5)
    for u in rng.random(200):
        a, _ = oracle.sample(v, u)
        cdf = np.cumsum(v / v.sum())
        assert a == int(np.searchsorted(cdf, u, side="right"))


def _rows(rng, B, N, scale=1.5):
    target = (rng.normal(size=(B + 1, N)) * scale).astype(np.float32)
    draft = (target[:B] + rng.normal(size=(B, N)) * 0.8).astype(np.float32)
    return draft, target


def _filtered(z, T, k, p):
    return oracle.filter_rows(z, T, k, p)["dense"]


@pytest.mark.parametrize("T,k,p", [(1.0, 0, 1.0), (0.8, 5, 0.9), (1.3, 3, 1.0)])
def test_linear_is_lossless(T, k, p):
    rng = np.random.default_rng(11)
    B, N, n = 3, 8, 120_000
    draft, target = _rows(rng, B, N)
    out = oracle.linear(draft, target, T, k, p, seed=1234, offset=0,
                        request_ids=np.arange(n, dtype=np.uint32), batch=n)
    tok, acc = out["tokens"], out["accept_len"]
    P = _filtered(target, T, k, p)
    Q = _filtered(draft, T, k, p)
    # token at index j, among cycles that emit it, follows the filtered target row j
    for j in range(B + 1):
        sel = acc >= j + 1
        assert chisq_pvalue(tok[sel, j], P[j]) > P_MIN, j
    # acceptance: alpha_j = sum min(p_j, q_j); E[accept_len] = sum_n prod_{j<n} alpha_j
    alpha = np.minimum(P[:B], Q).sum(axis=1)
    expect = sum(np.prod(alpha[:m]) for m in range(B + 1))
    assert abs(mean_zscore(acc, expect)) < 4.0
    # after a rejection at j the emitted token follows max(0, p_j - q_j) renormalised
    for j in range(B):
        sel = acc == j + 1
        if sel.sum() < 2000:
            continue
        res = np.maximum(P[j] - Q[j], 0.0)
        assert chisq_pvalue(tok[sel, j], res / res.sum()) > P_MIN, j
    # proposals follow the filtered draft rows
    for j in range(B):
        assert chisq_pvalue(out["proposals"][:, j], Q[j]) > P_MIN


def test_q_equals_p_accepts_every_proposal():
    rng = np.random.default_rng(12)
    B, N = 5, 300
    target = rng.normal(size=(B + 1, N)).astype(np.float32) * 2
    for (T, k, p) in [(1.0, 0, 1.0), (1.0, 50, 0.95), (0.6, 7, 1.0)]:
        out = oracle.linear(target[:B], target, T, k, p, seed=7, offset=3,
                            request_ids=np.arange(5000, dtype=np.uint32), batch=5000)
        assert np.all(out["accept_len"] == B + 1)
        np.testing.assert_array_equal(out["tokens"][:, :B], out["proposals"])


def test_disjoint_supports_accept_nothing():
    rng = np.random.default_rng(13)
    B, N, n = 3, 40, 60_000
    target = rng.normal(size=(B + 1, N)).astype(np.float32)
    draft = rng.normal(size=(B, N)).astype(np.float32)
    target[:, :4] += 20.0    # target top-4 = ids 0..3
    draft[:, 10:14] += 20.0  # draft top-4 = ids 10..13
    out = oracle.linear(draft, target, 1.0, 4, 1.0, seed=99, offset=0,
                        request_ids=np.arange(n, dtype=np.uint32), batch=n)
    assert np.all(out["accept_len"] == 1)
    assert np.all(out["tokens"][:, 1:] == -1)
    P = _filtered(target, 1.0, 4, 1.0)
    assert chisq_pvalue(out["tokens"][:, 0], P[0]) > P_MIN


def test_greedy_is_the_longest_matching_argmax_prefix():
    rng = np.random.default_rng(14)
    B, N = 6, 100
    for trial in range(20):
        target = rng.normal(size=(B + 1, N)).astype(np.float32)
        draft = rng.normal(size=(B, N)).astype(np.float32)
        m = int(rng.integers(0, B + 1))      # first m draft argmaxes agree with the target
        for j in range(m):
            draft[j] = target[j] + 0.01 * rng.normal(size=N).astype(np.float32)
            draft[j, np.argmax(target[j])] += 10
        out = oracle.linear(draft, target, 0.0, 0, 1.0, seed=trial, offset=0,
                            request_ids=np.arange(4, dtype=np.uint32), batch=4)
        ta = np.argmax(target, axis=1)
        da = np.argmax(draft, axis=1)
        L = 0
        while L < B and da[L] == ta[L]:
            L += 1
        expect = list(ta[:L]) + [int(ta[L])] + [-1] * (B - L)
        for b in range(4):
            assert out["accept_len"][b] == L + 1
            assert list(out["tokens"][b]) == expect


def test_batched_rows_match_per_request_calls():
    rng = np.random.default_rng(15)
    B, N, batch = 4, 64, 6
    draft = rng.normal(size=(batch, B, N)).astype(np.float32)
    target = rng.normal(size=(batch, B + 1, N)).astype(np.float32)
    rid = np.array([5, 9, 1, 0, 77, 3], dtype=np.uint32)
    out = oracle.linear(draft, target, 0.9, 10, 0.9, seed=5, offset=11, request_ids=rid)
    for b in range(batch):
        one = oracle.linear(draft[b], target[b], 0.9, 10, 0.9, seed=5, offset=11,
                            request_ids=rid[b:b + 1], batch=1)
        np.testing.assert_array_equal(one["tokens"][0], out["tokens"][b])
        assert one["accept_len"][0] == out["accept_len"][b]


def test_tpf_identity():
    acc = np.array([1, 2, 3, 9, 4], dtype=np.int32)
    # two target forwards per cycle: tokens / (2 * cycles)
    assert oracle.tpf(acc) == acc.sum() / (2 * acc.size)
