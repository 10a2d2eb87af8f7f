"""Pins for the oracle's row filter (temperature -> top-k -> renormalise -> top-p).

Each case is fixed by hand-derived closed forms, a textbook routine (softmax,
argmax, sort) on special cases, or invariants that follow from the definition.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle


def _support(res, row=0):
    n = int(res["n"][row])
    return list(res["ids"][row, :n]), np.array(res["probs"][row, :n])


# weights 1, 4, 2, 1, 8 -> logits log(w); at T = 1 the softmax is w / sum(w)
W = np.array([1.0, 4.0, 2.0, 1.0, 8.0])
Z = np.log(W).astype(np.float32)
RT = 2e-6   # the logits are float32 roundings of log(w)


def test_hand_example_topk_then_topp():
    # top-4 = ids 4, 1, 2, 0 (ids 0 and 3 tie, the smaller id wins), pi = [8,4,2,1]/15
    # top-p 0.9: cumsum before id 2 is 12/15 = 0.8 < 0.9 -> keep; before id 0 it
    # is 14/15 >= 0.9 -> stop.  Kept {4,1,2} renormalised: [8,4,2]/14.
    r = oracle.filter_rows(Z, 1.0, 4, 0.9)
    ids, p = _support(r)
    assert ids == [4, 1, 2]
    np.testing.assert_allclose(p, np.array([8, 4, 2]) / 14, rtol=RT)
    np.testing.assert_allclose(r["dense"][0], np.array([0, 4, 2, 0, 8]) / 14, rtol=RT)


def test_hand_example_topk_tie_goes_to_smaller_id():
    r = oracle.filter_rows(Z, 1.0, 4, 1.0)
    ids, p = _support(r)
    assert ids == [4, 1, 2, 0]
    np.testing.assert_allclose(p, np.array([8, 4, 2, 1]) / 15, rtol=RT)


def test_hand_example_topp_keeps_first_only():
    # pi(id 4) = 8/15 = 0.533 >= 0.5, so nothing after the first id is kept
    ids, p = _support(oracle.filter_rows(Z, 1.0, 4, 0.5))
    assert ids == [4] and p[0] == 1.0


def test_hand_example_temperature():
    # T = 2 halves the logits: pi ∝ sqrt(w); top-2 = ids 4, 1 -> [sqrt 8, 2] / (sqrt 8 + 2)
    ids, p = _support(oracle.filter_rows(Z, 2.0, 2, 1.0))
    assert ids == [4, 1]
    s8 = math.sqrt(8.0)
    np.testing.assert_allclose(p, [s8 / (s8 + 2), 2 / (s8 + 2)], rtol=RT)


def test_no_filters_is_textbook_softmax():
    rng = np.random.default_rng(3)
    z = rng.normal(size=(4, 257)).astype(np.float32) * 3
    for T in (0.5, 1.0, 1.7):
        r = oracle.filter_rows(z, T, 0, 1.0)
        ref = softmax(z.astype(np.float64) / np.float64(np.float32(T)), axis=1)
        np.testing.assert_allclose(r["dense"], ref, rtol=1e-12, atol=1e-300)
        assert np.all(r["n"] == 257)


def test_topk_off_sentinels():
    z = np.random.default_rng(4).normal(size=(1, 50)).astype(np.float32)
    a = oracle.filter_rows(z, 1.0, 0, 1.0)["dense"]
    b = oracle.filter_rows(z, 1.0, -3, 1.0)["dense"]
    c = oracle.filter_rows(z, 1.0, 50, 1.0)["dense"]
    d = oracle.filter_rows(z, 1.0, 10**6, 1.0)["dense"]
    for x in (b, c, d):
        np.testing.assert_array_equal(a, x)


def test_topk_is_softmax_over_the_k_largest():
    rng = np.random.default_rng(5)
    z = rng.normal(size=(6, 300)).astype(np.float32)
    k = 17
    r = oracle.filter_rows(z, 0.8, k, 1.0)
    for i in range(z.shape[0]):
        order = np.argsort(-z[i].astype(np.float64), kind="stable")[:k]   # ties: smaller id
        ids, p = _support(r, i)
        assert ids == list(order)
        ref = softmax(z[i, order].astype(np.float64) / np.float64(np.float32(0.8)))
        np.testing.assert_allclose(p, ref, rtol=1e-12)


@pytest.mark.parametrize("k", [1, 5, 50])
def test_topk_one_and_tiny_topp_are_argmax(k):
    rng = np.random.default_rng(6)
    z = rng.normal(size=(5, 100)).astype(np.float32)
    z[2, 10] = z[2, 40] = z[2].max() + 1.0       # tie at the max -> id 10
    for res in (oracle.filter_rows(z, 1.0, 1, 1.0), oracle.filter_rows(z, 1.0, k, 1e-6)):
        for i in range(5):
            ids, p = _support(res, i)
            assert ids == [int(np.argmax(z[i]))] and p[0] == 1.0


def test_greedy_temperature_zero():
    rng = np.random.default_rng(7)
    z = rng.normal(size=(5, 64)).astype(np.float32)
    z[1, 3] = z[1, 9] = 50.0
    r = oracle.filter_rows(z, 0.0, 0, 1.0)
    for i in range(5):
        ids, p = _support(r, i)
        assert ids == [int(np.argmax(z[i]))] and p[0] == 1.0
    assert _support(r, 1)[0] == [3]


def test_invariants_random_rows():
    rng = np.random.default_rng(8)
    for trial in range(20):
        N = int(rng.integers(2, 400))
        z = (rng.normal(size=(3, N)) * rng.uniform(0.1, 4)).astype(np.float32)
        T = float(np.float32(rng.uniform(0.2, 2.0)))
        k = int(rng.integers(1, N + 1))
        p = float(np.float32(rng.uniform(0.05, 1.0)))
        r = oracle.filter_rows(z, T, k, p)
        for i in range(3):
            ids, probs = _support(r, i)
            n = len(ids)
            assert 1 <= n <= k
            assert abs(probs.sum() - 1.0) < 1e-12
            zi = z[i].astype(np.float64)
            # kept ids dominate every other id in (z desc, id asc)
            kept = np.zeros(N, bool)
            kept[ids] = True
            if (~kept).any():
                assert zi[kept].min() >= zi[~kept].max()
            # probability ratios are the temperature-scaled exponentials of logit gaps
            for a in range(n):
                np.testing.assert_allclose(probs[a] / probs[0],
                                           math.exp((zi[ids[a]] - zi[ids[0]]) / T), rtol=1e-12)
            # the kept set is the shortest filter-order prefix reaching mass p
            order = np.argsort(-zi, kind="stable")[: min(k, N)]
            pi = softmax(zi[order] / T)
            if p < 1.0:
                assert n == 1 or pi[: n - 1].sum() < p + 1e-12
                assert n == len(order) or pi[:n].sum() >= p - 1e-12
            else:
                assert n == len(order)


def test_nan_counts_as_minus_inf_and_invalid_rows():
    z = np.array([[0.0, np.nan, 1.0, -np.inf],
                  [0.0, np.inf, 1.0, 2.0],
                  [-np.inf, -np.inf, np.nan, -np.inf]], dtype=np.float32)
    r = oracle.filter_rows(z, 1.0, 0, 1.0)
    ids, p = _support(r, 0)
    assert sorted(ids) == [0, 2]
    np.testing.assert_allclose(r["dense"][0], [1 / (1 + math.e), 0, math.e / (1 + math.e), 0],
                               rtol=1e-15)
    assert r["n"][1] == -1 and r["n"][2] == -1
    assert np.all(r["dense"][1] == 0) and np.all(r["dense"][2] == 0)
    # a row with fewer finite logits than k keeps only the finite ones
    ids, p = _support(oracle.filter_rows(z[:1], 1.0, 3, 1.0), 0)
    assert ids == [2, 0]


def test_stats_match_definition():
    rng = np.random.default_rng(9)
    z = rng.normal(size=(2, 500)).astype(np.float32)
    r = oracle.filter_rows(z, 0.7, 0, 1.0)
    for i in range(2):
        m, S = r["stats"][i]
        assert m == z[i].max()
        T = np.float64(np.float32(0.7))
        ref = np.exp((z[i].astype(np.float64) - m) / T).sum()
        assert abs(S - ref) / ref < 1e-13
