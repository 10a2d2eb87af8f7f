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


# ---- joint filter order: the top-p cut on the full-vocabulary softmax ------------------

def test_hand_example_joint_keeps_more_than_topk_first():
    # weights 1, 4, 2, 1, 8 (sum 16); top-3 = ids 4, 1, 2 (weights 8, 4, 2).
    # Top-k first, top-p 0.8: pi = [8,4,2]/14; cumsum before id 2 is 12/14 >= 0.8 -> {4, 1}.
    # Joint, top-p 0.8: full-softmax pi = [8,4,2]/16; before id 2 it is 12/16 < 0.8 -> keep;
    # the top-k set ends there -> {4, 1, 2} renormalised: [8,4,2]/14.
    ids, p = _support(oracle.filter_rows(Z, 1.0, 3, 0.8))
    assert ids == [4, 1]
    np.testing.assert_allclose(p, [8 / 12, 4 / 12], rtol=RT)
    r = oracle.filter_rows(Z, 1.0, 3, 0.8, order=oracle.ORDER_JOINT)
    ids, p = _support(r)
    assert ids == [4, 1, 2]
    np.testing.assert_allclose(p, [8 / 14, 4 / 14, 2 / 14], rtol=RT)
    # the statistics report the full-vocabulary normaliser (weights relative to the max 8)
    np.testing.assert_allclose(r["stats"][0], [math.log(8.0), 16 / 8], rtol=RT)
    # top-p 0.7: 12/16 >= 0.7 stops the joint cut before id 2 as well
    ids, p = _support(oracle.filter_rows(Z, 1.0, 3, 0.7, order=oracle.ORDER_JOINT))
    assert ids == [4, 1]
    np.testing.assert_allclose(p, [8 / 12, 4 / 12], rtol=RT)


@pytest.mark.parametrize("T,k,p", [(1.0, 20, 1.0), (0.7, 0, 0.9), (1.3, 1, 0.5), (0.0, 10, 0.9),
                                   (1.0, 400, 0.9)])
def test_joint_equals_topk_first_when_one_filter_is_off(T, k, p):
    # with top-p off, top-k off (k 0 or >= vocab), k = 1 or greedy there is only one reading
    rng = np.random.default_rng(11)
    z = (rng.standard_normal((6, 300)) * 2).astype(np.float32)
    a = oracle.filter_rows(z, T, k, p)
    b = oracle.filter_rows(z, T, k, p, order=oracle.ORDER_JOINT)
    for key in ("n", "ids", "probs"):
        assert np.array_equal(a[key], b[key]), key


def test_joint_is_the_smallest_prefix_reaching_top_p():
    # brute force on small rows: over the top-k order, the joint support is the
    # shortest prefix whose full-softmax mass (scipy) reaches top_p, capped at k;
    # the default order's support is never larger
    rng = np.random.default_rng(12)
    N, checked = 40, 0
    for trial in range(300):
        T = float(rng.choice([0.5, 1.0, 1.7]))
        k = int(rng.integers(2, 30))
        p = float(rng.uniform(0.2, 0.99))
        z = (rng.standard_normal(N) * 2).astype(np.float32)
        order = sorted(range(N), key=lambda i: (-float(z[i]), i))
        full = softmax(z.astype(np.float64) / float(np.float32(T)))    # parameters are float32
        mass = np.cumsum(full[order])
        if np.any(np.abs(mass[:k] - p) < 1e-9):
            continue
        L = next((n + 1 for n in range(k) if mass[n] >= p), k)
        r = oracle.filter_rows(z, T, k, p, order=oracle.ORDER_JOINT)
        ids, pr = _support(r)
        assert ids == order[:L], (trial, ids, order[:L])
        np.testing.assert_allclose(pr, full[order[:L]] / full[order[:L]].sum(), rtol=1e-12)
        ids_default, _ = _support(oracle.filter_rows(z, T, k, p))
        assert ids[:len(ids_default)] == ids_default and len(ids_default) <= L
        checked += 1
    assert checked > 250


def test_full_vocabulary_nucleus_is_the_smallest_prefix():
    # top-k off, top-p on: brute force over the whole row (scipy softmax, stable
    # sort): the support is the shortest (z desc, id asc) prefix whose mass reaches
    # top_p, ties at the cut going to the smaller ids; coarse values make ties common
    rng = np.random.default_rng(21)
    checked = 0
    for trial in range(120):
        N = int(rng.integers(300, 3000))
        T = float(np.float32(rng.choice([0.6, 1.0, 1.5])))
        p = float(np.float32(rng.uniform(0.3, 0.99)))
        z = (np.round(rng.standard_normal(N) * 8) / 4).astype(np.float32)
        order = sorted(range(N), key=lambda i: (-float(z[i]), i))
        full = softmax(z.astype(np.float64) / T)
        mass = np.cumsum(full[order])
        if np.any(np.abs(mass - p) < 1e-9):
            continue
        L = int(np.argmax(mass >= p)) + 1
        ids, pr = _support(oracle.filter_rows(z, T, 0, p))
        assert ids == order[:L], trial
        np.testing.assert_allclose(pr, full[order[:L]] / full[order[:L]].sum(), rtol=1e-12)
        checked += 1
    assert checked > 100
