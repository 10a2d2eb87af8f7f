"""Pins for the oracle's near-threshold margins.

Every GPU/oracle mismatch is excused or fails on the margin the oracle returns,
so each of its parts is pinned here on hand-worked cases whose probabilities
are exact binary fractions (ties, one-hot rows):
  - the inverse-CDF margin: distance of u from the ends of the picked interval,
    in units of the total weight;
  - the acceptance gap |u1 - p(y)/q(y)| of a proposal that p does not always
    accept (reading: thresholds 1.0, i.e. accept iff u1 * q(y) < p(y));
  - every proposal's draw, including those past the first rejection (they are
    reported, so they are compared);
  - the top-p gap |exclusive cumulative sum - top_p| along the filter order;
  - the tree build's smallest relative gap between a popped score and a
    distinct competing frontier score;
  - the walk's draws at every visited node.
The uniforms come from the oracle's Philox, which the published known-answer
vectors pin (test_oracle_philox.py); the expected margins below are worked out
by hand for each case.
"""
import numpy as np
import pytest

import oracle

NEG = -np.inf


def _u(seed, req, pos, offset):
    return [oracle.uniform(seed, req, pos, offset, lane) for lane in range(4)]


@pytest.mark.parametrize("delta", [2.0**-20, 2.0**-30, 2.0**-8])
def test_sample_margin_w13(delta):
    # weights [1, 3]: cumulative 1, 4; u = 0.25 -+ delta puts t = 4u at 1 -+ 4 delta
    w = np.array([1.0, 3.0])
    assert oracle.sample(w, 0.25 - delta) == (0, delta)
    assert oracle.sample(w, 0.25 + delta) == (1, delta)
    # far from the boundary the nearest end decides: u = 0.5 -> t = 2, ends 1 and 4
    assert oracle.sample(w, 0.5) == (1, 0.25)
    # zero weights add no boundaries of their own
    assert oracle.sample(np.array([0.0, 1.0, 0.0, 3.0]), 0.25 + delta) == (3, delta)


def test_sample_margin_single_weight_is_distance_to_either_end():
    for u in (0.125, 0.75, 2.0**-40):
        s, m = oracle.sample(np.array([0.0, 2.0]), u)
        assert s == 1 and m == min(u, 1.0 - u)


def test_top_p_gap():
    # four tied logits: pi = 1/4 each; exclusive sums 0, 1/4, 1/2, 3/4
    z = np.zeros((1, 4), dtype=np.float32)
    p = float(np.float32(0.6))               # parameters cross the boundary as float32
    o = oracle.filter_rows(z, 1.0, 0, 0.6)
    assert o["n"][0] == 3
    assert o["margin"][0] == p - 0.5          # the gap at the third id (1/2 < p), nearest of .35, .1, .15
    o = oracle.filter_rows(z, 1.0, 0, 0.5)     # a cut exactly at a cumulative sum: margin 0
    assert o["n"][0] == 2 and o["margin"][0] == 0.0
    o = oracle.filter_rows(z, 1.0, 0, 0.875)   # gaps .625, .375, .125
    assert o["n"][0] == 4 and o["margin"][0] == 0.125
    o = oracle.filter_rows(z, 1.0, 0, 1.0)     # top-p off: no gap
    assert o["n"][0] == 4 and o["margin"][0] == np.inf
    o = oracle.filter_rows(z, 1.0, 2, 0.75)    # top-k 2 first: pi = 1/2, 1/2; gap |1/2 - 3/4|
    assert o["n"][0] == 2 and o["margin"][0] == 0.25


def test_linear_margin_acceptance_gap():
    # B = 1, vocab 2.  q_0 = one-hot(0), p_0 = (1/2, 1/2), bonus p_1 = one-hot(1).
    # Proposal y_0 = 0 always (margin min(u0, 1-u0)); accept iff u1 < 1/2 (gap
    # |u1 - p/q| = |u1 - 1/2|); accepted: bonus id 1, margin min(u2, 1-u2);
    # rejected: residual (0, 1/2) -> id 1, margin min(u2, 1-u2).
    draft = np.array([[0.0, NEG]], dtype=np.float32)
    target = np.array([[0.0, 0.0], [NEG, 0.0]], dtype=np.float32)
    n, seed, cyc = 4000, 77, 5
    o = oracle.linear(draft, target, 1.0, 0, 1.0, seed, cyc, request_ids=np.arange(n, dtype=np.uint32), batch=n)
    binding = 0
    for r in range(n):
        u0, u1, u2, _ = _u(seed, r, 0, cyc)
        gap = abs(u1 - 0.5)
        want = min(u0, 1 - u0, gap)
        if u1 < 0.5:
            u0b, u1b, u2b, _ = _u(seed, r, 1, cyc)      # the bonus draws word 2 of position B = 1
            want = min(want, u2b, 1 - u2b)
            assert o["tokens"][r].tolist() == [0, 1] and o["accept_len"][r] == 2
        else:
            want = min(want, u2, 1 - u2)
            assert o["tokens"][r].tolist() == [1, -1] and o["accept_len"][r] == 1
        assert o["margin"][r] == want, r
        binding += want == gap
    assert binding > 100            # the acceptance gap decides the margin on many requests


def test_linear_margin_covers_proposals_past_the_first_rejection():
    # B = 2: position 0 always rejects (q_0 = one-hot(0), p_0 = one-hot(1):
    # gap |u1 - 0|); position 1 lies past j* = 0 but its proposal is reported:
    # q_1 = (1/2, 1/2) picks id 0 for u < 1/2 (interval [0, 1/2)), else id 1.
    # The residual at j* = 0 is (0, 1) -> id 1 with margin min(u2, 1 - u2).
    draft = np.array([[0.0, NEG], [0.0, 0.0]], dtype=np.float32)
    target = np.array([[NEG, 0.0], [0.0, 0.0], [0.0, 0.0]], dtype=np.float32)
    n, seed, cyc = 3000, 5, 2**33 + 9          # a cycle index above 2^32
    o = oracle.linear(draft, target, 1.0, 0, 1.0, seed, cyc, request_ids=np.arange(n, dtype=np.uint32), batch=n)
    binding = 0
    for r in range(n):
        u0, u1, u2, _ = _u(seed, r, 0, cyc)
        v0 = _u(seed, r, 1, cyc)[0]
        m_late = min(v0, 0.5 - v0) if v0 < 0.5 else min(v0 - 0.5, 1 - v0)
        want = min(u0, 1 - u0, u1, u2, 1 - u2, m_late)
        assert o["margin"][r] == want, r
        assert o["accept_len"][r] == 1 and o["tokens"][r, 0] == 1
        assert o["proposals"][r].tolist() == [0, 0 if v0 < 0.5 else 1]
        binding += want == m_late
    assert binding > 100


def test_linear_per_request_offsets_match_separate_calls():
    rng = np.random.default_rng(3)
    B, N, n = 3, 40, 12
    draft = (rng.standard_normal((n, B, N)) * 2).astype(np.float32)
    target = (rng.standard_normal((n, B + 1, N)) * 2).astype(np.float32)
    offs = rng.integers(0, 2**40, size=n, dtype=np.uint64)
    rid = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    o = oracle.linear(draft, target, 1.0, 10, 0.9, 2**35 + 1, 0, request_ids=rid, offsets=offs)
    for b in range(n):
        s = oracle.linear(draft[b:b + 1], target[b:b + 1], 1.0, 10, 0.9, 2**35 + 1, int(offs[b]),
                          request_ids=rid[b:b + 1])
        for k in ("tokens", "accept_len", "proposals", "margin"):
            assert np.array_equal(o[k][b], s[k][0]), (b, k)


def test_build_min_gap():
    # depth 1: two tied ids (1/2 each); depth 2: four tied ids (1/4 each), K = 2.
    # Pops: (1/2, rank 0) -- its only competitor ties exactly, no gap; then
    # (1/2, rank 1) against two children of score 1/8: gap (1/2 - 1/8) / (1/2);
    # then a child of score 1/8 against equal scores only.
    draft = np.array([[[0.0, 0.0, NEG, NEG], [0.0, 0.0, 0.0, 0.0]]], dtype=np.float32)
    o = oracle.build_tree(draft, 2, 3, 1.0, 0, 1.0)
    assert o["min_gap"][0] == 0.75
    assert o["num_nodes"][0] == 4
    assert o["node_token"][0].tolist() == [-1, 0, 1, 0]
    assert o["node_parent"][0].tolist() == [-1, 0, 0, 1]
    assert o["node_score"][0].tolist() == [1.0, 0.5, 0.5, 0.125]
    # a chain of one-hot rows has no competitor at all
    chain = np.array([[[0.0, NEG], [NEG, 0.0]]], dtype=np.float32)
    assert oracle.build_tree(chain, 2, 2, 1.0, 0, 1.0)["min_gap"][0] == np.inf


def test_walk_margin():
    # root row (1/2, 1/2); node 1 (token 1, depth 1) has the one-hot row (1, 0).
    # u2 of depth 0 picks id 0 (interval [0, 1/2)) or id 1 ([1/2, 1)); id 1 moves
    # to node 1, whose draw (word 2 of depth 1) has margin min(u, 1 - u).
    target = np.array([[0.0, 0.0], [0.0, NEG]], dtype=np.float32)
    tok, par = np.array([-1, 1], np.int32), np.array([-1, 0], np.int32)
    n, seed, cyc = 2000, 11, 3
    o = oracle.verify_tree(target, 1, tok, par, np.array([2]), 1.0, 0, 1.0, seed, cyc,
                           request_ids=np.arange(n, dtype=np.uint32), batch=n)
    for r in range(n):
        w = _u(seed, r, 0, cyc)[2]
        if w < 0.5:
            want = min(w, 0.5 - w)
            assert o["tokens"][r].tolist() == [0, -1] and o["path"][r].tolist() == [0, -1]
        else:
            w1 = _u(seed, r, 1, cyc)[2]
            want = min(w - 0.5, 1 - w, w1, 1 - w1)
            assert o["tokens"][r].tolist() == [1, 0] and o["path"][r].tolist() == [0, 1]
        assert o["margin"][r] == want, r
