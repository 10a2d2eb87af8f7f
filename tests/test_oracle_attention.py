"""Pins for the oracle's tree-suffix attention with the prefix-state merge.

The merge must equal one softmax attention over the prefix keys and the visible
suffix keys together (a textbook identity of log-sum-exp merging); a chain tree
is causal attention; a lone node returns its own value; padding nodes are never
read.  Every reference here is computed directly with numpy/scipy.
"""
import numpy as np
from scipy.special import logsumexp, softmax

import oracle


def _inputs(rng, batch, n, Hq, Hkv, D, P):
    q = rng.standard_normal((batch, n, Hq, D)).astype(np.float32)
    k = rng.standard_normal((batch, n, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((batch, n, Hkv, D)).astype(np.float32)
    kp = rng.standard_normal((batch, P, Hkv, D)).astype(np.float32)
    vp = rng.standard_normal((batch, P, Hkv, D)).astype(np.float32)
    return q, k, v, kp, vp


def _random_tree(rng, n):
    par = np.full(n, -1, dtype=np.int32)
    for i in range(1, n):
        par[i] = rng.integers(0, i)
    return par


def _ancestors(par, i):
    out = []
    while i >= 0:
        out.append(i)
        i = par[i]
    return out


def test_merge_equals_one_softmax_over_prefix_and_visible_suffix():
    rng = np.random.default_rng(1)
    batch, n, Hq, Hkv, D, P = 3, 9, 8, 2, 16, 11
    G = Hq // Hkv
    scale = float(np.float32(1 / np.sqrt(D)))
    q, k, v, kp, vp = _inputs(rng, batch, n, Hq, Hkv, D, P)
    par = np.stack([_random_tree(rng, n) for _ in range(batch)])
    # the prefix state of every query: attention over the prefix keys alone
    op = np.zeros((batch, n, Hq, D), np.float32)
    lp = np.zeros((batch, n, Hq), np.float32)
    for b in range(batch):
        for i in range(n):
            for h in range(Hq):
                s = scale * (kp[b, :, h // G].astype(np.float64) @ q[b, i, h].astype(np.float64))
                lp[b, i, h] = logsumexp(s)
                op[b, i, h] = softmax(s) @ vp[b, :, h // G].astype(np.float64)
    r = oracle.tree_attention(q, k, v, op, lp, par, np.full(batch, n), scale)
    for b in range(batch):
        for i in range(n):
            vis = sorted(_ancestors(par[b], i))
            for h in range(Hq):
                K = np.concatenate([kp[b, :, h // G], k[b, vis, h // G]]).astype(np.float64)
                Vv = np.concatenate([vp[b, :, h // G], v[b, vis, h // G]]).astype(np.float64)
                s = scale * (K @ q[b, i, h].astype(np.float64))
                # the prefix state went through float32, so compare at that precision
                np.testing.assert_allclose(r["lse"][b, i, h], logsumexp(s), rtol=1e-6, atol=1e-6)
                np.testing.assert_allclose(r["o"][b, i, h], softmax(s) @ Vv, rtol=1e-5, atol=1e-6)


def test_chain_tree_is_causal_attention_and_empty_prefix():
    rng = np.random.default_rng(2)
    batch, n, Hq, Hkv, D = 2, 7, 4, 4, 8
    q, k, v, _, _ = _inputs(rng, batch, n, Hq, Hkv, D, 1)
    par = np.tile(np.arange(-1, n - 1, dtype=np.int32), (batch, 1))
    lp = np.full((batch, n, Hq), -np.inf, np.float32)
    op = rng.standard_normal((batch, n, Hq, D)).astype(np.float32)     # ignored: empty prefix
    scale = 0.5
    r = oracle.tree_attention(q, k, v, op, lp, par, np.full(batch, n), scale)
    for b in range(batch):
        for h in range(Hq):
            s = scale * (q[b, :, h].astype(np.float64) @ k[b, :, h].astype(np.float64).T)
            s[np.triu_indices(n, 1)] = -np.inf
            np.testing.assert_allclose(r["lse"][b, :, h], logsumexp(s, axis=1), rtol=1e-12)
            np.testing.assert_allclose(r["o"][b, :, h], softmax(s, axis=1) @ v[b, :, h].astype(np.float64),
                                       rtol=1e-12, atol=1e-12)


def test_lone_root_returns_its_value():
    rng = np.random.default_rng(3)
    q, k, v, _, _ = _inputs(rng, 1, 1, 2, 1, 4, 1)
    r = oracle.tree_attention(q, k, v, np.zeros((1, 1, 2, 4), np.float32), np.full((1, 1, 2), -np.inf, np.float32),
                              np.array([[-1]], np.int32), np.array([1]), 0.25)
    for h in range(2):
        np.testing.assert_allclose(r["o"][0, 0, h], v[0, 0, 0], rtol=1e-15)
        assert abs(r["lse"][0, 0, h] - 0.25 * float(q[0, 0, h].astype(np.float64) @ k[0, 0, 0])) < 1e-12


def test_padding_nodes_are_not_read():
    rng = np.random.default_rng(4)
    batch, n, Hq, Hkv, D = 2, 10, 4, 2, 8
    q, k, v, _, _ = _inputs(rng, batch, n, Hq, Hkv, D, 1)
    par = np.stack([_random_tree(rng, n) for _ in range(batch)])
    op = rng.standard_normal((batch, n, Hq, D)).astype(np.float32)
    lp = rng.standard_normal((batch, n, Hq)).astype(np.float32)
    nn = np.array([6, 10])
    a = oracle.tree_attention(q, k, v, op, lp, par, nn, 0.3)
    k2, v2, q2 = k.copy(), v.copy(), q.copy()
    k2[0, 6:] = 1e3
    v2[0, 6:] = -1e3
    q2[0, 6:] = 7.0
    b = oracle.tree_attention(q2, k2, v2, op, lp, par, nn, 0.3)
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["lse"], b["lse"])
    assert np.all(a["o"][0, 6:] == 0) and np.all(a["lse"][0, 6:] == 0)
