"""GPU parity of per-request sampling parameters (the *_ex entry points):
greedy and stochastic requests with their own temperature, top-k, top-p and
filter order in one call, each checked against the oracle run with its own set."""
import numpy as np
import pytest
import torch

import lossless_draft_verify_amd as uno
import oracle
from lossless_draft_verify_amd import synth
from gpu_util import Tally, device, np_of, say

pytestmark = pytest.mark.gpu

# (temperature, top_k, top_p, order): greedy, the pages' 50 / 0.95, no top-p, a
# large k, a tiny k, the joint order (all joint sets at temperature 1)
SETS = [(0.0, 0, 1.0, 0), (1.0, 50, 0.95, 0), (0.7, 20, 1.0, 0), (1.3, 256, 0.9, 0), (1.0, 3, 0.5, 0),
        (1.0, 50, 0.9, 1), (0.5, 8, 0.8, 0), (1.0, 100, 0.99, 1)]


def _params(n):
    s = [SETS[i % len(SETS)] for i in range(n)]
    return [np.array([x[j] for x in s]) for j in range(4)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows,N", [(64, 3001), (24, 151936), (300, 1003)])
def test_filter_per_row_parameters(dtype, rows, N):
    # 3001 logits: one workgroup per row; 151936: rows split into segments whose
    # lists (sized for the largest k) the merge reads with each row's own k;
    # 300 rows: more sets than the kernel arguments carry (the staged copy)
    dev = device()
    rng = np.random.default_rng(50)
    z = torch.from_numpy((rng.standard_normal((rows, N)) * 2).astype(np.float32)).to(dev).to(dtype)
    T, K, P, O = _params(rows)
    g = uno.filter_rows(z, T, K, P, order=O)
    torch.cuda.synchronize()
    zh = z.float().cpu().numpy()
    gn, gi, gp = np_of(g["count"]), np_of(g["ids"]), np_of(g["probs"])
    for r in range(rows):
        o = oracle.filter_rows(zh[r:r + 1], T[r], K[r], P[r], cap=gi.shape[1], dense=False, order=int(O[r]))
        if o["margin"][0] < 1e-9:
            continue
        n = int(o["n"][0])
        assert gn[r] == n, (r, gn[r], n)
        assert np.array_equal(gi[r, :n], o["ids"][0, :n]), r
        np.testing.assert_allclose(gp[r, :n], o["probs"][0, :n], rtol=1e-12, atol=0)


def test_linear_per_request_parameters():
    dev = device()
    w = synth.WORKLOADS["linear_8_1_8"]
    batch = 16
    T, K, P, O = _params(batch)
    t = Tally()
    for c in range(2):
        draft, target = synth.linear_inputs(w, cycle=c, device=dev, batch=batch)
        g = uno.sample_linear(draft, target, T, K, P, w.seed, c, order=O)
        torch.cuda.synchronize()
        d, tg = synth.as_float32_numpy(draft), synth.as_float32_numpy(target)
        gg = {k: np_of(g[k]) for k in ("tokens", "accept_len", "proposals")}
        for b in range(batch):
            o = oracle.linear(d[b:b + 1], tg[b:b + 1], T[b], K[b], P[b], w.seed, c,
                              request_ids=np.array([b], np.uint32), order=int(O[b]))
            t.compare({k: v[b:b + 1] for k, v in gg.items()}, o, ("tokens", "accept_len", "proposals"),
                      f"per-request linear cycle {c} request {b}")
    t.check_rate()
    say(f"per-request linear: {t.total} request-cycles, excused {t.excused}")


def test_tree_per_request_parameters():
    dev = device()
    w = synth.WORKLOADS["tree_8_16_8"]
    batch = 8
    T, K, P, O = _params(batch)
    draft, R = synth.tree_inputs(w, cycle=0, device=dev, batch=batch)
    g = uno.build_tree(draft, w.K, w.V, T, K, P, order=O)
    torch.cuda.synchronize()
    d = synth.as_float32_numpy(draft)
    trees = [oracle.build_tree(d[b:b + 1], w.K, w.V, T[b], K[b], P[b], order=int(O[b])) for b in range(batch)]
    for b, o in enumerate(trees):
        for key in ("node_token", "node_parent", "node_depth", "num_nodes"):
            same = np.array_equal(np_of(g[key])[b], o[key][0])
            assert same or o["min_gap"][0] < 1e-12, (b, key)
    node_depth = torch.from_numpy(np.stack([o["node_depth"][0] for o in trees]))
    num_nodes = torch.from_numpy(np.array([o["num_nodes"][0] for o in trees], np.int32))
    tgt = synth.tree_target_rows(R, node_depth, num_nodes, w.V)
    tk = torch.from_numpy(np.stack([o["node_token"][0] for o in trees])).to(dev)
    pa = torch.from_numpy(np.stack([o["node_parent"][0] for o in trees])).to(dev)
    gv = uno.verify_tree(tgt, w.B, tk, pa, num_nodes.to(dev), T, K, P, w.seed, 3, order=O)
    torch.cuda.synchronize()
    th = synth.as_float32_numpy(tgt)
    t = Tally()
    for b in range(batch):
        o = oracle.verify_tree(th[b:b + 1], w.B, np_of(tk)[b:b + 1], np_of(pa)[b:b + 1], np_of(num_nodes)[b:b + 1],
                               T[b], K[b], P[b], w.seed, 3, request_ids=np.array([b], np.uint32), order=int(O[b]))
        t.compare({k: np_of(gv[k])[b:b + 1] for k in ("tokens", "path", "accept_len")}, o,
                  ("tokens", "path", "accept_len"), f"per-request walk {b}")
    t.check_rate()


def test_linear_8_1_8_mixed_full_size():
    # the bench's mixed workload: the headline shape (64 requests, 151936 fp32
    # logits) with one parameter set per request, every request checked
    dev = device()
    w = synth.WORKLOADS["linear_8_1_8_mixed"]
    sets = [w.request_params(b) for b in range(w.batch)]
    T, K, P, O = (np.array([s[j] for s in sets]) for j in range(4))
    draft, target = synth.linear_inputs(w, cycle=0, device=dev)
    g = uno.sample_linear(draft, target, T, K, P, w.seed, 0, order=O)
    torch.cuda.synchronize()
    d, tg = synth.as_float32_numpy(draft), synth.as_float32_numpy(target)
    gg = {k: np_of(g[k]) for k in ("tokens", "accept_len", "proposals")}
    t = Tally()
    for b in range(w.batch):
        o = oracle.linear(d[b:b + 1], tg[b:b + 1], T[b], K[b], P[b], w.seed, 0,
                          request_ids=np.array([b], np.uint32), order=int(O[b]))
        t.compare({k: v[b:b + 1] for k, v in gg.items()}, o, ("tokens", "accept_len", "proposals"),
                  f"mixed linear_8_1_8 request {b}")
    t.check_rate()
    say(f"linear_8_1_8_mixed: {t.total} requests, excused {t.excused}, mean accept_len {gg['accept_len'].mean():.3f}")


# ---- sets that mix the top-k path with full-vocabulary rows ----------------------------
# greedy, top-k 50 / top-p 0.95, the full softmax at two temperatures, a nucleus
# without top-k, joint-order sets at two temperatures and a large k
FULL_SETS = [(0.0, 0, 1.0, 0), (1.0, 50, 0.95, 0), (1.0, 0, 1.0, 0), (0.8, 0, 0.9, 0), (1.0, 50, 0.9, 1),
             (0.7, 100, 0.9, 1), (1.3, 256, 0.9, 0), (0.6, 0, 1.0, 0)]


def _full_params(n):
    s = [FULL_SETS[i % len(FULL_SETS)] for i in range(n)]
    return [np.array([x[j] for x in s]) for j in range(4)]


def _oracle_linear_by_set(d, tg, T, K, P, O, seed, offset):
    """The oracle over each set's requests at once (their own request ids)."""
    batch = d.shape[0]
    out = {k: np.zeros((batch,) + shp, dt) for k, shp, dt in
           (("tokens", (d.shape[1] + 1,), np.int32), ("accept_len", (), np.int32), ("proposals", (d.shape[1],), np.int32),
            ("margin", (), np.float64))}
    keys = sorted(set(zip(T.tolist(), K.tolist(), P.tolist(), O.tolist())))
    for key in keys:
        sel = np.flatnonzero((T == key[0]) & (K == key[1]) & (P == key[2]) & (O == key[3]))
        o = oracle.linear(d[sel], tg[sel], key[0], int(key[1]), key[2], seed, offset,
                          request_ids=sel.astype(np.uint32), order=int(key[3]))
        for k in out:
            out[k][sel] = o[k]
    return out


def test_linear_8_1_8_full_vocab_mixed_full_size():
    # the headline shape (64 requests, 151936 fp32 logits) with greedy, top-k,
    # full-softmax and nucleus requests and joint sets at two temperatures in
    # one call; every request checked against the oracle run with its own set
    dev = device()
    w = synth.WORKLOADS["linear_8_1_8"]
    T, K, P, O = _full_params(w.batch)
    t = Tally("mixed full-vocabulary linear_8_1_8")
    for c in range(2):
        draft, target = synth.linear_inputs(w, cycle=c, device=dev)
        g = uno.sample_linear(draft, target, T, K, P, w.seed, c, order=O)
        gg = {k: np_of(g[k]) for k in ("tokens", "accept_len", "proposals")}
        o = _oracle_linear_by_set(synth.as_float32_numpy(draft), synth.as_float32_numpy(target), T, K, P, O, w.seed, c)
        t.compare(gg, o, ("tokens", "accept_len", "proposals"), f"mixed linear_8_1_8 cycle {c}")
    t.check_rate()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_linear_full_vocab_mixed_small_vocab(dtype):
    # several chunks and a ragged tail per row, B = 5, ids of every request
    dev = device()
    rng = np.random.default_rng(51)
    batch, B, N = 40, 5, 5003
    R = (rng.standard_normal((batch, B + 1, N)) * 2).astype(np.float32)
    d = (R[:, :B] + 0.5 * rng.standard_normal((batch, B, N))).astype(np.float32)
    draft = torch.from_numpy(d).to(dev).to(dtype).contiguous()
    target = torch.from_numpy(R).to(dev).to(dtype).contiguous()
    T, K, P, O = _full_params(batch)
    t = Tally(f"mixed full-vocabulary small vocab {dtype}")
    for c in range(3):
        g = uno.sample_linear(draft, target, T, K, P, 19, c, order=O)
        gg = {k: np_of(g[k]) for k in ("tokens", "accept_len", "proposals")}
        o = _oracle_linear_by_set(synth.as_float32_numpy(draft), synth.as_float32_numpy(target), T, K, P, O, 19, c)
        t.compare(gg, o, ("tokens", "accept_len", "proposals"), f"mixed small vocab cycle {c}")
    t.check_rate()


@pytest.mark.parametrize("rows,N", [(64, 5003), (24, 151936)])
def test_filter_full_vocab_mixed_rows(rows, N):
    # per-row sets over both paths: top-k rows report their support, full-softmax
    # rows their number of finite logits, nucleus rows their nucleus size, every
    # row its (m, S) statistics
    dev = device()
    rng = np.random.default_rng(52)
    z = torch.from_numpy((rng.standard_normal((rows, N)) * 2).astype(np.float32)).to(dev)
    T, K, P, O = _full_params(rows)
    g = uno.filter_rows(z, T, K, P, order=O)
    zh = z.cpu().numpy()
    gn, gs = np_of(g["count"]), np_of(g["stats"])
    gi, gp = np_of(g["ids"]), np_of(g["probs"])
    for r in range(rows):
        o = oracle.filter_rows(zh[r:r + 1], T[r], K[r], P[r], cap=gi.shape[1], dense=False, order=int(O[r]))
        full = T[r] > 0 and (K[r] <= 0 or K[r] >= N)
        if full:
            assert np.all(gi[r] == -1) and np.all(gp[r] == 0.0), r
            assert gs[r, 0] == o["stats"][0, 0], r
            assert abs(gs[r, 1] - o["stats"][0, 1]) <= 2 * N * 2.0**-53 * o["stats"][0, 1], r
            if P[r] >= 1.0:
                assert gn[r] == N, r
            elif o["margin"][0] >= 1e-9:
                assert gn[r] == o["n"][0], (r, gn[r], o["n"][0])
            continue
        if o["margin"][0] < 1e-9:
            continue
        n = int(o["n"][0])
        assert gn[r] == n, (r, gn[r], n)
        assert np.array_equal(gi[r, :n], o["ids"][0, :n]), r
        np.testing.assert_allclose(gp[r, :n], o["probs"][0, :n], rtol=1e-12, atol=0)


def test_tree_full_vocab_mixed():
    # tree 8/16/8 rows (bf16, batch 16) with the mixed sets: top-k requests
    # build from their filtered rows, full-vocabulary requests from the K most
    # likely ids of the full softmax or the nucleus; the walk samples each
    # request's node rows on its own path
    from test_gpu_tree import _check_tied_tree
    dev = device()
    w = synth.WORKLOADS["tree_8_16_8"]
    batch = 16
    T, K, P, O = _full_params(batch)
    draft, R = synth.tree_inputs(w, cycle=0, device=dev, batch=batch)
    g = uno.build_tree(draft, w.K, w.V, T, K, P, order=O)
    d = synth.as_float32_numpy(draft)
    G = {key: np_of(g[key]) for key in ("node_token", "node_parent", "node_depth", "num_nodes", "node_score")}
    trees = []
    for b in range(batch):
        o = oracle.build_tree(d[b:b + 1], w.K, w.V, T[b], K[b], P[b], order=int(O[b]))
        trees.append(o)
        same = all(np.array_equal(G[key][b].ravel(), o[key][0].ravel())
                   for key in ("node_token", "node_parent", "node_depth", "num_nodes"))
        full = T[b] > 0 and K[b] <= 0
        if full and not same:
            f = oracle.filter_rows(d[b], T[b], 0, P[b], cap=w.K, dense=False)
            sub = {key: G[key][b:b + 1] for key in G}
            _check_tied_tree(sub, o, f, 0, w.B, f"mixed tree request {b}")
        else:
            assert same or o["min_gap"][0] < 1e-12, b
            if same:
                np.testing.assert_allclose(G["node_score"][b], o["node_score"][0], rtol=1e-12, atol=0)
    node_depth = torch.from_numpy(np.stack([o["node_depth"][0] for o in trees]))
    num_nodes = torch.from_numpy(np.array([o["num_nodes"][0] for o in trees], np.int32))
    tgt = synth.tree_target_rows(R, node_depth, num_nodes, w.V)
    tk = torch.from_numpy(np.stack([o["node_token"][0] for o in trees])).to(dev)
    pa = torch.from_numpy(np.stack([o["node_parent"][0] for o in trees])).to(dev)
    t = Tally("mixed full-vocabulary walk")
    th = synth.as_float32_numpy(tgt)
    for c in range(3):
        gv = uno.verify_tree(tgt, w.B, tk, pa, num_nodes.to(dev), T, K, P, w.seed, c, order=O)
        for b in range(batch):
            o = oracle.verify_tree(th[b:b + 1], w.B, np_of(tk)[b:b + 1], np_of(pa)[b:b + 1],
                                   np_of(num_nodes)[b:b + 1], T[b], K[b], P[b], w.seed, c,
                                   request_ids=np.array([b], np.uint32), order=int(O[b]))
            t.compare({k: np_of(gv[k])[b:b + 1] for k in ("tokens", "path", "accept_len")}, o,
                      ("tokens", "path", "accept_len"), f"mixed walk cycle {c} request {b}")
    t.check_rate()
