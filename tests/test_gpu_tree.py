"""GPU parity of uno_build_tree and uno_verify_tree against the oracle."""
import dataclasses

import numpy as np
import pytest
import torch

import lossless_draft_verify_amd as uno
import oracle
from lossless_draft_verify_amd import synth
from gpu_util import Tally, device, np_of, say
from stats_util import chisq_pvalue

pytestmark = pytest.mark.gpu

TREE_KEYS = ("node_token", "node_parent", "node_depth", "num_nodes")


def _tree_paths(tok, par, num):
    """Token path (root to node) of every non-root node."""
    out = {}
    for n in range(1, int(num)):
        seq, q = [], n
        while q > 0:
            seq.append(int(tok[q]))
            q = int(par[q])
        out[n] = tuple(reversed(seq))
    return out


def _check_tied_tree(g, o, f, b, B, label):
    """A tree that differs from the oracle's is valid when only the order of
    scores equal in exact arithmetic differs: every node's score is the product
    of the filtered probabilities on its path, nodes come in best-first order,
    and the node sets differ only by entries tied with the last one kept."""
    num = int(o["num_nodes"][b])
    assert int(g["num_nodes"][b]) == num, (label, b)

    def path_score(path):
        s = 1.0
        for d, t in enumerate(path):
            ids = list(f["ids"][b * B + d])
            assert t in ids, (label, b, d, t)
            s *= f["probs"][b * B + d][ids.index(t)]
        return s

    gp = _tree_paths(g["node_token"][b], g["node_parent"][b], num)
    op = _tree_paths(o["node_token"][b], o["node_parent"][b], num)
    for n, path in gp.items():
        assert int(g["node_depth"][b][n]) == len(path), (label, b, n)
        s = path_score(path)
        assert abs(g["node_score"][b][n] - s) <= 1e-12 * s, (label, b, n)
    sc = g["node_score"][b][1:num]
    assert np.all(sc[1:] <= sc[:-1] * (1 + 1e-12)), (label, b)
    lowest = min(o["node_score"][b][1:num]) if num > 1 else 1.0
    for path in set(gp.values()) ^ set(op.values()):
        assert abs(path_score(path) - lowest) <= 1e-12 * lowest, (label, b, path)


def _build_parity(draft, K, V, T, k, p, label):
    g = uno.build_tree(draft, K, V, T, k, p)
    torch.cuda.synchronize()
    dh = synth.as_float32_numpy(draft)
    o = oracle.build_tree(dh, K, V, T, k, p)
    batch, B, N = dh.shape
    G = {key: np_of(g[key]) for key in TREE_KEYS + ("node_score",)}
    bad = np.zeros(batch, dtype=bool)
    for key in TREE_KEYS:
        bad |= np.any(G[key].reshape(batch, -1) != o[key].reshape(batch, -1), axis=1)
    full_vocab = T > 0 and (k <= 0 or k >= N) and N > uno.MAX_TOP_K
    if full_vocab:
        # full-softmax (or nucleus) normalisers are summed in another order on the
        # device, so scores equal in exact arithmetic may round apart and pop in
        # either order
        f = oracle.filter_rows(dh.reshape(batch * B, N), T, 0, p, cap=K, dense=False)
        for b in np.flatnonzero(bad):
            _check_tied_tree(G, o, f, int(b), B, label)
        same = ~bad
        np.testing.assert_allclose(G["node_score"][same], o["node_score"][same], rtol=1e-12, atol=0)
        return g, o
    # a pop order may only differ where two scores are within rounding of each other
    assert not np.any(bad & (o["min_gap"] >= 1e-12)), (label, np.flatnonzero(bad)[:4])
    # scores are products of filtered probabilities, each within an ulp or two of
    # the reference (the device and host exp may differ in the last bit)
    np.testing.assert_allclose(G["node_score"], o["node_score"], rtol=1e-12, atol=0)
    return g, o


def _verify_parity(target, B, tree, T, k, p, seed, offset, tally, label, request_ids=None):
    dev = target.device
    tk = torch.from_numpy(tree["node_token"]).to(dev)
    pa = torch.from_numpy(tree["node_parent"]).to(dev)
    nn = torch.from_numpy(tree["num_nodes"]).to(dev)
    g = uno.verify_tree(target, B, tk, pa, nn, T, k, p, seed, offset, request_ids=request_ids)
    torch.cuda.synchronize()
    rid = None if request_ids is None else np.asarray(request_ids, dtype=np.uint32)
    o = oracle.verify_tree(synth.as_float32_numpy(target), B, tree["node_token"], tree["node_parent"],
                           tree["num_nodes"], T, k, p, seed=seed, offset=offset, request_ids=rid)
    gg = {key: np_of(g[key]) for key in ("tokens", "path", "accept_len")}
    tally.compare(gg, o, ("tokens", "path", "accept_len"), label)
    return gg


def _tree_cycles(w, cycles, batch=None, label=None):
    dev = device()
    tally = Tally()
    acc = []
    for c in range(cycles):
        draft, R = synth.tree_inputs(w, cycle=c, device=dev, batch=batch)
        _, o = _build_parity(draft, w.K, w.V, w.temperature, w.top_k, w.top_p, f"{w.name} build {c}")
        # the walk checks against the oracle's own tree, so its inputs never come from the HIP path
        tgt = synth.tree_target_rows(R, torch.from_numpy(o["node_depth"]), torch.from_numpy(o["num_nodes"]), w.V)
        gg = _verify_parity(tgt, w.B, o, w.temperature, w.top_k, w.top_p, w.seed, c, tally,
                            f"{w.name} verify {c}")
        acc.append(gg["accept_len"])
    tally.check_rate()
    a = np.concatenate(acc)
    say(f"{label or w.name}: {tally.total} request-cycles, excused {tally.excused}, mean accept_len "
        f"{a.mean():.3f}, TPF {oracle.tpf(a):.3f}")


def test_tree_16_32_32_full_size():
    _tree_cycles(synth.WORKLOADS["tree_16_32_32"], 6)


def test_tree_8_16_8_reduced_batch():
    _tree_cycles(synth.WORKLOADS["tree_8_16_8"], 3, batch=8, label="tree_8_16_8 b8")


def test_tree_8_16_8_full_size():
    _tree_cycles(synth.WORKLOADS["tree_8_16_8"], 1, label="tree_8_16_8 b64")


@pytest.mark.parametrize("B,K,V,T,k,p", [(3, 3, 10, 1.0, 5, 1.0),
                                         (4, 1, 4, 1.0, 50, 0.95), (2, 8, 16, 0.5, 8, 1.0),
                                         (5, 16, 128, 1.0, 16, 1.0), (6, 4, 20, 0.0, 0, 1.0),
                                         (8, 256, 8, 1.0, 256, 1.0)])
def test_tree_shapes_small_vocab(B, K, V, T, k, p):
    dev = device()
    rng = np.random.default_rng(B * 100 + K)
    batch, N = 12, 301
    d = (rng.standard_normal((batch, B, N)) * 2).astype(np.float32)
    draft = torch.from_numpy(d).to(dev)
    _, o = _build_parity(draft, K, V, T, k, p, f"shape B{B} K{K} V{V}")
    tgt = torch.from_numpy((rng.standard_normal((batch, V + 1, N)) * 2).astype(np.float32)).to(dev)
    t = Tally()
    rid = np.arange(batch, dtype=np.uint32) * 7919
    for c in range(3):
        _verify_parity(tgt, B, o, T, k, p, 17, c, t, f"walk B{B} K{K} V{V}", request_ids=rid)
    t.check_rate()


def test_tree_ties_in_bf16():
    # coarse logits give exact probability ties between siblings and across depths
    dev = device()
    rng = np.random.default_rng(41)
    batch, B, N = 16, 4, 500
    d = np.round(rng.standard_normal((batch, B, N)) * 2) / 2
    draft = torch.from_numpy(d.astype(np.float32)).to(dev).to(torch.bfloat16)
    _build_parity(draft, 6, 24, 1.0, 10, 1.0, "bf16 ties")


def test_walk_is_lossless_small_vocab():
    dev = device()
    rng = np.random.default_rng(42)
    B, K, V, N, n = 3, 3, 7, 9, 100_000
    d = (rng.standard_normal((1, B, N)) * 1.2).astype(np.float32)
    tree = oracle.build_tree(d, K, V, 1.0, 0, 1.0)
    target_rows = (rng.standard_normal((V + 1, N)) * 1.2).astype(np.float32)
    tgt = torch.from_numpy(target_rows).to(dev).expand(n, V + 1, N).contiguous()
    rep = lambda a: torch.from_numpy(np.ascontiguousarray(np.tile(a, (n, 1)))).to(dev)
    g = uno.verify_tree(tgt, B, rep(tree["node_token"]), rep(tree["node_parent"]),
                        torch.full((n,), int(tree["num_nodes"][0]), dtype=torch.int32, device=dev),
                        1.0, 5, 1.0, 77, 0)
    torch.cuda.synchronize()
    P = oracle.filter_rows(target_rows, 1.0, 5, 1.0)["dense"]
    tok, path = np_of(g["tokens"]), np_of(g["path"])
    for node in range(int(tree["num_nodes"][0])):
        for dd in range(B + 1):
            sel = path[:, dd] == node
            if sel.sum() > 3000:
                assert chisq_pvalue(tok[sel, dd], P[node]) > 1e-4, (node, dd)


# ---- full-vocabulary filters (dense tree mode) ----------------------------------------

def test_dense_tree_16_32_32_full_size():
    _tree_cycles(synth.WORKLOADS["tree_dense_16_32_32"], 4)


def test_dense_tree_8_16_8_reduced_batch():
    _tree_cycles(synth.WORKLOADS["tree_dense_8_16_8"], 2, batch=8, label="tree_dense_8_16_8 b8")


@pytest.mark.parametrize("B,K,V,T,N,bf16", [(3, 3, 10, 1.0, 5000, False), (2, 8, 16, 0.5, 4099, True),
                                            (5, 16, 128, 1.0, 3 * 2048, False), (4, 256, 8, 1.0, 700, False),
                                            (6, 4, 20, 2.0, 257, True), (3, 4, 12, 1.0, 300007, True)])
def test_dense_tree_shapes(B, K, V, T, N, bf16):
    # several chunks and a ragged tail, K up to the top-k limit, V up to 128,
    # rows of more than 128 chunks
    dev = device()
    rng = np.random.default_rng(B * 1000 + K + N)
    batch = 10
    d = torch.from_numpy((rng.standard_normal((batch, B, N)) * 2).astype(np.float32)).to(dev)
    tg = torch.from_numpy((rng.standard_normal((batch, V + 1, N)) * 2).astype(np.float32)).to(dev)
    if bf16:
        d, tg = d.to(torch.bfloat16), tg.to(torch.bfloat16)
    label = f"dense B{B} K{K} V{V} N{N}"
    _, o = _build_parity(d, K, V, T, 0, 1.0, label)
    t = Tally()
    rid = np.arange(batch, dtype=np.uint32) * 7919 + 3
    for c in range(3):
        _verify_parity(tg, B, o, T, 0, 1.0, 23, c, t, label, request_ids=rid)
    t.check_rate()


def test_dense_walk_invalid_rows_and_unread_rows():
    # a live node row with no finite logit stops the walk with -1 (flagged);
    # rows at or past num_nodes hold +inf and must not be read
    dev = device()
    rng = np.random.default_rng(5)
    batch, B, K, V, N = 6, 3, 4, 12, 3000
    d = (rng.standard_normal((batch, B, N)) * 1.5).astype(np.float32)
    tree = oracle.build_tree(d, K, V, 1.0, 0, 1.0)
    tree["num_nodes"] = np.minimum(tree["num_nodes"], 7).astype(np.int32)
    tg = (rng.standard_normal((batch, V + 1, N)) * 1.5).astype(np.float32)
    tg[:, 7:, :] = np.inf
    tg[1, 0, :] = -np.inf                     # request 1: the root row is empty
    tg[2, :, :5] = np.nan                     # NaN logits count as -inf
    tg[3, 0, 100] = np.inf                    # request 3: the root row is invalid
    g = _verify_parity(torch.from_numpy(tg).to(dev), B, tree, 1.0, 0, 1.0, 9, 4, Tally(), "dense invalid")
    assert g["tokens"][1, 0] == -1 and g["accept_len"][1] == 1
    assert g["tokens"][3, 0] == -1 and g["accept_len"][3] == 1


def test_dense_walk_is_lossless():
    # vocabulary above the top-k limit, so the full-softmax path runs
    dev = device()
    rng = np.random.default_rng(43)
    B, K, V, N, n = 3, 3, 7, 300, 60_000
    # peaked rows, and node rows equal to the draft row of their depth, so that
    # walks often follow a child and reach the deeper nodes
    R = (rng.standard_normal((B + 1, N)) * 3.0).astype(np.float32)
    tree = oracle.build_tree(R[None, :B], K, V, 1.0, 0, 1.0)
    dep = np.maximum(tree["node_depth"][0], 0)
    target_rows = np.ascontiguousarray(R[dep])
    tgt = torch.from_numpy(target_rows).to(dev).expand(n, V + 1, N).contiguous()
    rep = lambda a: torch.from_numpy(np.ascontiguousarray(np.tile(a, (n, 1)))).to(dev)
    g = uno.verify_tree(tgt, B, rep(tree["node_token"]), rep(tree["node_parent"]),
                        torch.full((n,), int(tree["num_nodes"][0]), dtype=torch.int32, device=dev),
                        1.0, 0, 1.0, 78, 0)
    torch.cuda.synchronize()
    P = oracle.filter_rows(target_rows, 1.0, 0, 1.0)["dense"]
    tok, path = np_of(g["tokens"]), np_of(g["path"])
    checked = 0
    for node in range(int(tree["num_nodes"][0])):
        for dd in range(B + 1):
            sel = path[:, dd] == node
            if sel.sum() > 3000:
                assert chisq_pvalue(tok[sel, dd], P[node]) > 1e-4, (node, dd)
                checked += 1
    assert checked >= 2



def test_tree_joint_order():
    # tree 8/16/8 rows (reduced batch) with the joint filter order for build and walk
    dev = device()
    w = synth.WORKLOADS["tree_8_16_8"]
    t = Tally()
    for c in range(2):
        draft, R = synth.tree_inputs(w, cycle=c, device=dev, batch=8)
        g = uno.build_tree(draft, w.K, w.V, w.temperature, w.top_k, w.top_p, order=uno.ORDER_JOINT)
        torch.cuda.synchronize()
        o = oracle.build_tree(synth.as_float32_numpy(draft), w.K, w.V, w.temperature, w.top_k, w.top_p,
                              order=oracle.ORDER_JOINT)
        for key in TREE_KEYS:
            bad = np.any(np_of(g[key]).reshape(8, -1) != o[key].reshape(8, -1), axis=1)
            assert not np.any(bad & (o["min_gap"] >= 1e-12)), (key, c)
        tgt = synth.tree_target_rows(R, torch.from_numpy(o["node_depth"]), torch.from_numpy(o["num_nodes"]), w.V)
        dv = tgt.device
        gv = uno.verify_tree(tgt, w.B, torch.from_numpy(o["node_token"]).to(dv),
                             torch.from_numpy(o["node_parent"]).to(dv), torch.from_numpy(o["num_nodes"]).to(dv),
                             w.temperature, w.top_k, w.top_p, w.seed, c, order=uno.ORDER_JOINT)
        torch.cuda.synchronize()
        ov = oracle.verify_tree(synth.as_float32_numpy(tgt), w.B, o["node_token"], o["node_parent"],
                                o["num_nodes"], w.temperature, w.top_k, w.top_p, seed=w.seed, offset=c,
                                order=oracle.ORDER_JOINT)
        t.compare({k: np_of(gv[k]) for k in ("tokens", "path", "accept_len")}, ov,
                  ("tokens", "path", "accept_len"), f"tree joint {c}")
    t.check_rate()


@pytest.mark.parametrize("B,K,V,T,p,N,bf16", [(3, 3, 10, 1.0, 0.9, 5000, False), (2, 8, 16, 0.5, 0.5, 4099, True),
                                              (4, 64, 8, 1.0, 0.3, 700, False), (5, 16, 128, 1.0, 0.95, 3 * 2048, True)])
def test_dense_tree_nucleus_shapes(B, K, V, T, p, N, bf16):
    # top-k off, top-p on: candidates from each draft row's nucleus (fewer than K
    # when the nucleus is small), node tokens from each target row's nucleus
    dev = device()
    rng = np.random.default_rng(B * 7 + K + N)
    batch = 10
    d = torch.from_numpy((rng.standard_normal((batch, B, N)) * 2.5).astype(np.float32)).to(dev)
    tg = torch.from_numpy((rng.standard_normal((batch, V + 1, N)) * 2.5).astype(np.float32)).to(dev)
    if bf16:
        d, tg = d.to(torch.bfloat16), tg.to(torch.bfloat16)
    label = f"nucleus tree B{B} K{K} V{V} p{p} N{N}"
    _, o = _build_parity(d, K, V, T, 0, p, label)
    t = Tally()
    rid = np.arange(batch, dtype=np.uint32) * 31 + 5
    for c in range(3):
        _verify_parity(tg, B, o, T, 0, p, 29, c, t, label, request_ids=rid)
    t.check_rate()


def test_dense_tree_16_32_32_nucleus_full_size():
    w = dataclasses.replace(synth.WORKLOADS["tree_dense_16_32_32"], top_p=0.95, name="tree 16/32/32 nucleus")
    _tree_cycles(w, 3)
