"""Pins for the oracle's tree construction and target-sampled tree walk."""
import itertools

import numpy as np

import oracle
from stats_util import chisq_pvalue, mean_zscore

P_MIN = 1e-4


def _prefixes_of(res, b=0):
    """Token prefix of every non-root node, in node order."""
    tok, par = res["node_token"][b], res["node_parent"][b]
    out = []
    for n in range(1, int(res["num_nodes"][b])):
        seq, m = [], n
        while m > 0:
            seq.append(int(tok[m]))
            m = int(par[m])
        out.append(tuple(reversed(seq)))
    return out


def test_build_matches_brute_force_enumeration():
    rng = np.random.default_rng(21)
    B, K, N = 3, 3, 12
    for trial in range(8):
        draft = (rng.normal(size=(1, B, N)) * 1.5).astype(np.float32)
        T, k, p = 1.0, 6, 1.0
        f = oracle.filter_rows(draft[0], T, k, p, cap=N)
        cands = []
        for d in range(B):
            n = int(f["n"][d])
            cands.append([(int(f["ids"][d, r]), float(f["probs"][d, r])) for r in range(min(K, n))])
        # every prefix of length 1..B over the per-depth candidates, scored by the
        # product of its draft probabilities (root to leaf)
        allp = []
        for L in range(1, B + 1):
            for combo in itertools.product(*[range(len(cands[d])) for d in range(L)]):
                s = 1.0
                for d, r in enumerate(combo):
                    s = s * cands[d][r][1]
                allp.append((s, tuple(cands[d][r][0] for d, r in enumerate(combo))))
        allp.sort(key=lambda t: -t[0])
        for V in (1, 2, 5, 9, 17, 39):
            res = oracle.build_tree(draft, K, V, T, k, p)
            got = _prefixes_of(res)
            assert len(got) == min(V, len(allp))
            assert got == [t[1] for t in allp[:len(got)]], (trial, V)
            np.testing.assert_array_equal(res["node_score"][0, 1:len(got) + 1],
                                          [t[0] for t in allp[:len(got)]])
            # structural fields
            dep = res["node_depth"][0]
            par = res["node_parent"][0]
            assert dep[0] == 0 and par[0] == -1
            for n in range(1, len(got) + 1):
                assert dep[n] == dep[par[n]] + 1 and par[n] < n


def test_k1_tree_is_the_argmax_chain():
    rng = np.random.default_rng(22)
    B, N = 6, 50
    draft = rng.normal(size=(2, B, N)).astype(np.float32)
    res = oracle.build_tree(draft, 1, B, 1.0, 0, 1.0)
    for b in range(2):
        assert res["num_nodes"][b] == B + 1
        assert list(res["node_token"][b, 1:]) == list(np.argmax(draft[b], axis=1))
        assert list(res["node_parent"][b, 1:]) == list(range(B))
        assert list(res["node_depth"][b]) == list(range(B + 1))


def test_small_supports_give_a_smaller_tree():
    # greedy rows have one candidate per depth: the tree is the chain of B nodes
    rng = np.random.default_rng(23)
    B, N = 4, 30
    draft = rng.normal(size=(1, B, N)).astype(np.float32)
    res = oracle.build_tree(draft, 8, 20, 0.0, 0, 1.0)
    assert res["num_nodes"][0] == B + 1
    assert np.all(res["node_score"][0, : B + 1] == 1.0)
    assert np.all(res["node_token"][0, B + 1:] == -1)


def test_tie_rule_depth_then_parent_then_rank():
    # two equal top logits per depth, top-k 2 -> every candidate has q = 1/2
    B, N = 3, 10
    draft = np.full((1, B, N), -30.0, dtype=np.float32)
    draft[0, :, 2] = 5.0
    draft[0, :, 7] = 5.0
    res = oracle.build_tree(draft, 2, 6, 1.0, 2, 1.0)
    # depth-1 nodes (score 1/2) first, ranked by candidate rank (id 2 before id 7);
    # then depth 2 (score 1/4): parent 1's children before parent 2's
    assert _prefixes_of(res) == [(2,), (7,), (2, 2), (2, 7), (7, 2), (7, 7)]
    assert list(res["node_parent"][0, 1:7]) == [0, 0, 1, 1, 2, 2]


def _walk_expected_len(tree_tok, tree_par, nn, P):
    """1 + sum over non-root nodes of the probability that the walk reaches them."""
    reach = np.zeros(nn)
    reach[0] = 1.0
    for n in range(1, nn):
        a = tree_par[n]
        reach[n] = reach[a] * P[a][tree_tok[n]]
    return reach.sum()


def test_walk_is_lossless_and_matches_closed_form_length():
    rng = np.random.default_rng(24)
    B, K, V, N, n = 3, 3, 7, 9, 150_000
    draft = (rng.normal(size=(1, B, N)) * 1.2).astype(np.float32)
    tree = oracle.build_tree(draft, K, V, 1.0, 0, 1.0)
    nn = int(tree["num_nodes"][0])
    target = (rng.normal(size=(V + 1, N)) * 1.2).astype(np.float32)
    for (T, k, p) in [(1.0, 0, 1.0), (0.7, 4, 0.9)]:
        out = oracle.verify_tree(target, B, tree["node_token"][0], tree["node_parent"][0],
                                 tree["num_nodes"][0], T, k, p, seed=31, offset=2,
                                 request_ids=np.arange(n, dtype=np.uint32), batch=n)
        P = oracle.filter_rows(target, T, k, p)["dense"]
        tok, path, acc = out["tokens"], out["path"], out["accept_len"]
        assert np.all(path[:, 0] == 0)
        # the first token follows the root's filtered target row
        assert chisq_pvalue(tok[:, 0], P[0]) > P_MIN
        # at any visited node the emitted token follows that node's row
        for node in range(nn):
            for d in range(B + 1):
                sel = path[:, d] == node
                if sel.sum() > 3000:
                    assert chisq_pvalue(tok[sel, d], P[node]) > P_MIN, (node, d)
        E = _walk_expected_len(tree["node_token"][0], tree["node_parent"][0], nn, P)
        assert abs(mean_zscore(acc, E)) < 4.0
        # the walk only follows tree edges whose token it emitted
        for b in range(200):
            for d in range(1, acc[b]):
                c = path[b, d]
                assert tree["node_parent"][0][c] == path[b, d - 1]
                assert tree["node_token"][0][c] == tok[b, d - 1]


def test_one_hot_target_on_a_child_is_always_followed():
    B, N = 3, 12
    draft = np.full((1, B, N), -10.0, dtype=np.float32)
    for d in range(B):
        draft[0, d, d] = 3.0
        draft[0, d, d + 5] = 2.0
    tree = oracle.build_tree(draft, 2, 5, 1.0, 2, 1.0)
    nn = int(tree["num_nodes"][0])
    # greedy target: each node's target argmax is its first-rank child (or id 11 at leaves)
    target = np.full((5 + 1, N), 0.0, dtype=np.float32)
    for n in range(nn):
        kids = [c for c in range(1, nn) if tree["node_parent"][0][c] == n]
        target[n, tree["node_token"][0][kids[0]] if kids else 11] = 9.0
    out = oracle.verify_tree(target, B, tree["node_token"][0], tree["node_parent"][0],
                             tree["num_nodes"][0], 0.0, 0, 1.0, seed=1, offset=0,
                             request_ids=np.arange(50, dtype=np.uint32), batch=50)
    # follow rank-0 children until a node without children
    n, expect = 0, []
    while True:
        kids = [c for c in range(1, nn) if tree["node_parent"][0][c] == n]
        if not kids:
            expect.append(11)
            break
        expect.append(int(tree["node_token"][0][kids[0]]))
        n = kids[0]
    assert np.all(out["accept_len"] == len(expect))
    for b in range(50):
        assert list(out["tokens"][b, :len(expect)]) == expect


def test_tie_rule_prefers_the_shallower_node():
    # depth 1: ids 2 and 7 with q = 1/2 each; depth 2: id 4 with q = 1 (the other
    # top-2 id has probability ~1e-57).  Child (2, 4) then ties its parent's
    # sibling (7,) at score 1/2 and must come after it.
    B, N = 2, 10
    draft = np.full((1, B, N), -30.0, dtype=np.float32)
    draft[0, 0, 2] = draft[0, 0, 7] = 5.0
    draft[0, 1, 4] = 100.0
    res = oracle.build_tree(draft, 2, 4, 1.0, 2, 1.0)
    assert _prefixes_of(res) == [(2,), (7,), (2, 4), (7, 4)]
    np.testing.assert_array_equal(res["node_score"][0, 1:5], [0.5, 0.5, 0.5, 0.5])
