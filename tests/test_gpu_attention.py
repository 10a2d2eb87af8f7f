"""GPU parity of uno_tree_attention (tree-suffix attention merged with the prefix
state) against the oracle, on the tree verification shapes of the workloads."""
import numpy as np
import pytest
import torch

import lossless_draft_verify_amd as uno
import oracle
from gpu_util import device, np_of, say

pytestmark = pytest.mark.gpu

# Bounds: the output is rounded to bf16 (half an ulp, 2^-9 relative) after fp32
# scores, softmax and sums (relative errors near 1e-6 of the terms, which may
# cancel); the log-sum-exp stays fp32.
O_RTOL = 2.0**-8
O_ATOL = 2e-3
LSE_ATOL = 1e-4


def _tree(rng, n):
    par = np.full(n, -1, dtype=np.int32)
    for i in range(1, n):
        par[i] = rng.integers(max(0, i - 8), i)        # deep and wide trees
    return par


def _case(batch, n, Hq, Hkv, seed, num_nodes=None, empty_prefix_rows=0):
    dev = device()
    rng = np.random.default_rng(seed)
    D = 128
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(dev).to(torch.bfloat16).contiguous()
    q = bf(rng.standard_normal((batch, n, Hq, D)))
    k = bf(rng.standard_normal((batch, n, Hkv, D)))
    v = bf(rng.standard_normal((batch, n, Hkv, D)))
    op = bf(rng.standard_normal((batch, n, Hq, D)))
    lp = (rng.standard_normal((batch, n, Hq)) * 3).astype(np.float32)
    if empty_prefix_rows:
        lp[:empty_prefix_rows] = -np.inf
    par = np.stack([_tree(rng, n) for _ in range(batch)])
    nn = np.full(batch, n, dtype=np.int32) if num_nodes is None else np.asarray(num_nodes, dtype=np.int32)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    out = dict(o=torch.full_like(q, 7.0), lse=torch.full((batch, n, Hq), 7.0, dtype=torch.float32, device=dev))
    g = uno.tree_attention(q, k, v, op, torch.from_numpy(lp).to(dev), torch.from_numpy(par).to(dev),
                           torch.from_numpy(nn).to(dev), scale, out=out)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy()
    o = oracle.tree_attention(f(q), f(k), f(v), f(op), lp, par, nn, scale)
    go, gl = np_of(g["o"].float()), np_of(g["lse"])
    worst = 0.0
    for b in range(batch):
        m = int(nn[b])
        ref = o["o"][b, :m]
        err = np.abs(go[b, :m] - ref)
        assert np.all(err <= O_RTOL * np.abs(ref) + O_ATOL), (b, float(err.max()))
        assert np.all(np.abs(gl[b, :m] - o["lse"][b, :m]) <= LSE_ATOL * (1 + np.abs(o["lse"][b, :m]))), b
        # tokens past num_nodes are neither read nor written
        assert np.all(go[b, m:] == 7.0) and np.all(gl[b, m:] == 7.0), b
        worst = max(worst, float((err / (np.abs(ref) + 1e-3)).max()) if m else 0.0)
    say(f"tree attention b{batch} n{n} Hq{Hq} Hkv{Hkv}: worst relative error {worst:.2e}")


def test_tree_8_16_8_shape():
    _case(64, 9, 32, 8, 1)                 # tree 8/16/8: 64 requests, V + 1 = 9 verify tokens


def test_tree_16_32_32_shape():
    _case(1, 33, 32, 8, 2)                 # tree 16/32/32: one request, 33 verify tokens


def test_largest_tree_and_partial_requests():
    _case(3, 129, 8, 2, 3, num_nodes=[129, 70, 1])


def test_multi_head_and_empty_prefix():
    _case(5, 20, 4, 4, 4, num_nodes=[20, 0, 7, 20, 13], empty_prefix_rows=2)


def test_chain_tree_is_causal():
    # a chain (parent = i - 1) with no prefix is causal self-attention
    dev = device()
    rng = np.random.default_rng(5)
    batch, n, H, D = 2, 17, 4, 128
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(dev).to(torch.bfloat16).contiguous()
    q, k, v = (bf(rng.standard_normal((batch, n, H, D))) for _ in range(3))
    par = torch.from_numpy(np.tile(np.arange(-1, n - 1, dtype=np.int32), (batch, 1))).to(dev)
    lp = torch.full((batch, n, H), -float("inf"), dtype=torch.float32, device=dev)
    g = uno.tree_attention(q, k, v, torch.zeros_like(q), lp, par, None, 0.125)
    torch.cuda.synchronize()
    qf, kf, vf = (t.double().cpu() for t in (q, k, v))
    s = torch.einsum("bihd,bjhd->bhij", qf, kf) * 0.125
    s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), -float("inf"))
    ref = torch.einsum("bhij,bjhd->bihd", torch.softmax(s, -1), vf).numpy()
    got = np_of(g["o"].float())
    assert np.all(np.abs(got - ref) <= O_RTOL * np.abs(ref) + O_ATOL)
