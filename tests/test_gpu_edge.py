"""GPU edge cases: Philox high words, nucleus cuts inside long runs of ties, and a
call on a side stream."""
import numpy as np
import pytest
import torch

import lossless_draft_verify_amd as uno
import oracle
from gpu_util import Tally, device, np_of, say

pytestmark = pytest.mark.gpu

SEED_HI = 0x1_3579_BDF1          # seed >= 2^32: the key's high word is 1
OFFSET_HI = 0x3_0000_0007        # cycle index >= 2^32: the counter's fourth word is 3


def _rows(rng, shape, scale=2.0):
    return (rng.standard_normal(shape) * scale).astype(np.float32)


@pytest.mark.parametrize("T,k,p", [(1.0, 50, 0.9), (0.8, 0, 1.0), (1.0, 0, 0.9)])
def test_linear_high_seed_and_offset_words(T, k, p):
    # sparse, dense and nucleus samplers; request ids with the top bit set
    dev = device()
    rng = np.random.default_rng(61)
    batch, B, N = 32, 4, 3001
    R = _rows(rng, (batch, B + 1, N))
    d = (R[:, :B] + 0.6 * rng.standard_normal((batch, B, N))).astype(np.float32)
    rid = (np.arange(batch, dtype=np.uint64) * 2654435761 + 2**31).astype(np.uint32)
    g = uno.sample_linear(torch.from_numpy(d).to(dev), torch.from_numpy(R).to(dev), T, k, p, SEED_HI, OFFSET_HI,
                          request_ids=rid)
    gg = {key: np_of(g[key]) for key in ("tokens", "accept_len", "proposals")}
    o = oracle.linear(d, R, T, k, p, SEED_HI, OFFSET_HI, request_ids=rid)
    t = Tally(f"high words linear T{T} k{k} p{p}")
    t.compare(gg, o, ("tokens", "accept_len", "proposals"), "high words")
    t.check_rate()
    # the high words matter: dropping either changes most proposals
    for s, off in ((SEED_HI & 0xFFFFFFFF, OFFSET_HI), (SEED_HI, OFFSET_HI & 0xFFFFFFFF)):
        lo = oracle.linear(d, R, T, k, p, s, off, request_ids=rid)
        assert np.mean(lo["proposals"] != o["proposals"]) > 0.3


@pytest.mark.parametrize("k", [50, 0])
def test_walk_high_seed_and_offset_words(k):
    dev = device()
    rng = np.random.default_rng(62)
    batch, B, K, V, N = 16, 4, 4, 12, 3001
    d = _rows(rng, (batch, B, N), 2.5)
    tree = oracle.build_tree(d, K, V, 1.0, k, 1.0)
    tg = _rows(rng, (batch, V + 1, N), 2.5)
    rid = (np.arange(batch, dtype=np.uint64) * 40503 + 2**31 + 7).astype(np.uint32)
    gv = uno.verify_tree(torch.from_numpy(tg).to(dev), B, torch.from_numpy(tree["node_token"]).to(dev),
                         torch.from_numpy(tree["node_parent"]).to(dev), torch.from_numpy(tree["num_nodes"]).to(dev),
                         1.0, k, 1.0, SEED_HI, OFFSET_HI, request_ids=rid)
    o = oracle.verify_tree(tg, B, tree["node_token"], tree["node_parent"], tree["num_nodes"], 1.0, k, 1.0,
                           SEED_HI, OFFSET_HI, request_ids=rid)
    t = Tally(f"high words walk k{k}")
    t.compare({key: np_of(gv[key]) for key in ("tokens", "path", "accept_len")}, o, ("tokens", "path", "accept_len"),
              "high words walk")
    t.check_rate()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_nucleus_cut_inside_a_single_key_run(dtype):
    # Rows whose nucleus ends inside one run of equal logits, so the value bin
    # holding the cut is a single key:
    #   0: ids 2048..4095 hold 1e9, the rest 0 (every other term underflows):
    #      2048 ties of 1/2048, top-p 0.9 keeps 1844;
    #   1: 3001 ties of 5.0 in ids 0..3000 of coarse values at T 1e-4 (only the
    #      ties survive the temperature), top-p 0.5 keeps 1501;
    #   2: the same run spread over the whole row (every 50th id).
    # Each wave's chunks hold far more than the one-pass list has room for.
    dev = device()
    rng = np.random.default_rng(63)
    N = 151936
    z0 = np.zeros(N, np.float32)
    z0[2048:4096] = 1e9
    z1 = np.round(rng.standard_normal(N) * 2) / 2
    z1 = np.minimum(z1, 4.5).astype(np.float32)
    z2 = z1.copy()
    z1[:3001] = 5.0
    z2[::50][:3001] = 5.0
    cases = [(z0[None], 1.0, 0.9, [1844]), (np.stack([z1, z2]), 1e-4, 0.5, [1501, 1501])]
    for z, T, p, want in cases:
        zt = torch.from_numpy(z).to(dev).to(dtype).contiguous()
        zh = zt.float().cpu().numpy()
        o = oracle.filter_rows(zh, T, 0, p, cap=1, dense=False)
        assert o["n"].tolist() == want, o["n"]
        assert np.all(o["margin"] > 1e-5)
        g = uno.filter_rows(zt, T, 0, p)
        gc, gs = np_of(g["count"]), np_of(g["stats"])
        assert gc.tolist() == want, (dtype, T, p, gc)
        assert np.array_equal(gs[:, 0], o["stats"][:, 0])
        say(f"nucleus single-key run {dtype} T{T} p{p}: {gc.tolist()}")
    # the samplers read the same keep threshold: draft = target, so every
    # proposal is accepted and every token is one of the kept ties
    rows = torch.from_numpy(np.stack([z1] * 3)).to(dev).to(dtype)
    g = uno.sample_linear(rows[:2][None].contiguous(), rows[None].contiguous(), 1e-4, 0, 0.5, 3, 1)
    toks = np_of(g["tokens"])[0]
    assert np_of(g["accept_len"])[0] == 3
    kept = set(np.flatnonzero(z1 == 5.0)[:1501].tolist())
    assert set(toks.tolist()) <= kept, toks
    zh = rows.float().cpu().numpy()
    o = oracle.linear(zh[:2][None], zh[None], 1e-4, 0, 0.5, 3, 1)
    t = Tally(f"nucleus single-key run sampler {dtype}")
    t.compare({key: np_of(g[key]) for key in ("tokens", "accept_len", "proposals")}, o,
              ("tokens", "accept_len", "proposals"), "nucleus ties sampler")
    t.check_rate()


def test_side_stream_matches_default_stream():
    dev = device()
    rng = np.random.default_rng(64)
    batch, B, N = 24, 4, 5000
    R = torch.from_numpy(_rows(rng, (batch, B + 1, N))).to(dev)
    D = (R[:, :B] + 0.5 * torch.randn(batch, B, N, device=dev)).contiguous()
    rid = np.arange(batch, dtype=np.uint32) * 977 + 5
    ref = uno.sample_linear(D, R, 1.0, 50, 0.9, 12, 4, request_ids=rid)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        got = uno.sample_linear(D, R, 1.0, 50, 0.9, 12, 4, request_ids=rid, stream=s)
        s.synchronize()
        for key in ("tokens", "accept_len", "proposals"):
            assert torch.equal(got[key], ref[key]), key


@pytest.mark.parametrize("nbytes,wg", [(607744 * 5, 607744), (1 << 20, 4096), (16 * 1000 + 48, 1024)])
def test_stream_read_folds_every_word_once(nbytes, wg):
    # the bandwidth reference reads each 16-byte vector of its range exactly
    # once: per workgroup, the XOR of all its 32-bit words
    dev = device()
    lib = uno.load_library()
    import ctypes
    rng = np.random.default_rng(65)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(dev)
    groups = (nbytes + wg - 1) // wg
    out = torch.zeros(groups, dtype=torch.int32, device=dev)
    st = lib.uno_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, wg, ctypes.c_void_p(out.data_ptr()),
                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    got = np_of(out).view(np.uint32)
    words = wg // 4
    want = [np.bitwise_xor.reduce(host[g * words:(g + 1) * words]) for g in range(groups)]
    assert np.array_equal(got, np.array(want, dtype=np.uint32))
