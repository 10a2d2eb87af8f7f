"""GPU parity of uno_sample_linear against the oracle on the linear workloads."""
import numpy as np
import pytest
import torch

import lossless_draft_verify_amd as uno
import oracle
from lossless_draft_verify_amd import synth
from gpu_util import Tally, device, np_of, say
from stats_util import chisq_pvalue

pytestmark = pytest.mark.gpu


def _run(draft, target, T, k, p, seed, offset, request_ids=None, tally=None, label="",
         order=uno.ORDER_TOPK_FIRST):
    g = uno.sample_linear(draft, target, T, k, p, seed, offset, request_ids=request_ids, order=order)
    torch.cuda.synchronize()
    rid = None if request_ids is None else np.asarray(request_ids, dtype=np.uint32)
    o = oracle.linear(synth.as_float32_numpy(draft), synth.as_float32_numpy(target), T, k, p,
                      seed=seed, offset=offset, request_ids=rid, order=order)
    gg = dict(tokens=np_of(g["tokens"]), accept_len=np_of(g["accept_len"]),
              proposals=np_of(g["proposals"]))
    t = tally or Tally()
    t.compare(gg, o, ("tokens", "accept_len", "proposals"), label)
    return gg, o


def _cycles(w, n, batch=None, label=None, order=uno.ORDER_TOPK_FIRST):
    dev = device()
    tally = Tally()
    acc = []
    for c in range(n):
        draft, target = synth.linear_inputs(w, cycle=c, device=dev, batch=batch)
        gg, o = _run(draft, target, w.temperature, w.top_k, w.top_p, w.seed, c, tally=tally,
                     label=f"{label or w.name} cycle {c}", order=order)
        acc.append(gg["accept_len"])
    tally.check_rate()
    a = np.concatenate(acc)
    say(f"{label or w.name}: {tally.total} request-cycles, excused {tally.excused}, "
        f"mean accept_len {a.mean():.3f}, TPF {oracle.tpf(a):.3f}")
    return a


def test_tiny_workload_all_cycles():
    # the tiny workload in full: batch 2, B 4, vocab 1000, dense path, 100 cycles
    _cycles(synth.WORKLOADS["tiny"], 100)


def test_linear_8_1_8_reduced_batch():
    _cycles(synth.WORKLOADS["linear_8_1_8"], 4, batch=8, label="linear_8_1_8 b8")


def test_linear_8_1_8_full_size():
    # the full workload shape and launch configuration of the bench, one cycle
    _cycles(synth.WORKLOADS["linear_8_1_8"], 1, label="linear_8_1_8 b64")


def test_linear_dense_reduced():
    _cycles(synth.WORKLOADS["linear_dense"], 2, batch=6, label="linear_dense b6")


def test_linear_dense_full_size_sampled_requests():
    # full batch 256 in one launch; the oracle checks 16 requests spread over it
    dev = device()
    w = synth.WORKLOADS["linear_dense"]
    draft, target = synth.linear_inputs(w, cycle=0, device=dev)
    g = uno.sample_linear(draft, target, w.temperature, w.top_k, w.top_p, w.seed, 0)
    torch.cuda.synchronize()
    pick = np.array([0, 1, 17, 40, 63, 77, 100, 128, 141, 170, 199, 200, 222, 240, 254, 255])
    pt = torch.from_numpy(pick).to(dev)
    o = oracle.linear(synth.as_float32_numpy(draft[pt]), synth.as_float32_numpy(target[pt]),
                      w.temperature, w.top_k, w.top_p, seed=w.seed, offset=0,
                      request_ids=pick.astype(np.uint32))
    t = Tally("linear_dense b256 sample")
    gg = {k: np_of(g[k])[pick] for k in ("tokens", "accept_len", "proposals")}
    t.compare(gg, o, ("tokens", "accept_len", "proposals"), "linear_dense b256 sample")
    t.check_rate()
    acc = np_of(g["accept_len"])
    assert acc.min() >= 1 and acc.max() <= w.B + 1
    say(f"linear_dense b256: mean accept_len {acc.mean():.3f}, excused {t.excused}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("T,k,p", [(0.0, 0, 1.0), (1.0, 1, 1.0), (0.8, 20, 0.9), (1.0, 0, 1.0),
                                   (1.5, 256, 0.99)])
def test_parameter_grid_small_vocab(dtype, T, k, p):
    dev = device()
    rng = np.random.default_rng(31)
    batch, B, N = 24, 5, 1003
    R = rng.standard_normal((batch, B + 1, N)).astype(np.float32) * 2
    d = (R[:, :B] + 0.5 * rng.standard_normal((batch, B, N))).astype(np.float32)
    draft = torch.from_numpy(d).to(dev).to(dtype).contiguous()
    target = torch.from_numpy(R).to(dev).to(dtype).contiguous()
    rid = rng.integers(0, 2**32, size=batch, dtype=np.uint64).astype(np.uint32)
    t = Tally()
    for c in range(3):
        _run(draft, target, T, k, p, 99, 1000 + c, request_ids=rid, tally=t,
             label=f"grid {dtype} T{T} k{k} p{p}")
    t.check_rate()


def test_q_equals_p_accepts_everything_on_gpu():
    dev = device()
    rng = np.random.default_rng(32)
    batch, B, N = 16, 6, 5000
    R = torch.from_numpy((rng.standard_normal((batch, B + 1, N)) * 2).astype(np.float32)).to(dev)
    for (T, k, p) in [(1.0, 50, 0.95), (1.0, 0, 1.0)]:
        g = uno.sample_linear(R[:, :B].contiguous(), R, T, k, p, 5, 0)
        torch.cuda.synchronize()
        assert torch.all(g["accept_len"] == B + 1)
        assert torch.equal(g["tokens"][:, :B], g["proposals"])


def test_gpu_output_is_lossless_small_vocab():
    # many requests share one set of rows; Philox varies with the request id
    dev = device()
    rng = np.random.default_rng(33)
    B, N, n = 3, 8, 200_000
    R = (rng.standard_normal((B + 1, N)) * 1.5).astype(np.float32)
    D = (R[:B] + rng.standard_normal((B, N)) * 0.8).astype(np.float32)
    draft = torch.from_numpy(D).to(dev).expand(n, B, N).contiguous()
    target = torch.from_numpy(R).to(dev).expand(n, B + 1, N).contiguous()
    for (T, k, p) in [(1.0, 0, 1.0), (0.8, 5, 0.9)]:
        g = uno.sample_linear(draft, target, T, k, p, 2024, 0)
        torch.cuda.synchronize()
        tok, acc = np_of(g["tokens"]), np_of(g["accept_len"])
        P = oracle.filter_rows(R, T, k, p)["dense"]
        for j in range(B + 1):
            sel = acc >= j + 1
            assert chisq_pvalue(tok[sel, j], P[j]) > 1e-4, (T, k, p, j)
        say(f"lossless T{T} k{k} p{p}: mean accept_len {acc.mean():.3f}")


def test_linear_is_deterministic():
    dev = device()
    w = synth.WORKLOADS["linear_8_1_8"]
    draft, target = synth.linear_inputs(w, cycle=3, device=dev, batch=16)
    a = uno.sample_linear(draft, target, 1.0, 50, 0.95, 42, 3)
    b = uno.sample_linear(draft, target, 1.0, 50, 0.95, 42, 3)
    torch.cuda.synchronize()
    for key in ("tokens", "accept_len", "proposals"):
        assert torch.equal(a[key], b[key])


def test_linear_8_1_8_joint_order():
    # the headline workload with the joint filter order (full batch, two cycles)
    _cycles(synth.WORKLOADS["linear_8_1_8"], 2, label="linear_8_1_8 joint", order=uno.ORDER_JOINT)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("T,k,p", [(1.0, 20, 0.8), (0.7, 256, 0.95)])
def test_joint_order_small_vocab(dtype, T, k, p):
    dev = device()
    rng = np.random.default_rng(33)
    batch, B, N = 24, 5, 3001
    R = rng.standard_normal((batch, B + 1, N)).astype(np.float32) * 2
    d = (R[:, :B] + 0.5 * rng.standard_normal((batch, B, N))).astype(np.float32)
    draft = torch.from_numpy(d).to(dev).to(dtype).contiguous()
    target = torch.from_numpy(R).to(dev).to(dtype).contiguous()
    t = Tally()
    for c in range(3):
        _run(draft, target, T, k, p, 5, c, tally=t, label=f"joint {dtype} T{T} k{k} p{p}",
             order=uno.ORDER_JOINT)
    t.check_rate()


# ---- full-vocabulary nucleus (top-p without top-k) ---------------------------------------

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("T,p", [(1.0, 0.9), (0.7, 0.5), (1.3, 0.99)])
def test_nucleus_small_vocab(dtype, T, p):
    dev = device()
    rng = np.random.default_rng(34)
    batch, B, N = 24, 5, 3001
    R = rng.standard_normal((batch, B + 1, N)).astype(np.float32) * 2
    d = (R[:, :B] + 0.5 * rng.standard_normal((batch, B, N))).astype(np.float32)
    draft = torch.from_numpy(d).to(dev).to(dtype).contiguous()
    target = torch.from_numpy(R).to(dev).to(dtype).contiguous()
    t = Tally()
    for c in range(3):
        _run(draft, target, T, 0, p, 8, c, tally=t, label=f"nucleus {dtype} T{T} p{p}")
    t.check_rate()


def test_linear_8_1_8_nucleus_reduced_batch():
    # the headline rows with top-k off and top-p 0.95 (a nucleus of thousands of ids)
    dev = device()
    w = synth.WORKLOADS["linear_8_1_8"]
    t = Tally()
    acc = []
    for c in range(2):
        draft, target = synth.linear_inputs(w, cycle=c, device=dev, batch=8)
        gg, _ = _run(draft, target, w.temperature, 0, w.top_p, w.seed, c, tally=t, label=f"L818 nucleus {c}")
        acc.append(gg["accept_len"])
    t.check_rate()
    say(f"linear_8_1_8 nucleus b8: mean accept_len {np.concatenate(acc).mean():.3f}, excused {t.excused}")


# ---- rows of more than 128 dense chunks ----------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("T,p", [(0.9, 1.0), (1.1, 0.9)])
def test_dense_rows_of_more_than_128_chunks(dtype, T, p):
    # 300007 logits: 146 whole chunks of 2048 and a ragged one, so the dense
    # draws read their chunk statistics from memory rather than from two
    # registers per lane, and bf16 rows start off 16-byte boundaries
    dev = device()
    rng = np.random.default_rng(61)
    batch, B, N = 3, 3, 300007
    R = (rng.standard_normal((batch, B + 1, N)) * 2).astype(np.float32)
    d = (R[:, :B] + 0.5 * rng.standard_normal((batch, B, N))).astype(np.float32)
    draft = torch.from_numpy(d).to(dev).to(dtype).contiguous()
    target = torch.from_numpy(R).to(dev).to(dtype).contiguous()
    t = Tally(f"long dense rows {dtype} T{T} p{p}")
    for c in range(3):
        _run(draft, target, T, 0, p, 7, 500 + c, tally=t, label=f"long dense rows {dtype} T{T} p{p} cycle {c}")
    t.check_rate()
