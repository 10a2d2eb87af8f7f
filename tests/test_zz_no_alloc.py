"""uno_sample_linear_noalloc (the allocation-free entry point) against
uno_sample_linear, through the C ABI: two calls in a row, the second with a
smaller input, each bit-identical to the workspace entry point's output."""
import ctypes

import numpy as np
import pytest
import torch

import lossless_draft_verify_amd as uno
from lossless_draft_verify_amd import synth
from gpu_util import device, np_of, say

pytestmark = pytest.mark.gpu


def _noalloc(lib, draft, target, T, k, p, seed, offset, rid):
    batch, B, vocab = draft.shape
    dev = draft.device
    out = dict(tokens=torch.full((batch, B + 1), -7, dtype=torch.int32, device=dev),
               accept_len=torch.full((batch,), -7, dtype=torch.int32, device=dev),
               proposals=torch.full((batch, B), -7, dtype=torch.int32, device=dev),
               flags=torch.full((batch,), -7, dtype=torch.int32, device=dev))
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    sp = uno.Sampling(T, k, p, 0)
    dt = 0 if draft.dtype == torch.float32 else 1
    st = lib.uno_sample_linear_noalloc(P(draft), P(target), dt, batch, B, vocab, ctypes.byref(sp), seed, offset,
                                       P(rid), P(out["tokens"]), P(out["accept_len"]), P(out["proposals"]),
                                       P(out["flags"]), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.uno_status_string(st)
    return out


@pytest.mark.parametrize("name,T,k,p,small", [("linear_8_1_8", 1.0, 50, 0.95, 16),
                                              ("linear_dense", 0.7, 0, 1.0, 40),
                                              ("linear_8_1_8", 1.0, 0, 0.95, 8)])
def test_no_alloc_matches_workspace_entry_point(name, T, k, p, small):
    dev = device()
    lib = uno.load_library()
    w = synth.WORKLOADS[name]
    for i, batch in enumerate((w.batch, small)):
        draft, target = synth.linear_inputs(w, cycle=5 + i, device=dev, batch=batch)
        rid = torch.arange(batch, dtype=torch.int32, device=dev) * 3 + 11
        size = uno.workspace_bytes(uno.OP_SAMPLE_LINEAR, batch, w.B, 1, w.B, w.vocab, 0 if w.dtype == "f32" else 1,
                                   T, k, p)
        assert size <= uno.NOALLOC_SCRATCH_BYTES
        got = _noalloc(lib, draft, target, T, k, p, w.seed, 40 + i, rid)
        ref = uno.sample_linear(draft, target, T, k, p, w.seed, 40 + i, request_ids=rid)
        torch.cuda.synchronize()
        for key in ("tokens", "accept_len", "proposals", "flags"):
            assert torch.equal(got[key], ref[key]), (name, batch, key)
        say(f"no-alloc {name} T{T} k{k} p{p} batch {batch}: workspace {size} bytes, "
            f"mean accept_len {np_of(got['accept_len']).mean():.3f}")
