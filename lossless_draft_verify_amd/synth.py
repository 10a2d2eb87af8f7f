"""Seeded synthetic logits for the UNO sampling workloads.

This module only generates inputs; it holds none of the method's arithmetic,
and both the GPU path and the oracle consume what it returns.

Recipe (stands in for Qwen3-8B logits on GSM8K / MATH500 / AIME25, which are not
available here).  For each request b and position d = 0..B a reference row is
drawn:  R_d[i] = -slope * log(1 + rank_d(i)) + N(0, 1), where rank_d is a
seeded uniformly random permutation of the vocabulary.  Target row d is R_d;
draft row d (d < B) is R_d + sigma_d * N(0, 1).  In tree mode the target row of
node n is R_{depth(n)} (rows of equal depth share their content).  bf16
workloads round the float32 values to nearest-even bfloat16.  Each cycle draws
fresh rows from a generator seeded with (seed, cycle).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple

import torch

VOCAB_QWEN3 = 151936


@dataclass(frozen=True)
class Workload:
    name: str
    mode: str            # "linear" or "tree"
    batch: int
    B: int
    vocab: int
    dtype: str           # "f32" or "bf16"
    slope: float
    sigma: Tuple[float, ...]   # draft noise per position (length B)
    temperature: float
    top_k: int           # <= 0: off
    top_p: float         # 1.0: off
    seed: int
    cycles: int
    K: int = 1
    V: int = 0
    order: int = 0       # filter order: 0 top-k first, 1 joint
    sets: tuple = ()     # per-request sets: request b takes sets[b % len] instead of the scalars above
    note: str = field(default="", compare=False)

    @property
    def mixed(self) -> bool:
        return len(self.sets) > 0

    def request_params(self, b: int):
        """(temperature, top_k, top_p, order) of request b."""
        if self.sets:
            return self.sets[b % len(self.sets)]
        return (self.temperature, self.top_k, self.top_p, self.order)

    @property
    def rows_per_cycle(self) -> int:
        """Logit rows the sampling path reads per cycle (draft + target)."""
        if self.mode == "linear":
            return self.batch * (2 * self.B + 1)
        return self.batch * (self.B + self.V + 1)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def bytes_per_cycle(self) -> int:
        return self.rows_per_cycle * self.vocab * self.elem_bytes

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


def _const(v, n):
    return tuple(float(v) for _ in range(n))


# Per-request parameter sets of the mixed workload: greedy, the pages' top-k 50 /
# top-p 0.95, no top-p, a large k, a tiny k and the joint order.
MIXED_SETS = ((0.0, 0, 1.0, 0), (1.0, 50, 0.95, 0), (0.7, 20, 1.0, 0), (1.3, 256, 0.9, 0), (1.0, 3, 0.5, 0),
              (1.0, 50, 0.9, 1), (0.5, 8, 0.8, 0), (1.0, 100, 0.99, 1))

# Per-request sets over both paths: greedy, top-k 50 / top-p 0.95, the full
# softmax at two temperatures, a nucleus without top-k, joint-order sets at two
# temperatures and a large k.
MIXED_FULL_SETS = ((0.0, 0, 1.0, 0), (1.0, 50, 0.95, 0), (1.0, 0, 1.0, 0), (0.8, 0, 0.9, 0), (1.0, 50, 0.9, 1),
                   (0.7, 100, 0.9, 1), (1.3, 256, 0.9, 0), (0.6, 0, 1.0, 0))

WORKLOADS = {
    "tiny": Workload("tiny", "linear", batch=2, B=4, vocab=1000, dtype="f32", slope=1.0,
                     sigma=_const(0.5, 4), temperature=1.0, top_k=0, top_p=1.0, seed=42,
                     cycles=100, note="tiny linear UNO, dense full-softmax path"),
    "linear_8_1_8": Workload("linear_8_1_8", "linear", batch=64, B=8, vocab=VOCAB_QWEN3,
                             dtype="f32", slope=1.2,
                             sigma=tuple(0.3 + 0.1 * j for j in range(8)), temperature=1.0,
                             top_k=50, top_p=0.95, seed=42, cycles=1000,
                             note="Linear 8/1/8, 64 requests, sparse top-k 50 / top-p 0.95"),
    # the headline shape with the joint filter order (top-p on the full softmax)
    "linear_8_1_8_joint": Workload("linear_8_1_8_joint", "linear", batch=64, B=8, vocab=VOCAB_QWEN3,
                                   dtype="f32", slope=1.2,
                                   sigma=tuple(0.3 + 0.1 * j for j in range(8)), temperature=1.0,
                                   top_k=50, top_p=0.95, seed=42, cycles=1000, order=1,
                                   note="Linear 8/1/8, 64 requests, joint top-k 50 / top-p 0.95"),
    # the headline shape with one parameter set per request (MIXED_SETS)
    "linear_8_1_8_mixed": Workload("linear_8_1_8_mixed", "linear", batch=64, B=8, vocab=VOCAB_QWEN3,
                                   dtype="f32", slope=1.2,
                                   sigma=tuple(0.3 + 0.1 * j for j in range(8)), temperature=1.0,
                                   top_k=50, top_p=0.95, seed=42, cycles=1000, sets=MIXED_SETS,
                                   note="Linear 8/1/8, 64 requests, per-request parameters"),
    # the headline shape with per-request sets that mix top-k and full-vocabulary rows
    "linear_8_1_8_mixed_full": Workload("linear_8_1_8_mixed_full", "linear", batch=64, B=8, vocab=VOCAB_QWEN3,
                                        dtype="f32", slope=1.2,
                                        sigma=tuple(0.3 + 0.1 * j for j in range(8)), temperature=1.0,
                                        top_k=50, top_p=0.95, seed=42, cycles=1000, sets=MIXED_FULL_SETS,
                                        note="Linear 8/1/8, 64 requests, top-k and full-vocabulary sets"),
    # the headline shape with top-k off: a full-vocabulary nucleus at top-p 0.95
    "linear_8_1_8_nucleus": Workload("linear_8_1_8_nucleus", "linear", batch=64, B=8, vocab=VOCAB_QWEN3,
                                     dtype="f32", slope=1.2,
                                     sigma=tuple(0.3 + 0.1 * j for j in range(8)), temperature=1.0,
                                     top_k=0, top_p=0.95, seed=42, cycles=1000,
                                     note="Linear 8/1/8, 64 requests, top-p 0.95 over the full vocabulary"),
    "linear_dense": Workload("linear_dense", "linear", batch=256, B=16, vocab=VOCAB_QWEN3,
                             dtype="bf16", slope=1.0, sigma=_const(0.5, 16), temperature=0.7,
                             top_k=0, top_p=1.0, seed=7, cycles=200,
                             note="Linear dense, 256 requests, B=16, full-vocab residual"),
    "tree_16_32_32": Workload("tree_16_32_32", "tree", batch=1, B=16, K=32, V=32,
                              vocab=VOCAB_QWEN3, dtype="f32", slope=1.2, sigma=_const(0.3, 16),
                              temperature=1.0, top_k=50, top_p=0.95, seed=42, cycles=2000,
                              note="Tree 16/32/32, one request"),
    "tree_8_16_8": Workload("tree_8_16_8", "tree", batch=64, B=8, K=16, V=8, vocab=VOCAB_QWEN3,
                            dtype="bf16", slope=1.0, sigma=_const(0.4, 8), temperature=1.0,
                            top_k=50, top_p=0.95, seed=123, cycles=500,
                            note="Tree 8/16/8, 64 requests"),
    # the tree shapes with filters that keep the whole vocabulary (dense tree mode)
    "tree_dense_16_32_32": Workload("tree_dense_16_32_32", "tree", batch=1, B=16, K=32, V=32,
                                    vocab=VOCAB_QWEN3, dtype="f32", slope=1.2, sigma=_const(0.3, 16),
                                    temperature=1.0, top_k=0, top_p=1.0, seed=42, cycles=2000,
                                    note="Tree 16/32/32, one request, full-softmax filters"),
    "tree_dense_8_16_8": Workload("tree_dense_8_16_8", "tree", batch=64, B=8, K=16, V=8,
                                  vocab=VOCAB_QWEN3, dtype="bf16", slope=1.0, sigma=_const(0.4, 8),
                                  temperature=1.0, top_k=0, top_p=1.0, seed=123, cycles=500,
                                  note="Tree 8/16/8, 64 requests, full-softmax filters"),
}


def _generator(seed: int, cycle: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + int(cycle)) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def reference_rows(g: torch.Generator, shape, vocab: int, slope: float, device) -> torch.Tensor:
    """R[..., i] = -slope*log(1+rank(i)) + N(0,1), one random rank per row."""
    n = 1
    for s in shape:
        n *= s
    rank = torch.argsort(torch.rand(n, vocab, generator=g, device=device), dim=1)
    z = -float(slope) * torch.log1p(rank.to(torch.float32))
    z += torch.randn(n, vocab, generator=g, device=device)
    return z.view(*shape, vocab)


def linear_inputs(w: Workload, cycle: int = 0, device="cpu", batch: int | None = None):
    """(draft [batch, B, N], target [batch, B+1, N]) in the workload's dtype."""
    batch = w.batch if batch is None else batch
    g = _generator(w.seed, cycle, device)
    R = reference_rows(g, (batch, w.B + 1), w.vocab, w.slope, device)
    sig = torch.tensor(w.sigma, dtype=torch.float32, device=device).view(1, w.B, 1)
    draft = R[:, : w.B] + sig * torch.randn(batch, w.B, w.vocab, generator=g, device=device)
    return draft.to(w.torch_dtype).contiguous(), R.to(w.torch_dtype).contiguous()


def tree_inputs(w: Workload, cycle: int = 0, device="cpu", batch: int | None = None):
    """(draft [batch, B, N], reference rows R [batch, B+1, N]) in the workload's dtype.

    Target rows for the tree's nodes come from ``tree_target_rows``."""
    return linear_inputs(w, cycle, device, batch)


def tree_target_rows(R: torch.Tensor, node_depth: torch.Tensor, num_nodes: torch.Tensor,
                     V: int) -> torch.Tensor:
    """Target [batch, V+1, N]: row n = R[b, depth(n)]; rows past num_nodes copy row 0."""
    batch = R.shape[0]
    dep = node_depth.to(torch.long).clone().to(R.device)
    nn = num_nodes.to(torch.long).to(R.device)
    idx = torch.arange(V + 1, device=R.device).view(1, -1)
    dep = torch.where(idx < nn.view(-1, 1), dep, torch.zeros_like(dep))
    dep = dep.clamp(min=0)
    out = torch.gather(R, 1, dep.view(batch, V + 1, 1).expand(batch, V + 1, R.shape[-1]))
    return out.contiguous()


def as_float32_numpy(t: torch.Tensor):
    """Exact float32 view of f32/bf16 logits for the host side."""
    return t.detach().to("cpu").to(torch.float32).contiguous().numpy()


# Tree-suffix attention inputs at the tree workloads' verify shapes (Qwen3-8B
# attention: 32 query heads, 8 key/value heads, head dimension 128).
ATTENTION_WORKLOADS = {
    "tree_attention_8_16_8": dict(batch=64, n=9, Hq=32, Hkv=8, D=128, seed=123),
    "tree_attention_16_32_32": dict(batch=1, n=33, Hq=32, Hkv=8, D=128, seed=42),
}


def attention_inputs(batch: int, n: int, Hq: int, Hkv: int, D: int, seed: int, device="cpu"):
    """q, k, v, o_prefix (bf16), lse_prefix (fp32), node_parent (int32, parents
    before children) for `batch` requests of n verify tokens each."""
    g = _generator(seed, 0, device)
    q = torch.randn(batch, n, Hq, D, generator=g, device=device).to(torch.bfloat16)
    k = torch.randn(batch, n, Hkv, D, generator=g, device=device).to(torch.bfloat16)
    v = torch.randn(batch, n, Hkv, D, generator=g, device=device).to(torch.bfloat16)
    o_prefix = torch.randn(batch, n, Hq, D, generator=g, device=device).to(torch.bfloat16)
    lse_prefix = 3.0 * torch.randn(batch, n, Hq, generator=g, device=device)
    u = torch.rand(batch, n, generator=g, device=device)
    idx = torch.arange(n, device=device).view(1, n)
    parent = torch.floor(u * idx).to(torch.int32)           # uniform over the earlier nodes
    parent[:, 0] = -1
    return q, k, v, o_prefix, lse_prefix.contiguous(), parent.contiguous()
