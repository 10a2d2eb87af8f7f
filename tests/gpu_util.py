"""Shared helpers for the GPU parity tests (comparison and excusal accounting)."""
import numpy as np
import pytest
import torch

MARGIN_TOL = 1e-6          # a decision whose uniform lies this close to its threshold may differ
EXCUSED_RATE_MAX = 1e-4    # excused request-cycles must stay below 0.01 %

# Every Tally of the session adds here; conftest.py reports the combined rate.
SESSION = {"total": 0, "excused": 0, "near": 0, "by_test": []}


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


class Tally:
    """Counts request-cycles, excused mismatches and near-threshold request-cycles.

    A request-cycle whose outputs differ from the oracle's is excused only when
    the oracle's margin (the smallest distance of any of its decisions' uniforms
    from the decision's threshold, relative) is below MARGIN_TOL; any other
    difference fails at once.  `near` counts the request-cycles with such a
    margin whether or not they differ (the literal near-threshold count)."""

    def __init__(self, label=""):
        self.label = label
        self.total = 0
        self.excused = 0
        self.near = 0

    def compare(self, gpu: dict, orc: dict, keys, what=""):
        n = orc["margin"].shape[0]
        bad = np.zeros(n, dtype=bool)
        for k in keys:
            g = np.asarray(gpu[k]).reshape(n, -1)
            o = np.asarray(orc[k]).reshape(n, -1)
            bad |= np.any(g != o, axis=1)
        near = orc["margin"] < MARGIN_TOL
        hard = bad & ~near
        if np.any(hard):
            i = int(np.flatnonzero(hard)[0])
            msg = {k: (np.asarray(gpu[k]).reshape(n, -1)[i].tolist(),
                       np.asarray(orc[k]).reshape(n, -1)[i].tolist()) for k in keys}
            raise AssertionError(f"{what}: {int(hard.sum())} unexcused mismatches; first at "
                                 f"request {i} (margin {orc['margin'][i]:.3g}): {msg}")
        self.total += n
        self.excused += int(bad.sum())
        self.near += int(near.sum())

    def check_rate(self):
        """The excused rate bar; the counts also go to the session summary."""
        SESSION["total"] += self.total
        SESSION["excused"] += self.excused
        SESSION["near"] += self.near
        SESSION["by_test"].append((self.label, self.total, self.excused, self.near))
        say(f"[tally] {self.label}: {self.total} request-cycles, excused {self.excused}, "
            f"near-threshold {self.near}")
        assert self.excused <= EXCUSED_RATE_MAX * self.total, (self.label, self.excused, self.total)


def np_of(t):
    return t.detach().cpu().numpy()
