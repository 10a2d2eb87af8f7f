"""Shared helpers for the GPU parity tests (comparison and excusal accounting)."""
import numpy as np
import pytest
import torch

MARGIN_TOL = 1e-6          # a decision whose uniform lies this close to its threshold may differ
EXCUSED_RATE_MAX = 1e-4    # excused request-cycles must stay below 0.01 %


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


class Tally:
    """Counts request-cycles, exact matches and excused mismatches."""

    def __init__(self):
        self.total = 0
        self.excused = 0

    def compare(self, gpu: dict, orc: dict, keys, what=""):
        """Rows that differ in any key must have an oracle margin below MARGIN_TOL."""
        n = orc["margin"].shape[0]
        bad = np.zeros(n, dtype=bool)
        for k in keys:
            g = np.asarray(gpu[k]).reshape(n, -1)
            o = np.asarray(orc[k]).reshape(n, -1)
            bad |= np.any(g != o, axis=1)
        hard = bad & ~(orc["margin"] < MARGIN_TOL)
        if np.any(hard):
            i = int(np.flatnonzero(hard)[0])
            msg = {k: (np.asarray(gpu[k]).reshape(n, -1)[i].tolist(),
                       np.asarray(orc[k]).reshape(n, -1)[i].tolist()) for k in keys}
            raise AssertionError(f"{what}: {int(hard.sum())} unexcused mismatches; first at "
                                 f"request {i} (margin {orc['margin'][i]:.3g}): {msg}")
        self.total += n
        self.excused += int(bad.sum())

    def check_rate(self):
        assert self.excused <= EXCUSED_RATE_MAX * self.total, (self.excused, self.total)


def np_of(t):
    return t.detach().cpu().numpy()
