"""Philox4x32-10 in the oracle against the published known-answer vectors."""
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def _kat():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            w = [int(x, 16) for x in line.split()]
            rows.append((w[0:4], w[4:6], w[6:10]))
    return rows


def test_philox_known_answers():
    kat = _kat()
    assert len(kat) == 3
    for ctr, key, out in kat:
        got = oracle.philox4x32_10(ctr, key)
        assert [int(x) for x in got] == out, (ctr, key, [hex(int(x)) for x in got])


def test_uniform_counter_layout():
    # counter = (request, position, offset lo, offset hi), key = (seed lo, seed hi),
    # u = word * 2^-32
    seed, req, pos, off = 0x0123456789ABCDEF, 77, 5, 0x1_0000_0003
    w = oracle.philox4x32_10([req, pos, off & 0xFFFFFFFF, off >> 32],
                             [seed & 0xFFFFFFFF, seed >> 32])
    for lane in range(4):
        assert oracle.uniform(seed, req, pos, off, lane) == float(w[lane]) * 2.0 ** -32


def test_uniforms_look_uniform():
    u = np.array([oracle.uniform(42, r, 0, 0, 0) for r in range(20000)])
    assert u.min() >= 0.0 and u.max() < 1.0
    assert abs(u.mean() - 0.5) < 0.01
    hist = np.histogram(u, bins=10, range=(0, 1))[0]
    assert hist.min() > 1800
