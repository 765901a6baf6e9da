"""Pins for oracle/schedule_ref.py: linear scan, binary search and brute force agree."""
import numpy as np
import pytest

from oracle import schedule_ref as sr


def _cases():
    rng = np.random.default_rng(0)
    cases = [
        ([0] * 7, 3), ([5], 1), ([5], 7), ([1, 0, 0, 2, 0], 4), ([0, 3, 0], 10),
        ([0, 0, 1], 2), ([100], 3), ([1] * 50, 7), ([0, 1] * 20, 6),
    ]
    for _ in range(40):
        B = int(rng.integers(1, 40))
        c = rng.integers(0, 6, size=B)
        c[rng.random(B) < 0.3] = 0
        cases.append((c.tolist(), int(rng.integers(1, 80))))
    return cases


@pytest.mark.parametrize("c,W", _cases())
def test_searches_agree_with_bruteforce(c, W):
    lin = sr.starts_linear(c, W)
    bis = sr.starts_binary(c, W)
    assert lin == bis
    T = sum(c)
    seq = sr.enumerate_units(c)
    assert len(seq) == T
    bf = sr.worker_units_bruteforce(c, W)
    for w in range(W):
        units = sr.walk(c, bis[w], bis[w + 1])
        assert units == bf[w]
        assert len(units) in (T // W, -(-T // W))
        if units:
            assert bis[w] == units[0]
            assert c[bis[w][0]] > 0                   # never starts on an empty row
    assert bis[W] == (len(c), 0)
    # every unit exactly once, in order
    assert [u for ws in bf for u in ws] == seq


def test_zero_total_gives_terminal_starts():
    assert sr.starts_binary([0, 0, 0], 4) == [(3, 0)] * 5


def test_units_per_row():
    assert sr.units_per_row([0, 1, 255, 256, 257, 512, 65536]) == [0, 1, 1, 1, 2, 2, 256]
    with pytest.raises(ValueError):
        sr.units_per_row([3, -1])


def test_large_batch_binary_equals_linear():
    rng = np.random.default_rng(1)
    ctx = np.clip(np.rint(np.exp(rng.normal(np.log(4096), 1.0, 2048))), 1, 65536).astype(int)
    ctx[rng.choice(2048, 205, replace=False)] = 0
    c = sr.units_per_row(ctx)
    for W in (1, 37, 256, 4096):
        assert sr.starts_linear(c, W) == sr.starts_binary(c, W)
