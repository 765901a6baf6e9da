"""Pins of oracle/topk.py against brute force, a library sort and hand cases."""
import itertools
import math

import numpy as np
import pytest

from oracle import topk


def _plain_key(x):
    """Plain Python float order, with the one rule IEEE comparison lacks made
    explicit: -0 < +0 (the pair compares the float first, and only two zeros
    of opposite sign reach the second item)."""
    x = float(x)
    return (x, 1 if x == 0.0 and math.copysign(1.0, x) > 0 else 0)


def _brute(values, n, k):
    """Best k-subset by exhaustive search: maximise the sorted values
    lexicographically (largest first), prefer lower indices on equal values.
    Independent of oracle/topk.py's bit-pattern keys."""
    row = list(np.asarray(values, np.float32)[:n])
    if n <= k:
        return list(range(n))
    key = [_plain_key(v) for v in row]
    best = None
    for sub in itertools.combinations(range(n), k):
        score = (sorted((key[i] for i in sub), reverse=True), [-i for i in sorted(sub)])
        if best is None or score > best[0]:
            best = (score, list(sub))
    return best[1]


@pytest.mark.parametrize("seed", range(40))
def test_matches_brute_force_on_tiny_rows(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 9))
    k = int(rng.integers(1, 6))
    pool = np.array([-1.5, -0.0, 0.0, 0.25, 0.25, 3.0, -np.inf, 7.0], np.float32)
    row = rng.choice(pool, size=max(n, 1)) if seed % 2 else \
        rng.standard_normal(max(n, 1)).astype(np.float32)
    idx, val = topk.select_topk(row, n, k)
    want = _brute(row, n, k)
    got = [i for i in idx.tolist() if i >= 0]
    assert got == sorted(want)
    assert np.array_equal(val[:len(got)], row[got])
    assert np.all(idx[len(got):] == -1) and np.all(np.isneginf(val[len(got):]))


def test_matches_library_sort():
    rng = np.random.default_rng(1)
    row = rng.standard_normal(5000).astype(np.float32)
    idx, val = topk.select_topk(row, 4000, 777)
    want = np.sort(np.argsort(-row[:4000].astype(np.float64), kind="stable")[:777])
    assert np.array_equal(idx, want)


def test_hand_ties_and_signed_zeros():
    row = np.array([1.0, -0.0, 2.0, 0.0, 1.0, 1.0, -3.0], np.float32)
    # k = 3: 2.0 (index 2), then the three 1.0s tie: indices 0 and 4
    idx, val = topk.select_topk(row, 7, 3)
    assert idx.tolist() == [0, 2, 4] and val.tolist() == [1.0, 2.0, 1.0]
    # k = 5: 2, 1, 1, 1, then +0 (index 3) beats -0 (index 1)
    idx, _ = topk.select_topk(row, 7, 5)
    assert idx.tolist() == [0, 2, 3, 4, 5]
    # only the first 2 columns are candidates
    idx, val = topk.select_topk(row, 2, 4)
    assert idx.tolist() == [0, 1, -1, -1]
    assert val[1] == 0 and np.signbit(val[1]) and np.isneginf(val[2:]).all()


def test_order_key_is_the_float_order():
    v = np.array([-np.inf, -3e38, -1.0, -1e-45, -0.0, 0.0, 1e-45, 1.0, 3e38, np.inf],
                 np.float32)
    k = topk.order_key(v)
    assert np.all(np.diff(k.astype(np.float64)) > 0)


def test_fused_row_length():
    assert topk.fused_row_length(1000, 1, 0, 4096, 4) == 1000
    assert topk.fused_row_length(1000, 2, 0, 4096, 4) == 999
    assert topk.fused_row_length(1000, 1, 0, 700, 4) == 700      # truncated
    assert topk.fused_row_length(1000, 1, 0, 4096, 3) == 768     # schedule covers 3 units
    assert topk.fused_row_length(0, 2, 0, 4096, 0) == 0


def test_order_key_against_plain_float_order_on_random_bit_patterns():
    """The bit-pattern key against plain float comparison (with -0 < +0) on
    20000 random fp32 bit patterns (NaN excluded) plus the special values:
    sorted by key, consecutive values never decrease in the plain order, and
    keys are equal exactly when the bit patterns are."""
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    special = np.array([-np.inf, np.inf, -0.0, 0.0, 1e-45, -1e-45, 1.0, -1.0],
                       np.float32).view(np.uint32)
    bits = np.concatenate([bits, special, special])
    v = bits.view(np.float32)
    v = v[~np.isnan(v)]
    key = topk.order_key(v)
    order = np.argsort(key, kind="stable")
    sv, sk = v[order], key[order]
    for a, b, ka, kb in zip(sv[:-1], sv[1:], sk[:-1], sk[1:]):
        pa, pb = _plain_key(a), _plain_key(b)
        assert pa <= pb
        assert (ka == kb) == (pa == pb)
