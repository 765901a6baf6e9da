"""Pins for oracle/reference.py against the rational brute force (oracle/exact.py)
and against the hand-derived fixtures in tests/golden/."""
from fractions import Fraction

import numpy as np
import pytest

import golden_fixtures as gf
from oracle import exact, formats, reference
from workloads import make_fp4, make_fp8


def _compare_exact(res, ex, weights_abs_bound=None):
    lg = res["logits"]
    f64 = res["fp64"]
    for i, row in enumerate(ex):
        for t, v in enumerate(row):
            if v is None:
                assert lg[i, t] == -np.inf and np.signbit(lg[i, t])
                continue
            # fp64 oracle within rounding of the exact value
            assert abs(Fraction(float(f64[i, t])) - v) <= Fraction(1, 10 ** 9) * (abs(v) + 1)
            # fp32 output is the correctly rounded exact value unless it sits
            # within fp64 noise of an fp32 rounding tie
            rounded = np.float32(float(v))
            if lg[i, t] != rounded:
                ulp = np.spacing(np.float32(abs(float(v))))
                mid = abs(abs(Fraction(float(lg[i, t])) + Fraction(float(rounded))) / 2 - abs(v))
                assert mid <= Fraction(float(ulp)) * Fraction(1, 10 ** 6), (i, t, lg[i, t], v)


@pytest.mark.parametrize("next_n", [1, 2])
@pytest.mark.parametrize("seed", [0, 1])
def test_fp8_matches_rational_bruteforce(next_n, seed):
    ctx = [0, 5, 9] if next_n == 1 else [1, 7, 2]
    d = make_fp8(ctx, next_n=next_n, max_context_len=10, seed=seed, num_heads=4,
                 head_dim=16, page_size=4, negative_scales=(seed == 1))
    res = reference.paged_mqa_logits_fp8(d["q"], d["kv_cache"], d["weights"], d["context_lens"],
                                         d["block_table"], d["max_context_len"], page_size=4,
                                         want_fp64=True)
    ex = exact.logits_fp8(d["q"], d["kv_cache"], d["weights"], d["context_lens"],
                          d["block_table"], d["max_context_len"], page_size=4)
    _compare_exact(res, ex)


def test_fp8_full_dims_matches_rational_bruteforce():
    d = make_fp8([3, 0], next_n=1, max_context_len=4, seed=7)
    res = reference.paged_mqa_logits_fp8(d["q"], d["kv_cache"], d["weights"], d["context_lens"],
                                         d["block_table"], d["max_context_len"], want_fp64=True)
    ex = exact.logits_fp8(d["q"], d["kv_cache"], d["weights"], d["context_lens"],
                          d["block_table"], d["max_context_len"])
    _compare_exact(res, ex)


@pytest.mark.parametrize("next_n", [1, 2])
def test_fp4_matches_rational_bruteforce(next_n):
    d = make_fp4([6, 0, 3], next_n=next_n, max_context_len=7, seed=3, num_heads=4,
                 head_dim=64, page_size=4)
    res = reference.paged_mqa_logits_fp4(d["q"], d["q_scale"], d["kv_cache"], d["weights"],
                                         d["context_lens"], d["block_table"],
                                         d["max_context_len"], page_size=4, want_fp64=True)
    ex = exact.logits_fp4(d["q"], d["q_scale"], d["kv_cache"], d["weights"], d["context_lens"],
                          d["block_table"], d["max_context_len"], page_size=4)
    _compare_exact(res, ex)


def test_fp8_contraction_is_exact_at_extremes():
    """Dot products of extreme E4M3 values (448, subnormals, mixed signs) are
    exact in fp64 whatever the summation order."""
    rng = np.random.default_rng(0)
    codes = np.array([0x7E, 0xFE, 0x01, 0x81, 0x07, 0x08, 0x77, 0xF7], np.uint8)
    a = rng.choice(codes, size=(16, 128))
    b = rng.choice(codes, size=(8, 128))
    prod = formats.decode_e4m3fn(a) @ formats.decode_e4m3fn(b).T
    fa = [[Fraction(float(x)) for x in r] for r in formats.decode_e4m3fn(a)]
    fb = [[Fraction(float(x)) for x in r] for r in formats.decode_e4m3fn(b)]
    for i in range(16):
        for j in range(8):
            assert Fraction(float(prod[i, j])) == sum(x * y for x, y in zip(fa[i], fb[j]))


@pytest.mark.parametrize("case", [0, 1])
def test_hand_fixture_fp8(case):
    f = gf.load_fp8(case)
    res = reference.paged_mqa_logits_fp8(f["q"], f["kv_cache"], f["weights"], f["context_lens"],
                                         f["block_table"], f["max_context_len"],
                                         page_size=f["page_size"])
    assert np.array_equal(res["logits"].astype(np.float64), f["expected"])


def test_hand_fixture_fp8_embedded():
    e = gf.embed_fp8(gf.load_fp8(1))
    res = reference.paged_mqa_logits_fp8(e["q"], e["kv_cache"], e["weights"], e["context_lens"],
                                         e["block_table"], e["max_context_len"])
    assert np.array_equal(res["logits"].astype(np.float64), e["expected"])


def test_hand_fixture_fp4():
    f = gf.load_fp4()
    res = reference.paged_mqa_logits_fp4(f["q"], f["q_scale"], f["kv_cache"], f["weights"],
                                         f["context_lens"], f["block_table"],
                                         f["max_context_len"], page_size=f["page_size"])
    assert np.array_equal(res["logits"].astype(np.float64), f["expected"])
    e = gf.embed_fp4(f)
    res = reference.paged_mqa_logits_fp4(e["q"], e["q_scale"], e["kv_cache"], e["weights"],
                                         e["context_lens"], e["block_table"], e["max_context_len"])
    assert np.array_equal(res["logits"].astype(np.float64), e["expected"])


def _check_tol(tol, bounds, rel=1e-12):
    """The oracle's per-entry bound against 2e-3 * (exact magnitude sum) + 1e-6."""
    for i, row in enumerate(bounds):
        for t, v in enumerate(row):
            if v is None:
                assert tol[i, t] == 0.0, (i, t)
                continue
            want = Fraction(2, 1000) * v + Fraction(1, 10 ** 6)
            assert abs(Fraction(float(tol[i, t])) - want) <= Fraction(rel) * want, \
                (i, t, float(tol[i, t]), float(want))


@pytest.mark.parametrize("next_n", [1, 2])
@pytest.mark.parametrize("seed", [0, 1])
def test_fp8_tol_matches_exact_bound(next_n, seed):
    """The parity bound 2e-3 * sum_h |w_h| |scale_t q_h.k_t| + 1e-6 (the
    stated tolerance) against the rational brute force's exact magnitude
    sums, with negative token scales in one seed."""
    ctx = [0, 5, 9] if next_n == 1 else [1, 7, 2]
    d = make_fp8(ctx, next_n=next_n, max_context_len=10, seed=seed, num_heads=4,
                 head_dim=16, page_size=4, negative_scales=(seed == 1))
    res = reference.paged_mqa_logits_fp8(d["q"], d["kv_cache"], d["weights"], d["context_lens"],
                                         d["block_table"], d["max_context_len"], page_size=4,
                                         want_tol=True)
    bounds = exact.bounds_fp8(d["q"], d["kv_cache"], d["weights"], d["context_lens"],
                              d["block_table"], d["max_context_len"], page_size=4)
    _check_tol(res["tol"], bounds)


@pytest.mark.parametrize("next_n", [1, 2])
def test_fp4_tol_matches_exact_bound(next_n):
    d = make_fp4([6, 0, 3], next_n=next_n, max_context_len=7, seed=3, num_heads=4,
                 head_dim=64, page_size=4)
    res = reference.paged_mqa_logits_fp4(d["q"], d["q_scale"], d["kv_cache"], d["weights"],
                                         d["context_lens"], d["block_table"],
                                         d["max_context_len"], page_size=4, want_tol=True)
    bounds = exact.bounds_fp4(d["q"], d["q_scale"], d["kv_cache"], d["weights"],
                              d["context_lens"], d["block_table"], d["max_context_len"],
                              page_size=4)
    _check_tol(res["tol"], bounds)


def _check_tol_hand(tol, bound, expected):
    """Hand-derived bounds: 2e-3 * bound + 1e-6 on scored entries, 0 on masked ones."""
    masked = np.isneginf(expected)
    assert np.all(tol[masked] == 0.0)
    want = 2e-3 * bound[~masked] + 1e-6
    assert np.allclose(tol[~masked], want, rtol=1e-12, atol=0.0), (tol, want)


@pytest.mark.parametrize("case", [0, 1])
def test_hand_fixture_fp8_tol(case):
    f = gf.load_fp8(case)
    res = reference.paged_mqa_logits_fp8(f["q"], f["kv_cache"], f["weights"], f["context_lens"],
                                         f["block_table"], f["max_context_len"],
                                         page_size=f["page_size"], want_tol=True)
    _check_tol_hand(res["tol"], f["bound"], f["expected"])
    e = gf.embed_fp8(f)
    res = reference.paged_mqa_logits_fp8(e["q"], e["kv_cache"], e["weights"], e["context_lens"],
                                         e["block_table"], e["max_context_len"], want_tol=True)
    _check_tol_hand(res["tol"], e["bound"], e["expected"])


def test_hand_fixture_fp4_tol():
    f = gf.load_fp4()
    res = reference.paged_mqa_logits_fp4(f["q"], f["q_scale"], f["kv_cache"], f["weights"],
                                         f["context_lens"], f["block_table"],
                                         f["max_context_len"], page_size=f["page_size"],
                                         want_tol=True)
    _check_tol_hand(res["tol"], f["bound"], f["expected"])
    e = gf.embed_fp4(f)
    res = reference.paged_mqa_logits_fp4(e["q"], e["q_scale"], e["kv_cache"], e["weights"],
                                         e["context_lens"], e["block_table"], e["max_context_len"],
                                         want_tol=True)
    _check_tol_hand(res["tol"], e["bound"], e["expected"])


def test_exact_bound_is_the_magnitude_sum():
    """On a fixture whose values are hand-derived, the brute force's exact
    magnitude sums are the hand-derived bounds."""
    for case in range(2):
        f = gf.load_fp8(case)
        b = exact.bounds_fp8(f["q"], f["kv_cache"], f["weights"], f["context_lens"],
                             f["block_table"], f["max_context_len"], page_size=f["page_size"])
        got = np.array([0.0 if v is None else float(v) for v in b[0]])
        assert np.array_equal(got, f["bound"][0])
    f = gf.load_fp4()
    b = exact.bounds_fp4(f["q"], f["q_scale"], f["kv_cache"], f["weights"], f["context_lens"],
                         f["block_table"], f["max_context_len"], page_size=f["page_size"])
    got = np.array([0.0 if v is None else float(v) for v in b[0]])
    assert np.array_equal(got, f["bound"][0])
