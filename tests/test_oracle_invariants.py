"""Pins for oracle/reference.py from properties the definition fixes.

Each test is chosen so that a plausible slip in the oracle (a dropped scale,
a flipped sign, a wrong causal offset, a page looked up through the wrong
index, the wrong query row) fails at least one of them.
"""
import numpy as np
import pytest
import torch

from oracle import reference
from workloads import make_fp4, make_fp8


def _run8(d, **kw):
    return reference.paged_mqa_logits_fp8(d["q"], d["kv_cache"], d["weights"], d["context_lens"],
                                          d["block_table"], d["max_context_len"],
                                          page_size=d["page_size"], **kw)


def _run4(d, **kw):
    return reference.paged_mqa_logits_fp4(d["q"], d["q_scale"], d["kv_cache"], d["weights"],
                                          d["context_lens"], d["block_table"],
                                          d["max_context_len"], page_size=d["page_size"], **kw)


@pytest.mark.parametrize("next_n", [1, 2])
def test_mask_positions(next_n):
    ctx = np.array([0, 1, 63, 64, 65, 200, 257], np.int32)
    M = 260
    d = make_fp8(ctx, next_n=next_n, max_context_len=M, seed=1)
    lg = _run8(d)["logits"]
    for b, L in enumerate(ctx):
        for j in range(next_n):
            lim = max(0, min(L - next_n + 1 + j, M))
            row = lg[b * next_n + j]
            assert np.all(np.isfinite(row[:lim]))
            assert np.all(row[lim:] == -np.inf)


def test_truncation_at_max_context_len():
    d = make_fp8([300, 90], max_context_len=300, seed=2)
    full = _run8(d)["logits"]
    d2 = dict(d, max_context_len=100)
    trunc = _run8(d2)["logits"]
    assert trunc.shape == (2, 100)
    assert np.array_equal(trunc, full[:, :100])


def test_zero_rows_all_neg_inf():
    d = make_fp8([0, 0, 5], max_context_len=64, seed=3)
    lg = _run8(d)["logits"]
    assert np.all(lg[:2] == -np.inf)


def _permute_pages(d, seed):
    rng = np.random.default_rng(seed)
    n = d["kv_cache"].shape[0]
    perm = rng.permutation(n)            # new position of old page p is perm[p]
    kv = np.empty_like(d["kv_cache"])
    kv[perm] = d["kv_cache"]
    return dict(d, kv_cache=kv, block_table=perm[d["block_table"]].astype(np.int32))


def test_page_permutation_invariance_fp8():
    d = make_fp8([130, 64, 1, 0, 77], next_n=2, max_context_len=140, seed=4)
    a = _run8(d)["logits"]
    b = _run8(_permute_pages(d, 9))["logits"]
    assert np.array_equal(a, b)
    # and a block table that names the wrong pages changes the result
    bad = dict(d, block_table=np.roll(d["block_table"], 1, axis=1))
    assert not np.array_equal(a, _run8(bad)["logits"])


def test_page_permutation_invariance_fp4():
    d = make_fp4([130, 64, 0, 77], max_context_len=140, seed=5)
    assert np.array_equal(_run4(d)["logits"], _run4(_permute_pages(d, 3))["logits"])


def test_one_hot_head_reduces_to_relu_dot():
    """w = e_h gives ReLU(scale_t * q_h . k_t); decoded here through torch."""
    d = make_fp8([70], max_context_len=70, seed=6, negative_scales=True)
    h = 17
    w = np.zeros_like(d["weights"])
    w[0, h] = 1.0
    lg = _run8(dict(d, weights=w))["logits"][0]
    P, D = 64, 128
    qv = torch.from_numpy(d["q"][0, 0, h].copy()).view(torch.float8_e4m3fn).double()
    for t in range(70):
        page = d["kv_cache"][d["block_table"][0, t // P]]
        kv = torch.from_numpy(page[(t % P) * D:(t % P + 1) * D].copy()).view(torch.float8_e4m3fn).double()
        s = float(page[P * D + 4 * (t % P):P * D + 4 * (t % P) + 4].view("<f4")[0])
        expect = max(0.0, s * float(torch.dot(qv, kv)))
        assert lg[t] == np.float32(expect)


def test_constant_q_k_closed_form():
    """q[h,:] = a_h and k_t[:] = b_t give sum_h w_h ReLU(128 * s_t * a_h * b_t)."""
    P, D, H = 64, 128, 64
    d = make_fp8([100], max_context_len=128, seed=7)
    rng = np.random.default_rng(7)
    codes = np.array([0x38, 0xB8, 0x30, 0xC4, 0x44, 0x01, 0x81, 0x7E], np.uint8)
    vals = {0x38: 1.0, 0xB8: -1.0, 0x30: 0.5, 0xC4: -3.0, 0x44: 3.0, 0x01: 2.0 ** -9,
            0x81: -2.0 ** -9, 0x7E: 448.0}
    a = rng.choice(codes, H)
    q = np.repeat(a[None, None, :, None], D, axis=3).astype(np.uint8)
    kv = d["kv_cache"].copy()
    bvals = rng.choice(codes, 100)
    svals = rng.choice([0.25, 2.0, 1.0 / 448, -0.5], 100).astype(np.float32)
    for t in range(100):
        pid = d["block_table"][0, t // P]
        kv[pid, (t % P) * D:(t % P + 1) * D] = bvals[t]
        kv[pid, P * D + 4 * (t % P):P * D + 4 * (t % P) + 4] = np.array([svals[t]], "<f4").view(np.uint8)
    lg = _run8(dict(d, q=q, kv_cache=kv))["logits"][0]
    w = d["weights"][0].astype(np.float64)
    for t in range(100):
        x = np.array([128.0 * float(svals[t]) * vals[int(ah)] * vals[int(bvals[t])] for ah in a])
        assert lg[t] == np.float32(np.maximum(x, 0.0) @ w)
    assert np.all(lg[100:] == -np.inf)


def test_linearity_power_of_two():
    d = make_fp8([150, 20], next_n=2, max_context_len=160, seed=8)
    base = _run8(d)["logits"]
    twice_w = _run8(dict(d, weights=(2 * d["weights"]).astype(np.float32)))["logits"]
    assert np.array_equal(twice_w, 2 * base)
    kv = d["kv_cache"].copy()
    s = kv[:, 64 * 128:].copy().view("<f4")
    kv[:, 64 * 128:] = (2 * s).astype("<f4").view(np.uint8)
    assert np.array_equal(_run8(dict(d, kv_cache=kv))["logits"], 2 * base)


def test_relu_is_applied_after_scaling():
    """Negating every scale must change the result (ReLU acts on scale*q.k)."""
    d = make_fp8([90], max_context_len=90, seed=9)
    kv = d["kv_cache"].copy()
    s = kv[:, 64 * 128:].copy().view("<f4")
    kv[:, 64 * 128:] = (-s).astype("<f4").view(np.uint8)
    pos = _run8(d, want_fp64=True)["fp64"][0]
    neg = _run8(dict(d, kv_cache=kv), want_fp64=True)["fp64"][0]
    # sum_h w ReLU(x) - sum_h w ReLU(-x) = sum_h w x
    d2 = dict(d, weights=np.ones_like(d["weights"]))
    assert not np.allclose(pos, neg)
    p1 = _run8(d2, want_fp64=True)["fp64"][0]
    n1 = _run8(dict(d2, kv_cache=kv), want_fp64=True)["fp64"][0]
    assert np.all(p1 >= 0) and np.all(n1 >= 0)


def test_next_n_reduces_to_single_query():
    ctx = np.array([1, 2, 65, 300], np.int32)
    M = 310
    d = make_fp8(ctx, next_n=2, max_context_len=M, seed=10)
    two = _run8(d)["logits"]
    for j in range(2):
        single = dict(d, q=np.ascontiguousarray(d["q"][:, j:j + 1]),
                      weights=np.ascontiguousarray(d["weights"][j::2]),
                      context_lens=(ctx - 1 + j).clip(0).astype(np.int32), next_n=1)
        one = _run8(single)["logits"]
        assert np.array_equal(two[j::2], one), j


def test_row_permutation_equivariance():
    ctx = np.array([10, 0, 200, 64], np.int32)
    d = make_fp8(ctx, max_context_len=200, seed=11)
    base = _run8(d)["logits"]
    p = np.array([2, 0, 3, 1])
    dp = dict(d, q=d["q"][p], weights=d["weights"][p], context_lens=ctx[p],
              block_table=d["block_table"][p])
    assert np.array_equal(_run8(dp)["logits"], base[p])


def test_rows_subset_equals_full():
    d = make_fp8([40, 0, 99], next_n=2, max_context_len=100, seed=12)
    full = _run8(d, want_tol=True)
    sub = _run8(d, rows=[5, 0, 3], want_tol=True)
    assert np.array_equal(sub["logits"], full["logits"][[5, 0, 3]])
    assert np.array_equal(sub["tol"], full["tol"][[5, 0, 3]])


def test_fp4_one_hot_and_closed_form():
    """MXFP4: constant element codes with block scales give a closed form."""
    d = make_fp4([40], max_context_len=64, seed=13)
    H, P = 64, 64
    q = np.full_like(d["q"], 0x22)                    # every element 1.0
    qs = np.full_like(d["q_scale"], 127)
    qs[0, 0, :, 1] = 128                               # block 1 scaled by 2
    kv = d["kv_cache"].copy()
    kv[:, :P * 64] = 0x44                              # every element 2.0
    kv[:, P * 64:] = 126                               # every block scale 1/2
    w = np.zeros_like(d["weights"])
    w[0, 5] = 1.5
    w[0, 9] = -0.25
    lg = _run4(dict(d, q=q, q_scale=qs, kv_cache=kv, weights=w))["logits"][0]
    # per head: blocks 0,2,3 contribute 32*1*1 each, block 1 32*2*1 -> 160
    assert np.all(lg[:40] == np.float32(160 * (1.5 - 0.25)))
    assert np.all(lg[40:] == -np.inf)
