"""select_topk against the oracle selection exactly, and the fused indexer
step (paged_mqa_topk_fp8/fp4) against the fp64 oracle logits."""
import numpy as np
import pytest
import torch

import parity
from gpu_util import announce, oracle, upload
from oracle import schedule_ref as sr
from oracle import topk as otk
from workloads import make_fp4, make_fp8, make_workload

pytestmark = pytest.mark.gpu
pmqa = pytest.importorskip("paged_mqa_logits_amd")


def _rows(rng, rows, M, pool):
    if pool:
        vals = np.array([-2.0, -0.0, 0.0, 0.5, 0.5, 1.0, 3.0, -np.inf, 7.25], np.float32)
        return rng.choice(vals, size=(rows, M)).astype(np.float32)
    return (rng.standard_normal((rows, M)) * 10).astype(np.float32)


@pytest.mark.parametrize("pool", [False, True])
@pytest.mark.parametrize("M,stride,k", [(1, 4, 1), (37, 40, 5), (1000, 1024, 7),
                                        (5000, 5004, 2048), (3000, 3000, 2999)])
def test_select_topk_matches_oracle(pool, M, stride, k):
    announce(f"select_topk M={M} k={k} pool={pool}")
    rng = np.random.default_rng(M + k + pool)
    rows = 64
    x = _rows(rng, rows, M, pool)
    n = rng.integers(0, M + 1, size=rows).astype(np.int32)
    n[:5] = [0, M, min(k, M), max(0, min(k - 1, M)), min(k + 1, M)]
    n[5] = -3                                      # clamped to 0
    buf = torch.full((rows, stride), float("nan"), device="cuda")
    buf[:, :M] = torch.from_numpy(x).cuda()        # NaN past the width: never read
    idx, val = pmqa.select_topk(buf[:, :M], torch.from_numpy(n).cuda(), k)
    idx, val = idx.cpu().numpy(), val.cpu().numpy()
    for r in range(rows):
        wi, wv = otk.select_topk(x[r], max(0, int(n[r])), k)
        assert np.array_equal(idx[r], wi), r
        assert np.array_equal(val[r].view(np.uint32), wv.view(np.uint32)), r


@pytest.mark.parametrize("rows", [3000, 8192, 8193])
def test_select_topk_many_rows(rows):
    """Workgroups take rows longest first (by count class) up to 8192 rows,
    in index order beyond: every row is still selected exactly once, with
    lengths spread over many classes and many rows per class."""
    announce(f"select_topk rows={rows}")
    rng = np.random.default_rng(rows)
    M, k = 300, 17
    x = (rng.standard_normal((rows, M)) * 3).astype(np.float32)
    n = rng.integers(0, M + 1, size=rows).astype(np.int32)
    n[rng.random(rows) < 0.3] = 40                 # a crowded class
    n[::97] = 0
    idx, val = pmqa.select_topk(torch.from_numpy(x).cuda(), torch.from_numpy(n).cuda(), k)
    idx, val = idx.cpu().numpy(), val.cpu().numpy()
    for r in range(rows):
        wi, wv = otk.select_topk(x[r], int(n[r]), k)
        assert np.array_equal(idx[r], wi), r
        assert np.array_equal(val[r].view(np.uint32), wv.view(np.uint32)), r


def test_select_topk_long_rows_sample_misses_and_overflows():
    """Rows too long for LDS are sampled (256 of every 4096 columns) to guess
    the bins of the k-th key.  An unrepresentative sample (the columns it
    reads hold only small values) and a gathered list that overflows one
    wavefront's share (every large value in the first eighth of the row)
    must both fall back to the exact three-pass path."""
    announce("select_topk sample misses / overflow")
    rng = np.random.default_rng(21)
    rows, M, k = 4, 65536, 2048
    x = rng.standard_normal((rows, M)).astype(np.float32)
    sampled = (np.arange(M) % 4096) < 256
    x[0, sampled] -= np.float32(100.0)              # the sample sees only small values
    x[1, : M // 8] += np.float32(10.0)              # all large values in one chunk
    n = np.array([M, M, M, 7681], np.int32)
    idx, val = pmqa.select_topk(torch.from_numpy(x).cuda(), torch.from_numpy(n).cuda(), k)
    idx, val = idx.cpu().numpy(), val.cpu().numpy()
    for r in range(rows):
        wi, wv = otk.select_topk(x[r], int(n[r]), k)
        assert np.array_equal(idx[r], wi), r
        assert np.array_equal(val[r].view(np.uint32), wv.view(np.uint32)), r


def test_select_topk_long_rows():
    announce("select_topk 131072 columns")
    rng = np.random.default_rng(9)
    rows, M, k = 6, 131072, 2048
    x = (rng.standard_normal((rows, M))).astype(np.float32)
    x[1] = np.float32(0.5)                         # all equal: the first k columns
    x[2, ::3] = np.float32(4.0)                    # many ties above the rest
    n = np.array([M, M, M, 70001, 2049, 2048], np.int32)
    idx, val = pmqa.select_topk(torch.from_numpy(x).cuda(), torch.from_numpy(n).cuda(), k)
    idx, val = idx.cpu().numpy(), val.cpu().numpy()
    for r in range(rows):
        wi, wv = otk.select_topk(x[r], int(n[r]), k)
        assert np.array_equal(idx[r], wi), r
        assert np.array_equal(val[r], wv), r


def _fused(d, k, dev=None, num_workers=None, schedule=None):
    dev = upload(d) if dev is None else dev
    nn = int(d["next_n"])
    fp8 = d["variant"] == "fp8"
    variant = pmqa.VARIANT_FP8 if fp8 else pmqa.VARIANT_FP4
    if schedule is None:
        schedule = pmqa.compute_schedule(dev["context_lens"], num_workers=num_workers,
                                         variant=variant, next_n=nn)
    M = int(d["max_context_len"])
    if fp8:
        idx, val = pmqa.paged_mqa_topk_fp8(dev["q"], dev["kv_cache"], dev["weights"],
                                           dev["context_lens"], dev["block_table"], schedule, M,
                                           k, num_workers=num_workers)
    else:
        idx, val = pmqa.paged_mqa_topk_fp4(dev["q"], dev["q_scale"], dev["kv_cache"],
                                           dev["weights"], dev["context_lens"],
                                           dev["block_table"], schedule, M, k,
                                           num_workers=num_workers)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), val.cpu().numpy()


def _row_lengths(d, rows=None):
    ctx = d["context_lens"]
    nn = int(d["next_n"])
    c = sr.units_per_row(np.maximum(ctx, 0))
    rows = range(len(ctx) * nn) if rows is None else rows
    return np.array([otk.fused_row_length(ctx[r // nn], nn, r % nn, d["max_context_len"],
                                          c[r // nn]) for r in rows])


@pytest.mark.parametrize("variant", ["fp8", "fp4"])
@pytest.mark.parametrize("next_n", [1, 2])
def test_fused_topk_against_oracle(variant, next_n):
    announce(f"fused top-k {variant} next_n={next_n}")
    rng = np.random.default_rng(20 + next_n)
    ctx = rng.integers(0, 3000, size=40)
    ctx[::6] = 0
    ctx[1], ctx[2] = 1, 2                          # rows shorter than next_n
    ctx[3] = 3500                                  # truncated at max_context_len
    mk = make_fp8 if variant == "fp8" else make_fp4
    d = mk(ctx, next_n=next_n, max_context_len=3100, seed=20 + next_n,
           bt_stride=-(-3500 // 64))
    ref = oracle(d)
    for k in (1, 100, 1024):
        idx, val = _fused(d, k)
        parity.check_topk(idx, val, ref, _row_lengths(d), k, f"{variant} k={k}")


def test_fused_topk_mismatched_schedule_selects_nothing():
    announce("fused top-k, foreign schedule")
    d = make_fp8([100, 300], max_context_len=400, seed=23)
    dev = upload(d)
    sched = pmqa.compute_schedule(dev["context_lens"], num_workers=16)
    idx, val = _fused(d, 8, dev=dev, num_workers=8, schedule=sched)
    assert np.all(idx == -1) and np.all(np.isneginf(val))


@pytest.mark.timeout(400)
def test_fused_topk_full_size_sampled():
    announce("fused top-k large_fp8 k=2048 (sampled rows)")
    d = make_workload("large_fp8")
    idx, val = _fused(d, 2048)
    ctx = d["context_lens"]
    rng = np.random.default_rng(24)
    rows = sorted(set(rng.choice(len(ctx), 6, replace=False).tolist()) |
                  {int(np.argmax(ctx)), int(np.nonzero(ctx == 0)[0][0])})
    ref = oracle(d, rows=rows)
    n = _row_lengths(d, rows)
    parity.check_topk(idx[rows], val[rows], ref, n, 2048, "large_fp8")
