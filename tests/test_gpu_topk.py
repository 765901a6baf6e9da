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


# "auto": the binding passes a workspace when rows are long enough to be
# split (more than 524288 columns, at most 512 rows); None: never split.
WS = ["auto", None]


def _check_rows(x, n, k, idx, val):
    for r in range(x.shape[0]):
        wi, wv = otk.select_topk(x[r], max(0, int(n[r])), k)
        assert np.array_equal(idx[r], wi), r
        assert np.array_equal(val[r].view(np.uint32), wv.view(np.uint32)), r


@pytest.mark.parametrize("ws", WS)
@pytest.mark.parametrize("pool", [False, True])
@pytest.mark.parametrize("M,stride,k", [(1, 4, 1), (37, 40, 5), (1000, 1024, 7),
                                        (5000, 5004, 2048), (3000, 3000, 2999)])
def test_select_topk_matches_oracle(pool, M, stride, k, ws):
    announce(f"select_topk M={M} k={k} pool={pool} ws={ws}")
    rng = np.random.default_rng(M + k + pool)
    rows = 64
    x = _rows(rng, rows, M, pool)
    n = rng.integers(0, M + 1, size=rows).astype(np.int32)
    n[:5] = [0, M, min(k, M), max(0, min(k - 1, M)), min(k + 1, M)]
    n[5] = -3                                      # clamped to 0
    buf = torch.full((rows, stride), float("nan"), device="cuda")
    buf[:, :M] = torch.from_numpy(x).cuda()        # NaN past the width: never read
    idx, val = pmqa.select_topk(buf[:, :M], torch.from_numpy(n).cuda(), k,
                                select_workspace=ws)
    _check_rows(x, n, k, idx.cpu().numpy(), val.cpu().numpy())


@pytest.mark.parametrize("ws", WS)
@pytest.mark.parametrize("rows", [512, 513, 3000, 8192, 8193])
def test_select_topk_many_rows(rows, ws):
    """Rows of at most 6144 candidates are selected by one wavefront each,
    eight (or sixteen) to a workgroup: every row is selected exactly once
    however the rows fall into the groups, with many empty and equal
    lengths."""
    announce(f"select_topk rows={rows} ws={ws}")
    rng = np.random.default_rng(rows)
    M, k = 300, 17
    x = (rng.standard_normal((rows, M)) * 3).astype(np.float32)
    n = rng.integers(0, M + 1, size=rows).astype(np.int32)
    n[rng.random(rows) < 0.3] = 40                 # a crowded class
    n[::97] = 0
    idx, val = pmqa.select_topk(torch.from_numpy(x).cuda(), torch.from_numpy(n).cuda(), k,
                                select_workspace=ws)
    _check_rows(x, n, k, idx.cpu().numpy(), val.cpu().numpy())


@pytest.mark.parametrize("ws", WS)
def test_select_topk_many_wide_rows(ws):
    """More rows than workgroups resident at once, most of them longer than
    a wavefront takes (one workgroup each, started as the short rows' slots
    free up), beside rows a wavefront takes and rows of at most k
    candidates."""
    announce(f"select_topk 1500 rows of up to 12000 ws={ws}")
    rng = np.random.default_rng(77)
    rows, M, k = 1500, 12000, 2048
    x = rng.standard_normal((rows, M)).astype(np.float32)
    n = rng.integers(6145, M + 1, size=rows).astype(np.int32)
    n[::5] = rng.integers(2049, 6145, size=len(n[::5]))
    n[::7] = rng.integers(0, 2049, size=len(n[::7]))
    n[3::11] = 6144
    n[4::11] = 6145
    idx, val = pmqa.select_topk(torch.from_numpy(x).cuda(), torch.from_numpy(n).cuda(), k,
                                select_workspace=ws)
    _check_rows(x, n, k, idx.cpu().numpy(), val.cpu().numpy())


@pytest.mark.parametrize("ws", WS)
@pytest.mark.parametrize("M,k", [(3000, 700), (3000, 2999), (20000, 2048), (20000, 9)])
def test_select_topk_special_cut_values(M, k, ws):
    """Rows whose k-th key lands on a special value: the write compares
    values against the cut directly only for normal cut values with a
    normal value just below them; zeros (-0 < +0), denormals, the smallest
    normals and infinities take the key compare.  Values drawn from a pool
    of such numbers, with many ties, at wavefront and workgroup lengths."""
    announce(f"select_topk special cut values M={M} k={k} ws={ws}")
    rng = np.random.default_rng(M + 7 * k)
    tiny = np.float32(np.finfo(np.float32).tiny)          # smallest normal
    den = np.float32(1e-40)                               # a denormal
    sub = np.array([1], np.uint32).view(np.float32)[0]    # smallest denormal
    pool = np.array([-np.inf, -1.0, -tiny, -den, -sub, -0.0, 0.0, sub, den, tiny,
                     np.float32(2) * tiny, 1.0, np.inf], np.float32)
    rows = 24
    x = rng.choice(pool, size=(rows, M)).astype(np.float32)
    x[1::3] = rng.choice(pool[3:10], size=(len(x[1::3]), M))  # cuts among zeros and denormals
    n = rng.integers(k + 1, M + 1, size=rows).astype(np.int32)
    n[0] = M
    idx, val = pmqa.select_topk(torch.from_numpy(x).cuda(), torch.from_numpy(n).cuda(), k,
                                select_workspace=ws)
    _check_rows(x, n, k, idx.cpu().numpy(), val.cpu().numpy())


@pytest.mark.parametrize("ws", WS)
def test_select_topk_rows_padded_with_neg_inf(ws):
    """Candidates past a row's finite values are -inf (a length beyond the
    context): rows of -inf only and rows with fewer than k finite values
    take the digit passes, whose histograms then count tens of thousands
    of equal keys; the -inf columns are taken in column order."""
    announce(f"select_topk -inf padded rows ws={ws}")
    rng = np.random.default_rng(41)
    rows, M, k = 12, 65536, 2048
    x = np.full((rows, M), -np.inf, np.float32)
    finite = [0, 1000, 3000, 0, 1500, 5000, 0, 2047, 2048, 2049, 100, 60000]
    for r, f in enumerate(finite):
        x[r, :f] = rng.standard_normal(f).astype(np.float32)
    n = np.array([M, M, M, 6144, 6144, 6144, 3000, M, M, M, 40000, M], np.int32)
    idx, val = pmqa.select_topk(torch.from_numpy(x).cuda(), torch.from_numpy(n).cuda(), k,
                                select_workspace=ws)
    _check_rows(x, n, k, idx.cpu().numpy(), val.cpu().numpy())


@pytest.mark.parametrize("offset", [0, 1, 2, 3])
def test_select_topk_output_alignment(offset):
    """Output rows are written in 16-byte stores only where both output rows
    start on a 16-byte boundary; outputs given as views starting 1-3
    elements into their storage take 4-byte stores, with the same result.
    Rows of at most k, of a wavefront's and of a workgroup's lengths, with k
    not a multiple of 256 (a partial last block)."""
    announce(f"select_topk output offset {offset}")
    rng = np.random.default_rng(300 + offset)
    rows, M, k = 96, 9000, 2000
    x = rng.standard_normal((rows, M)).astype(np.float32)
    n = rng.integers(0, M + 1, size=rows).astype(np.int32)
    n[:6] = [0, 1999, 2000, 2001, 6144, 6145]
    idx_buf = torch.full((rows, k + 8), -7, dtype=torch.int32, device="cuda")
    val_buf = torch.full((rows, k + 8), 7.0, dtype=torch.float32, device="cuda")
    idx, val = pmqa.select_topk(torch.from_numpy(x).cuda(), torch.from_numpy(n).cuda(), k,
                                indices=idx_buf[:, offset:offset + k],
                                values=val_buf[:, offset:offset + k], select_workspace=None)
    _check_rows(x, n, k, idx.cpu().numpy(), val.cpu().numpy())
    ib, vb = idx_buf.cpu().numpy(), val_buf.cpu().numpy()
    outside = np.r_[0:offset, offset + k:k + 8]    # columns of the storage outside the view
    assert (ib[:, outside] == -7).all() and (vb[:, outside] == 7.0).all()


@pytest.mark.parametrize("ws", WS)
def test_select_topk_long_rows_sample_misses_and_overflows(ws):
    """Rows of more than 6144 candidates are sampled (256 of every 4096
    columns) to set a threshold for the listing pass.  An unrepresentative
    sample (the columns it reads hold only small values: the list has fewer
    than k keys) and a list that overflows one wavefront's region (every
    large value in the first eighth of the row) must both fall back to the
    exact digit passes."""
    announce(f"select_topk sample misses / overflow ws={ws}")
    rng = np.random.default_rng(21)
    rows, M, k = 4, 65536, 2048
    x = rng.standard_normal((rows, M)).astype(np.float32)
    sampled = (np.arange(M) % 4096) < 256
    x[0, sampled] -= np.float32(100.0)              # the sample sees only small values
    x[1, : M // 8] += np.float32(10.0)              # all large values in one chunk
    n = np.array([M, M, M, 7681], np.int32)
    idx, val = pmqa.select_topk(torch.from_numpy(x).cuda(), torch.from_numpy(n).cuda(), k,
                                select_workspace=ws)
    _check_rows(x, n, k, idx.cpu().numpy(), val.cpu().numpy())


@pytest.mark.parametrize("ws", WS)
def test_select_topk_long_rows(ws):
    announce(f"select_topk 131072 columns ws={ws}")
    rng = np.random.default_rng(9)
    rows, M, k = 6, 131072, 2048
    x = (rng.standard_normal((rows, M))).astype(np.float32)
    x[1] = np.float32(0.5)                         # all equal: the first k columns
    x[2, ::3] = np.float32(4.0)                    # many ties above the rest
    n = np.array([M, M, M, 70001, 2049, 2048], np.int32)
    idx, val = pmqa.select_topk(torch.from_numpy(x).cuda(), torch.from_numpy(n).cuda(), k,
                                select_workspace=ws)
    _check_rows(x, n, k, idx.cpu().numpy(), val.cpu().numpy())


@pytest.mark.parametrize("k", [1, 100, 2048, 3000])
def test_select_topk_split_rows(k):
    """The split path (rows of more than 524288 columns with a workspace):
    lengths around the chunk boundaries (chunks of 16384 columns, one chunk
    up to 16384, a last chunk of one column, 16 wider chunks from 262144),
    values with many ties at the k-th key, signed zeros and -inf.  k = 3000
    expects too long a list, so those rows are not split."""
    announce(f"select_topk split rows k={k}")
    rng = np.random.default_rng(31 + k)
    M = 600000
    lens = [7681, 8192, 8193, 9000, 16385, 65536, 131072, 131073, 200000, 262145, 600000]
    rows = len(lens) + 2
    x = rng.standard_normal((rows, M)).astype(np.float32)
    x[1] = np.round(x[1] * 64) / 64                 # ties at the k-th key
    x[2, ::5] = np.float32(-0.0)
    x[2, 1::5] = np.float32(0.0)
    x[3, ::7] = -np.inf
    x[-2] = np.round(x[-2] * 8) / 8                 # few levels: lists overflow
    x[-1] = np.linspace(-1, 1, M, dtype=np.float32)  # the largest keys in the last chunk
    n = np.array(lens + [131072, 131072], np.int32)
    buf = torch.from_numpy(x).cuda()
    lens_t = torch.from_numpy(n).cuda()
    ws = torch.empty(pmqa.select_workspace_bytes(rows, M, k), dtype=torch.uint8, device="cuda")
    idx, val = pmqa.select_topk(buf, lens_t, k, select_workspace=ws)
    _check_rows(x, n, k, idx.cpu().numpy(), val.cpu().numpy())
    thr, cnt = _split_state(ws, rows)
    split = thr != 0xFFFFFFFF
    if k == 2048:   # the plain normal rows take the split path with whole lists
        for r in (0, 4, 5, 6, 7, 8, 9, 10):
            assert split[r], r
            nch = -(-int(n[r]) // _chunk_cols(int(n[r])))
            assert 2048 <= cnt[r, :nch].sum() <= 3840, (r, cnt[r, :nch])
    if k in (1, 100):
        assert split[0] and split[10]
    if k == 3000:
        assert not split.any()


def _chunk_cols(n):
    return max(16384, -(-n // 16384) * 1024)


def _split_state(ws, rows):
    """Thresholds [rows] and chunk counts [rows, 16] the split path left in
    its workspace (sections of whole 256-byte blocks: header, chunk list,
    map, lengths, thresholds, counts, keys, columns)."""
    w = ws.view(torch.int32).cpu().numpy()
    blk = -(-rows // 64) * 64
    c16 = -(-16 * rows // 64) * 64
    t0 = 64 + c16 + 2 * blk
    thr = w[t0: t0 + rows].view(np.uint32)
    n0 = 64 + c16 + 3 * blk
    return thr, w[n0: n0 + 16 * rows].reshape(rows, 16)


def test_select_workspace_reused_across_calls():
    """One workspace for two calls in a row, the second with fewer rows and
    shorter lengths: nothing of the first call's lists leaks into it."""
    announce("select_topk workspace reuse")
    rng = np.random.default_rng(41)
    ws = torch.empty(pmqa.select_workspace_bytes(12, 100000, 2048), dtype=torch.uint8, device="cuda")
    k = 2048
    for rows, M in ((12, 100000), (5, 40000)):
        x = rng.standard_normal((rows, M)).astype(np.float32)
        n = rng.integers(M // 2, M + 1, size=rows).astype(np.int32)
        idx, val = pmqa.select_topk(torch.from_numpy(x).cuda(), torch.from_numpy(n).cuda(), k,
                                    select_workspace=ws)
        _check_rows(x, n, k, idx.cpu().numpy(), val.cpu().numpy())


def _fused(d, k, dev=None, num_workers=None, schedule=None, ws="auto"):
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
                                           k, num_workers=num_workers, select_workspace=ws)
    else:
        idx, val = pmqa.paged_mqa_topk_fp4(dev["q"], dev["q_scale"], dev["kv_cache"],
                                           dev["weights"], dev["context_lens"],
                                           dev["block_table"], schedule, M, k,
                                           num_workers=num_workers, select_workspace=ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), val.cpu().numpy()


def _row_lengths(d, rows=None):
    ctx = d["context_lens"]
    nn = int(d["next_n"])
    c = sr.units_per_row(np.maximum(ctx, 0))
    rows = range(len(ctx) * nn) if rows is None else rows
    return np.array([otk.fused_row_length(ctx[r // nn], nn, r % nn, d["max_context_len"],
                                          c[r // nn]) for r in rows])


@pytest.mark.parametrize("ws", WS)
@pytest.mark.parametrize("variant", ["fp8", "fp4"])
@pytest.mark.parametrize("next_n", [1, 2])
def test_fused_topk_against_oracle(variant, next_n, ws):
    announce(f"fused top-k {variant} next_n={next_n} ws={ws}")
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
        idx, val = _fused(d, k, ws=ws)
        parity.check_topk(idx, val, ref, _row_lengths(d), k, f"{variant} k={k}")


@pytest.mark.parametrize("variant", ["fp8", "fp4"])
@pytest.mark.parametrize("next_n", [1, 2])
def test_fused_topk_split_rows(variant, next_n):
    """Rows of more than 6144 candidates (a workgroup each) beside shorter
    rows (a wavefront each) in the fused step, whose candidate counts come
    from the schedule."""
    announce(f"fused top-k split rows {variant} next_n={next_n}")
    ctx = np.array([0, 7700, 8193, 20000, 33000, 5000, 41000, 1], np.int64)
    mk = make_fp8 if variant == "fp8" else make_fp4
    d = mk(ctx, next_n=next_n, max_context_len=40000, seed=50 + next_n,
           bt_stride=-(-41000 // 64))
    ref = oracle(d)
    dev = upload(d)
    nn, M = int(d["next_n"]), int(d["max_context_len"])
    lens = torch.from_numpy(_row_lengths(d).astype(np.int32)).cuda()
    for k in (64, 2048):
        idx, val = _fused(d, k)
        parity.check_topk(idx, val, ref, _row_lengths(d), k, f"{variant} k={k}")
        # the same logits, selected by the single-kernel path: bit for bit
        logits = torch.empty((len(ctx) * nn, M), device="cuda")
        sched = pmqa.compute_schedule(dev["context_lens"], next_n=nn,
                                      variant=pmqa.VARIANT_FP8 if variant == "fp8"
                                      else pmqa.VARIANT_FP4)
        if variant == "fp8":
            i2, v2 = pmqa.paged_mqa_topk_fp8(dev["q"], dev["kv_cache"], dev["weights"],
                                             dev["context_lens"], dev["block_table"], sched, M,
                                             k, workspace=logits)
        else:
            i2, v2 = pmqa.paged_mqa_topk_fp4(dev["q"], dev["q_scale"], dev["kv_cache"],
                                             dev["weights"], dev["context_lens"],
                                             dev["block_table"], sched, M, k, workspace=logits)
        i1, v1 = pmqa.select_topk(logits, lens, k, select_workspace=None)
        assert torch.equal(i1, i2) and torch.equal(v1.view(torch.int32), v2.view(torch.int32))
        assert np.array_equal(idx, i2.cpu().numpy())


def test_fused_topk_mismatched_schedule_selects_nothing():
    announce("fused top-k, foreign schedule")
    d = make_fp8([100, 300], max_context_len=400, seed=23)
    dev = upload(d)
    sched = pmqa.compute_schedule(dev["context_lens"], num_workers=16)
    idx, val = _fused(d, 8, dev=dev, num_workers=8, schedule=sched)
    assert np.all(idx == -1) and np.all(np.isneginf(val))
