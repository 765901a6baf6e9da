"""GPU parity of paged_mqa_logits_fp8 / _fp4 against the fp64 oracle."""
import numpy as np
import pytest
import torch

import golden_fixtures as gf
import parity
from gpu_util import announce, oracle, run, upload
from workloads import CONFIGS, make_fp4, make_fp8, make_workload

pytestmark = pytest.mark.gpu
pmqa = pytest.importorskip("paged_mqa_logits_amd")


# ---------------------------------------------------------------- fixtures

@pytest.mark.parametrize("case", [0, 1])
def test_hand_fixture_fp8(case):
    announce(f"hand fixture fp8 case {case}")
    e = gf.embed_fp8(gf.load_fp8(case))
    e["variant"] = "fp8"
    lg, _ = run(e)
    assert np.array_equal(lg.astype(np.float64), e["expected"]), lg


def test_hand_fixture_fp4():
    announce("hand fixture fp4")
    e = gf.embed_fp4(gf.load_fp4())
    e["variant"] = "fp4"
    lg, _ = run(e)
    assert np.array_equal(lg.astype(np.float64), e["expected"]), lg


# ---------------------------------------------------------------- full compare

EDGE_CTX = [0, 1, 2, 63, 64, 65, 127, 255, 256, 257, 300, 511, 512, 513, 700, 1000, 1023, 1024]


@pytest.mark.parametrize("next_n", [1, 2])
@pytest.mark.parametrize("negative_scales", [False, True])
def test_fp8_edge_lengths(next_n, negative_scales):
    announce(f"fp8 edge lengths nn={next_n} neg={negative_scales}")
    d = make_fp8(EDGE_CTX, next_n=next_n, max_context_len=1024, seed=21 + next_n,
                 negative_scales=negative_scales)
    lg, _ = run(d)
    parity.check(lg, oracle(d), "fp8 edge")


@pytest.mark.parametrize("next_n", [1, 2])
def test_fp4_edge_lengths(next_n):
    announce(f"fp4 edge lengths nn={next_n}")
    d = make_fp4(EDGE_CTX, next_n=next_n, max_context_len=1024, seed=31 + next_n)
    lg, _ = run(d)
    parity.check(lg, oracle(d), "fp4 edge")


def test_tiny_config():
    announce("tiny_fp8 config")
    d = make_workload("tiny_fp8")
    lg, _ = run(d)
    parity.check(lg, oracle(d), "tiny_fp8")


@pytest.mark.parametrize("M", [1, 5, 100, 255, 257, 1000])
def test_fp8_truncation_and_odd_widths(M):
    announce(f"fp8 truncation M={M}")
    d = make_fp8([0, 3, 200, 900, 1100], next_n=1, max_context_len=M, seed=40 + M,
                 bt_stride=-(-1100 // 64))
    lg, _ = run(d)
    parity.check(lg, oracle(d), f"trunc M={M}")


def test_zero_rows_interleaved_at_worker_boundaries():
    """Zero-length rows between every non-empty row and many workers, so that
    worker ranges start right after skipped rows."""
    announce("zero rows interleaved")
    ctx = []
    for i in range(40):
        ctx += [0, 0, 256 * (i % 3) + 17 * i + 1]
    d = make_fp8(ctx, max_context_len=1024, seed=50)
    ref = oracle(d)
    for W in (1, 5, 37, 128, 1000):
        lg, _ = run(d, num_workers=W)
        parity.check(lg, ref, f"zero rows W={W}")


def test_all_rows_empty():
    announce("all rows empty")
    d = make_fp8([0, 0, 0, 0], max_context_len=300, seed=51)
    lg, _ = run(d)
    assert np.all(lg.view(np.uint32) == parity.NEG_INF_BITS)


def test_mid_config_full():
    announce("mid_fp8 config (full compare)")
    d = make_workload("mid_fp8")
    lg, _ = run(d)
    parity.check(lg, oracle(d), "mid_fp8")


def test_fp4_small_full():
    announce("fp4 small full compare")
    rng = np.random.default_rng(60)
    ctx = rng.integers(0, 5000, size=24)
    ctx[::5] = 0
    d = make_fp4(ctx, max_context_len=5000, seed=60)
    lg, _ = run(d)
    parity.check(lg, oracle(d), "fp4 small")


def test_tail_columns_covered():
    """Every column is written, by the -inf fill or by a unit: truncated rows
    (context past max_context_len), a width that is not a multiple of 4 or
    256, two query rows per batch row, several worker counts, on a poisoned
    output."""
    announce("tail coverage")
    rng = np.random.default_rng(74)
    M = 1001
    ctx = rng.integers(0, 1600, size=300)
    ctx[rng.random(300) < 0.2] = 0
    ctx[::17] = M + 300
    d = make_fp8(ctx, next_n=2, max_context_len=M, seed=74, bt_stride=-(-1900 // 64))
    ref = oracle(d)
    dev = upload(d)
    for W in (1, 7, 1024):
        lg, _ = run(d, dev=dev, num_workers=W)
        parity.check(lg, ref, f"tail coverage W={W}")


def test_tail_fill_pieces():
    """Small outputs get their -inf past the units from the unit kernel's
    workers, R output rows dealt out in W // R pieces: R == W, R < W with
    idle workers, many pieces per row, and R > W (the separate fill), on a
    poisoned output of a width that is not a multiple of 4."""
    announce("in-kernel tail fill pieces")
    M = 1001
    ctx = np.array([0, 300, 1001, 1500, 17], np.int64)
    d = make_fp8(ctx, next_n=2, max_context_len=M, seed=76, bt_stride=-(-1500 // 64))
    ref = oracle(d)
    dev = upload(d)
    for W in (10, 11, 37, 1024, 9):
        lg, _ = run(d, dev=dev, num_workers=W)
        parity.check(lg, ref, f"tail fill W={W}")


def test_large_batch_of_short_rows():
    """16385 batch rows, most of them empty: the schedule's prefix sums no
    longer fit its LDS table and are searched in global memory."""
    announce("batch 16385 short rows")
    rng = np.random.default_rng(75)
    ctx = rng.integers(1, 300, size=16385)
    ctx[rng.random(16385) < 0.9] = 0
    d = make_fp8(ctx, next_n=1, max_context_len=299, seed=75)
    lg, _ = run(d)
    parity.check(lg, oracle(d), "batch 16385")


@pytest.mark.parametrize("variant", ["fp8", "fp4"])
@pytest.mark.parametrize("next_n", [1, 2])
@pytest.mark.parametrize("heads", [32, 16])
def test_fewer_heads(variant, next_n, heads):
    """Query blocks of 32 and 16 heads (the kernels with 2 and 1 head groups)."""
    announce(f"{variant} heads={heads} next_n={next_n}")
    rng = np.random.default_rng(76 + heads + next_n)
    ctx = rng.integers(0, 2500, size=30)
    ctx[::7] = 0
    ctx[1] = 1
    ctx[2] = 2600                                   # truncated
    mk = make_fp8 if variant == "fp8" else make_fp4
    kw = dict(negative_scales=True) if variant == "fp8" else {}
    d = mk(ctx, next_n=next_n, max_context_len=2500, seed=76 + heads, num_heads=heads,
           bt_stride=-(-2600 // 64), **kw)
    ref = oracle(d)
    for W in (None, 7):
        lg, _ = run(d, num_workers=W)
        parity.check(lg, ref, f"{variant} H={heads} NN={next_n} W={W}")


# ---------------------------------------------------------------- self-consistency

def test_worker_count_invariance_and_determinism():
    announce("worker-count invariance")
    rng = np.random.default_rng(70)
    ctx = rng.integers(0, 3000, size=50)
    ctx[rng.random(50) < 0.3] = 0
    d = make_fp8(ctx, next_n=2, max_context_len=3000, seed=70)
    dev = upload(d)
    base, _ = run(d, dev=dev)
    again, _ = run(d, dev=dev)
    assert np.array_equal(base.view(np.uint32), again.view(np.uint32))
    for W in (1, 37, 256, 1024, 8192):
        lg, _ = run(d, dev=dev, num_workers=W)
        assert np.array_equal(base.view(np.uint32), lg.view(np.uint32)), W


def test_weight_doubling_is_exact():
    announce("weights x2")
    d = make_fp8([500, 70, 0, 1000], max_context_len=1000, seed=71)
    base, _ = run(d)
    d2 = dict(d, weights=(2 * d["weights"]).astype(np.float32))
    twice, _ = run(d2)
    assert np.array_equal(twice, 2 * base)


def test_page_permutation_invariance():
    announce("page permutation")
    d = make_fp8([900, 333, 64, 0, 1024], next_n=2, max_context_len=1024, seed=72)
    rng = np.random.default_rng(72)
    perm = rng.permutation(d["kv_cache"].shape[0])
    kv = np.empty_like(d["kv_cache"])
    kv[perm] = d["kv_cache"]
    d2 = dict(d, kv_cache=kv, block_table=perm[d["block_table"]].astype(np.int32))
    a, _ = run(d)
    b, _ = run(d2)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("variant", ["fp8", "fp4"])
def test_row_permutation_equivariance(variant):
    """Batch rows permuted together with their context lengths, block-table
    rows, queries and weights give the same output rows, permuted, bit for
    bit: zero-length rows (interleaved, so the permutation moves them across
    worker boundaries) are skipped by the same rule wherever they sit, and a
    row's values do not depend on which worker scores it."""
    announce(f"row permutation {variant}")
    rng = np.random.default_rng(78)
    ctx = rng.integers(1, 2000, size=48)
    ctx[::3] = 0
    ctx[4] = 1
    ctx[7] = 2100                                   # truncated
    nn = 2
    mk = make_fp8 if variant == "fp8" else make_fp4
    kw = dict(negative_scales=True) if variant == "fp8" else {}
    d = mk(ctx, next_n=nn, max_context_len=2048, seed=78, bt_stride=-(-2100 // 64), **kw)
    B = len(ctx)
    perm = rng.permutation(B)
    d2 = dict(d, context_lens=d["context_lens"][perm].copy(),
              block_table=d["block_table"][perm].copy(), q=d["q"][perm].copy(),
              weights=d["weights"].reshape(B, nn, -1)[perm].reshape(B * nn, -1).copy())
    if "q_scale" in d:
        d2["q_scale"] = d["q_scale"][perm].copy()
    rows = (perm[:, None] * nn + np.arange(nn)[None, :]).reshape(-1)
    for W in (None, 37, 5):
        a, _ = run(d, num_workers=W)
        b, _ = run(d2, num_workers=W)
        assert np.array_equal(b.view(np.uint32), a[rows].view(np.uint32)), W
    parity.check(a, oracle(d), f"row permutation {variant}")


def test_columns_past_max_context_untouched():
    announce("guard columns")
    d = make_fp8([100, 0, 300], next_n=2, max_context_len=301, seed=73)
    dev = upload(d)
    out = torch.full((6, 320), 12345.0, dtype=torch.float32, device="cuda")
    sched = pmqa.compute_schedule(dev["context_lens"])
    pmqa.paged_mqa_logits_fp8(dev["q"], dev["kv_cache"], dev["weights"], dev["context_lens"],
                              dev["block_table"], sched, 301, out=out)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[:, 301:] == 12345.0)
    parity.check(o[:, :301], oracle(d), "guard")


# ---------------------------------------------------------------- full sizes

def _sample_rows(d, k, seed):
    ctx = d["context_lens"]
    nn = d["next_n"]
    B = len(ctx)
    rng = np.random.default_rng(seed)
    picks = set(rng.choice(B, size=min(k, B), replace=False).tolist())
    picks |= {int(np.argmax(ctx)), int(np.argmin(ctx)), 0, B - 1}
    zero = np.nonzero(ctx == 0)[0]
    if len(zero):
        picks.add(int(zero[0]))
    return sorted(r for b in picks for r in range(b * nn, b * nn + nn))


@pytest.mark.timeout(400)
@pytest.mark.parametrize("variant,next_n", [("fp8", 1), ("fp4", 1), ("fp8", 2)])
def test_million_token_row(variant, next_n):
    """A context of 2^20 tokens (4096 units, 16384 pages) next to a shorter
    and an empty row, max_context_len 2^20: every element against the
    oracle, and the fused top-k (k = 2048, the split path with 16 chunks of
    65536 columns) against the same oracle logits."""
    announce(f"2^20-token row {variant} next_n={next_n}")
    M = 1 << 20
    ctx = np.array([M, 70001, 0])
    mk = make_fp8 if variant == "fp8" else make_fp4
    d = mk(ctx, next_n=next_n, max_context_len=M, seed=77)
    ref = oracle(d)
    lg, _ = run(d)
    parity.check(lg, ref, "2^20 row")
    dev = upload(d)
    vt = pmqa.VARIANT_FP8 if variant == "fp8" else pmqa.VARIANT_FP4
    sched = pmqa.compute_schedule(dev["context_lens"], variant=vt, next_n=next_n)
    if variant == "fp8":
        idx, val = pmqa.paged_mqa_topk_fp8(dev["q"], dev["kv_cache"], dev["weights"],
                                           dev["context_lens"], dev["block_table"], sched, M,
                                           2048)
    else:
        idx, val = pmqa.paged_mqa_topk_fp4(dev["q"], dev["q_scale"], dev["kv_cache"],
                                           dev["weights"], dev["context_lens"],
                                           dev["block_table"], sched, M, 2048)
    # candidates of row b*next_n + j: its causal limit (every unit is scheduled)
    n = np.clip(np.repeat(ctx, next_n) - next_n + 1 + np.tile(np.arange(next_n), len(ctx)), 0, M)
    parity.check_topk(idx.cpu().numpy(), val.cpu().numpy(), ref, n, 2048, "2^20 row top-k")


def _fused_topk(d, dev, k):
    """The fused indexer step at the default worker count: (indices, values)."""
    nn = int(d["next_n"])
    M = int(d["max_context_len"])
    if d["variant"] == "fp8":
        sched = pmqa.compute_schedule(dev["context_lens"], next_n=nn,
                                      num_heads=int(d["q"].shape[2]))
        idx, val = pmqa.paged_mqa_topk_fp8(dev["q"], dev["kv_cache"], dev["weights"],
                                           dev["context_lens"], dev["block_table"], sched, M, k)
    else:
        sched = pmqa.compute_schedule(dev["context_lens"], variant=pmqa.VARIANT_FP4, next_n=nn,
                                      num_heads=int(d["q"].shape[2]))
        idx, val = pmqa.paged_mqa_topk_fp4(dev["q"], dev["q_scale"], dev["kv_cache"],
                                           dev["weights"], dev["context_lens"],
                                           dev["block_table"], sched, M, k)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), val.cpu().numpy()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["large_fp8", "spec_fp8", "mxfp4", "large_fp8_h16"])
def test_full_size_config_all_rows(name):
    """Full configuration in the launch configuration the benchmark times
    (default worker count): every output row against the oracle, element by
    element (the oracle run in chunks of rows to bound host memory), and the
    fused top-k (k = 2048) of every row against the same oracle rows."""
    announce(f"{name} full size (every row)")
    d = make_workload(name)
    dev = upload(d)
    lg, _ = run(d, dev=dev)
    k = 2048
    idx, val = _fused_topk(d, dev, k)
    del dev
    torch.cuda.empty_cache()
    nn = int(d["next_n"])
    M = int(d["max_context_len"])
    ctx = d["context_lens"].astype(np.int64)
    c = -(-np.maximum(ctx, 0) // 256)
    R = len(ctx) * nn
    # fused candidates: causal limit, within the scheduled units and M
    lim = np.repeat(ctx, nn) - nn + 1 + np.tile(np.arange(nn), len(ctx))
    n = np.clip(np.minimum(lim, 256 * np.repeat(c, nn)), 0, M)
    chunk = max(nn, (1 << 23) // M // nn * nn)      # ~32 MB of fp32 logits per chunk
    masked = checked = 0
    worst = 0.0
    for r0 in range(0, R, chunk):
        rows = list(range(r0, min(R, r0 + chunk)))
        ref = oracle(d, rows=rows)
        st = parity.check(lg[r0:r0 + len(rows)], ref, f"{name} rows {r0}..")
        parity.check_topk(idx[r0:r0 + len(rows)], val[r0:r0 + len(rows)], ref,
                          n[r0:r0 + len(rows)], k, f"{name} top-k rows {r0}..")
        masked += st["masked"]
        checked += st["checked"]
        worst = max(worst, st["max_err_over_tol"])
        print(f"[gpu-case] {name}: rows {r0}..{r0 + len(rows) - 1} of {R} match", flush=True)
    assert masked + checked == R * M
    print(f"[gpu-case] {name}: {R} rows, {checked} scores within tolerance "
          f"(max |err|/tol {worst:.3g}), {masked} masked entries exact; "
          f"top-k k={k} of every row checked", flush=True)
