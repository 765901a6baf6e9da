"""GPU schedules (compute_schedule, compute_schedule_linear, refresh_schedule)
against the oracle partition, exactly."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_util import announce
from oracle import schedule_ref as sr

pytestmark = pytest.mark.gpu
pmqa = pytest.importorskip("paged_mqa_logits_amd")


def _check(ctx, W, linear=False):
    announce(f"schedule B={len(ctx)} W={W} linear={linear}")
    t = torch.from_numpy(np.asarray(ctx, np.int32)).cuda()
    fn = pmqa.compute_schedule_linear if linear else pmqa.compute_schedule
    s = fn(t, num_workers=W).cpu().numpy()
    B = len(ctx)
    c = sr.units_per_row(np.maximum(np.asarray(ctx), 0))
    # the oracle's linear scan on small cases; its binary search (pinned equal
    # to the linear scan on the CPU) where the scan would take too long
    small = linear and B * (W + 1) <= 2_000_000
    starts = sr.starts_linear(c, W) if small else sr.starts_binary(c, W)
    S = sr.prefix_sums(c)
    assert s[0] == pmqa.SCHED_MAGIC and s[1] == B and s[2] == W and s[3] == S[-1] and s[4] == 256
    got = [(int(s[8 + 2 * w]), int(s[9 + 2 * w])) for w in range(W + 1)]
    assert got == starts
    assert s[8 + 2 * (W + 1):].tolist() == S
    assert len(s) == pmqa.schedule_bytes(B, W) // 4


def _cases():
    rng = np.random.default_rng(0)
    out = [([0, 0, 0], 4), ([1], 1), ([300], 5), ([0, 1, 0, 256, 257, 0], 7)]
    for B, W in [(7, 3), (64, 37), (2048, 256), (2048, 3072), (5000, 1), (1500, 4096)]:
        ctx = rng.integers(0, 40000, size=B)
        ctx[rng.random(B) < 0.2] = 0
        out.append((ctx.tolist(), W))
    return out


@pytest.mark.parametrize("linear", [False, True])
@pytest.mark.parametrize("ctx,W", _cases())
def test_schedule_matches_oracle(ctx, W, linear):
    _check(ctx, W, linear)


@pytest.mark.parametrize("linear", [False, True])
def test_schedule_large_batch_multi_rows_per_thread(linear):
    rng = np.random.default_rng(1)
    ctx = rng.integers(0, 5000, size=70000)
    ctx[::3] = 0
    _check(ctx.tolist(), 2048, linear)


@pytest.mark.parametrize("linear", [False, True])
def test_schedule_negative_lengths_count_as_zero(linear):
    _check([5, -3, 700], 4, linear)


# ---------------------------------------------------------------- refresh_schedule

def _refresh(ctx_t, sched, W):
    flag = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    pmqa.refresh_schedule(ctx_t, sched, num_workers=W, recomputed=flag)
    torch.cuda.synchronize()
    return int(flag.item())


def _fresh(ctx_t, W):
    return pmqa.compute_schedule(ctx_t, num_workers=W).cpu().numpy()


@pytest.mark.parametrize("B,W", [(37, 5), (2048, 1024), (13000, 300)])
def test_refresh_rebuilds_garbage(B, W):
    announce(f"refresh garbage B={B} W={W}")
    rng = np.random.default_rng(90 + B)
    ctx = rng.integers(0, 20000, size=B).astype(np.int32)
    ctx[rng.random(B) < 0.2] = 0
    ctx_t = torch.from_numpy(ctx).cuda()
    words = pmqa.schedule_bytes(B, W) // 4
    sched = torch.from_numpy(rng.integers(-2**31, 2**31 - 1, size=words, dtype=np.int64)
                             .astype(np.int32)).cuda()
    assert _refresh(ctx_t, sched, W) == 1
    assert np.array_equal(sched.cpu().numpy(), _fresh(ctx_t, W))


def test_refresh_keeps_a_fresh_schedule_untouched():
    """A matching schedule is not rewritten: words that only a rebuild would
    overwrite (planted in the worker starts) survive, growth inside a 256-token
    unit keeps it, growth across a boundary rebuilds it."""
    announce("refresh keep / rebuild")
    rng = np.random.default_rng(91)
    B, W = 300, 64
    ctx = rng.integers(0, 5000, size=B).astype(np.int32)
    ctx[::7] = 0
    ctx[5] = 256 * 3 - 10
    ctx_t = torch.from_numpy(ctx).cuda()
    sched = pmqa.compute_schedule(ctx_t, num_workers=W)
    planted = sched.clone()
    planted[pmqa.SCHED_HEADER:pmqa.SCHED_HEADER + 2 * (W + 1)] = 12345
    sched.copy_(planted)
    assert _refresh(ctx_t, sched, W) == 0
    assert torch.equal(sched, planted)
    ctx[5] += 10                                   # 768: still 3 units
    ctx[8] = ctx[8] + 1 if ctx[8] % 256 else ctx[8]  # never crosses a boundary
    ctx_t.copy_(torch.from_numpy(ctx))
    assert _refresh(ctx_t, sched, W) == 0
    assert torch.equal(sched, planted)
    ctx[5] += 1                                    # 769: 4 units
    ctx_t.copy_(torch.from_numpy(ctx))
    assert _refresh(ctx_t, sched, W) == 1
    assert np.array_equal(sched.cpu().numpy(), _fresh(ctx_t, W))
    ctx[0] = 0 if ctx[0] else 1                    # a row appears or vanishes
    ctx_t.copy_(torch.from_numpy(ctx))
    assert _refresh(ctx_t, sched, W) == 1
    assert np.array_equal(sched.cpu().numpy(), _fresh(ctx_t, W))


def test_refresh_rebuilds_for_another_worker_count():
    announce("refresh other W")
    ctx = torch.tensor([700, 0, 3000, 12], dtype=torch.int32, device="cuda")
    big = torch.zeros(pmqa.schedule_bytes(4, 16) // 4, dtype=torch.int32, device="cuda")
    pmqa.compute_schedule(ctx, num_workers=16, out=big)
    assert _refresh(ctx, big, 16) == 0
    # the raw C entry point accepts a larger buffer; the binding does not
    lib = pmqa.library()
    st = lib.compute_schedule(ctypes.c_void_p(ctx.data_ptr()), 4, 8,
                              ctypes.c_void_p(big.data_ptr()),
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0                                   # header now says W = 8
    assert _refresh(ctx, big, 16) == 1
    assert np.array_equal(big.cpu().numpy(), _fresh(ctx, 16))


def test_binding_refuses_a_schedule_buffer_of_another_size():
    """A schedule buffer sized for 16 workers used for 8 would later be read
    by the logits wrappers as a 16-worker schedule: the binding refuses it,
    and the logits wrappers infer the worker count only from exact sizes."""
    announce("schedule buffer size")
    ctx = torch.tensor([700, 0, 3000, 12], dtype=torch.int32, device="cuda")
    big = torch.zeros(pmqa.schedule_bytes(4, 16) // 4, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="needs exactly"):
        pmqa.compute_schedule(ctx, num_workers=8, out=big)
    with pytest.raises(ValueError, match="needs exactly"):
        pmqa.refresh_schedule(ctx, big, num_workers=8)
    with pytest.raises(ValueError, match="needs exactly"):
        pmqa.compute_schedule_linear(ctx, num_workers=8, out=big)
    s8 = pmqa.compute_schedule(ctx, num_workers=8)
    assert pmqa.sched_workers(s8.numel(), 4) == 8


def test_num_workers_is_the_fp8_decode_grid():
    """pmqa_num_workers(device): the persistent grid of the fp8 batch-decode
    kernel, the same count pmqa_default_num_workers gives for (fp8, next_n 1,
    64 heads): three quarters of a multiple of the compute units, times 4
    wavefronts per workgroup (the MXFP4 grid keeps every workgroup)."""
    announce("pmqa_num_workers")
    w = pmqa.num_workers()
    assert w == pmqa.default_num_workers(pmqa.VARIANT_FP8, 1, num_heads=64)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert w % (3 * cus) == 0 and w >= 3 * cus
    w4 = pmqa.default_num_workers(pmqa.VARIANT_FP4, 1, num_heads=64)
    assert w4 % (4 * cus) == 0 and w4 >= 4 * cus
    assert pmqa.library().pmqa_num_workers(torch.cuda.current_device()) == w
