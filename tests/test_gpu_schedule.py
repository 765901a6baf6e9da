"""GPU schedule (compute_schedule) against the oracle partition, exactly."""
import numpy as np
import pytest
import torch

from gpu_util import announce
from oracle import schedule_ref as sr

pytestmark = pytest.mark.gpu
pmqa = pytest.importorskip("paged_mqa_logits_amd")


def _check(ctx, W):
    announce(f"schedule B={len(ctx)} W={W}")
    t = torch.from_numpy(np.asarray(ctx, np.int32)).cuda()
    s = pmqa.compute_schedule(t, num_workers=W).cpu().numpy()
    B = len(ctx)
    c = sr.units_per_row(np.maximum(np.asarray(ctx), 0))
    starts = sr.starts_binary(c, W)
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


@pytest.mark.parametrize("ctx,W", _cases())
def test_schedule_matches_oracle(ctx, W):
    _check(ctx, W)


def test_schedule_large_batch_multi_rows_per_thread():
    rng = np.random.default_rng(1)
    ctx = rng.integers(0, 5000, size=70000)
    ctx[::3] = 0
    _check(ctx.tolist(), 2048)


def test_schedule_negative_lengths_count_as_zero():
    _check([5, -3, 700], 4)
