"""Graph capture of [compute_schedule, logits] and validate mode."""
import os

import numpy as np
import pytest
import torch

import parity
from gpu_util import announce, oracle, upload
from workloads import make_fp8

pytestmark = pytest.mark.gpu
pmqa = pytest.importorskip("paged_mqa_logits_amd")


@pytest.mark.parametrize("mode", ["compute", "refresh"])
def test_graph_replay_tracks_context_lengths(mode):
    """Capture schedule + logits once; each step updates context_lens in place
    (some rows cross a 256-token boundary) and replays.  Every replay must
    match the oracle for that step's lengths.  Eager work and synchronizations
    sit between replays.  In refresh mode the schedule is rebuilt on the
    device only on the steps where some row's unit count changed."""
    announce(f"graph replay ({mode})")
    B, M = 24, 2048
    rng = np.random.default_rng(80)
    ctx0 = rng.integers(0, 1700, size=B).astype(np.int32)
    ctx0[[0, 5, 9]] = 0
    ctx0[3] = 255                      # crosses 256 at the first step
    ctx0[7] = 511
    d = make_fp8(ctx0 + 300, max_context_len=M, seed=80)   # pages for every step
    dev = upload(d)
    ctx_t = torch.from_numpy(ctx0.copy()).cuda()
    W = pmqa.default_num_workers()
    sched = torch.empty(pmqa.schedule_bytes(B, W) // 4, dtype=torch.int32, device="cuda")
    out = torch.empty((B, M), dtype=torch.float32, device="cuda")

    flag = torch.full((1,), -1, dtype=torch.int32, device="cuda")

    def step():
        if mode == "compute":
            pmqa.compute_schedule(ctx_t, num_workers=W, out=sched)
        else:
            pmqa.refresh_schedule(ctx_t, sched, num_workers=W, recomputed=flag)
        pmqa.paged_mqa_logits_fp8(dev["q"], dev["kv_cache"], dev["weights"], ctx_t,
                                  dev["block_table"], sched, M, out=out, num_workers=W)

    step()                              # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    ctx = ctx0.copy()
    rebuilt = 0
    for it in range(6):
        prev = ctx.copy()
        if it:
            grow = np.where(ctx > 0, 1 + 37 * (it % 2), 0).astype(np.int32)
            ctx = ctx + grow
        ctx_t.copy_(torch.from_numpy(ctx))
        out.fill_(7.0)                  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        ref = oracle(dict(d, context_lens=ctx))
        parity.check(got, ref, f"replay {it}")
        if mode == "refresh":
            crossed = bool(np.any((ctx + 255) // 256 != (prev + 255) // 256))
            assert int(flag.item()) == int(crossed), it
            rebuilt += crossed
    assert mode == "compute" or 0 < rebuilt < 6


def test_graph_replay_fused_topk_with_split_workspace():
    """Capture schedule + fused top-k with the split workspace (plan, gather
    and selection kernels); lengths change in place between replays (rows
    long enough to be split, some crossing chunk boundaries).  Every replay
    must equal an eager call on the same lengths, bit for bit, and be a
    selection the fp64 oracle accepts for that step's lengths."""
    announce("graph replay fused top-k (split workspace)")
    B, M, k = 6, 40000, 2048
    ctx0 = np.array([9000, 0, 16300, 30000, 7000, 38000], np.int32)
    d = make_fp8(ctx0 + 3000, max_context_len=M, seed=81)   # pages for every step
    dev = upload(d)
    ctx_t = torch.from_numpy(ctx0.copy()).cuda()
    W = pmqa.default_num_workers()
    sched = torch.empty(pmqa.schedule_bytes(B, W) // 4, dtype=torch.int32, device="cuda")
    logits = torch.empty((B, M), dtype=torch.float32, device="cuda")
    sws = torch.empty(pmqa.select_workspace_bytes(B, M, k), dtype=torch.uint8, device="cuda")
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    val = torch.empty((B, k), dtype=torch.float32, device="cuda")

    def step(i, v, ws):
        pmqa.compute_schedule(ctx_t, num_workers=W, out=sched)
        pmqa.paged_mqa_topk_fp8(dev["q"], dev["kv_cache"], dev["weights"], ctx_t,
                                dev["block_table"], sched, M, k, workspace=logits, indices=i,
                                values=v, num_workers=W, select_workspace=ws)

    step(idx, val, sws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step(idx, val, sws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    ctx = ctx0.copy()
    for it in range(5):
        if it:
            ctx = ctx + np.where(ctx > 0, 250 * it, 0).astype(np.int32)
        ctx_t.copy_(torch.from_numpy(ctx))
        idx.fill_(-7)                   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        got_i, got_v = idx.clone(), val.clone()
        ei = torch.empty_like(idx)
        ev = torch.empty_like(val)
        step(ei, ev, None)              # eager, single-kernel selection
        torch.cuda.synchronize()
        assert torch.equal(got_i, ei), it
        assert torch.equal(got_v.view(torch.int32), ev.view(torch.int32)), it
        # against the oracle: every unit of a row is scheduled, so a row's
        # candidates are its first min(ctx, M) columns
        ref = oracle(dict(d, context_lens=ctx))
        n = np.clip(ctx.astype(np.int64), 0, M)
        parity.check_topk(got_i.cpu().numpy(), got_v.cpu().numpy(), ref, n, k,
                          f"top-k replay {it}")


def test_validate_mode_detects_stale_schedule(monkeypatch):
    announce("validate: stale schedule")
    d = make_fp8([100, 250, 0], max_context_len=600, seed=81)
    dev = upload(d)
    sched = pmqa.compute_schedule(dev["context_lens"])
    monkeypatch.setenv("PMQA_VALIDATE_INPUTS", "1")
    pmqa.paged_mqa_logits_fp8(dev["q"], dev["kv_cache"], dev["weights"], dev["context_lens"],
                              dev["block_table"], sched, 600)
    # within the same 256-token unit: still valid
    dev["context_lens"].copy_(torch.tensor([120, 256, 0], dtype=torch.int32))
    pmqa.paged_mqa_logits_fp8(dev["q"], dev["kv_cache"], dev["weights"], dev["context_lens"],
                              dev["block_table"], sched, 600)
    # row 1 crosses 256 -> stale
    dev["context_lens"].copy_(torch.tensor([120, 257, 0], dtype=torch.int32))
    with pytest.raises(pmqa.PmqaError) as ei:
        pmqa.paged_mqa_logits_fp8(dev["q"], dev["kv_cache"], dev["weights"],
                                  dev["context_lens"], dev["block_table"], sched, 600)
    assert ei.value.status_name == "PMQA_ERR_STALE_SCHEDULE"
    torch.cuda.synchronize()


def test_validate_mode_detects_bad_page_and_length(monkeypatch):
    announce("validate: bad values")
    d = make_fp8([100, 70], max_context_len=200, seed=82)
    dev = upload(d)
    sched = pmqa.compute_schedule(dev["context_lens"])
    monkeypatch.setenv("PMQA_VALIDATE_INPUTS", "1")
    bt = dev["block_table"].clone()
    bt[1, 1] = d["kv_cache"].shape[0]            # one past the last page
    with pytest.raises(pmqa.PmqaError) as ei:
        pmqa.paged_mqa_logits_fp8(dev["q"], dev["kv_cache"], dev["weights"],
                                  dev["context_lens"], bt, sched, 200)
    assert ei.value.status_name == "PMQA_ERR_INVALID_VALUE"
    ctx = torch.tensor([100, -1], dtype=torch.int32, device="cuda")
    with pytest.raises(pmqa.PmqaError) as ei:
        pmqa.paged_mqa_logits_fp8(dev["q"], dev["kv_cache"], dev["weights"], ctx,
                                  dev["block_table"], sched, 200)
    assert ei.value.status_name == "PMQA_ERR_INVALID_VALUE"
    torch.cuda.synchronize()


def test_validate_mode_refuses_capturing_stream(monkeypatch):
    announce("validate: capturing stream")
    d = make_fp8([100, 70], max_context_len=200, seed=83)
    dev = upload(d)
    sched = pmqa.compute_schedule(dev["context_lens"])
    out = torch.empty((2, 200), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    monkeypatch.setenv("PMQA_VALIDATE_INPUTS", "1")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    err = None
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            try:
                pmqa.paged_mqa_logits_fp8(dev["q"], dev["kv_cache"], dev["weights"],
                                          dev["context_lens"], dev["block_table"], sched, 200,
                                          out=out)
            except pmqa.PmqaError as e:
                err = e
    torch.cuda.synchronize()
    assert err is not None and err.status_name == "PMQA_ERR_CAPTURING"


def test_invalid_schedule_header_writes_only_neg_inf():
    """A schedule built for another worker count is not used: the call writes
    -inf everywhere instead of reading outside the schedule."""
    announce("mismatched schedule")
    d = make_fp8([100, 300], max_context_len=400, seed=84)
    dev = upload(d)
    sched = pmqa.compute_schedule(dev["context_lens"], num_workers=16)
    out = pmqa.paged_mqa_logits_fp8(dev["q"], dev["kv_cache"], dev["weights"],
                                    dev["context_lens"], dev["block_table"], sched, 400,
                                    num_workers=8)
    torch.cuda.synchronize()
    assert np.all(out.cpu().numpy().view(np.uint32) == parity.NEG_INF_BITS)
