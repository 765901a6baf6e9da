"""Byte offsets past 4 GiB on every pointer the kernels index: a K cache
whose used pages all lie above 4 GiB (the space below full of 0xFF bytes,
NaN in E4M3 and in E8M0), and logits rows 1 GiB apart, so that rows 4 and 5
start past 4 GiB.  Moving pages to other ids and spacing the output rows
change no logit (the page's problem statement: the block table names each
row's pages; the output is a row per query), so the oracle runs on the
inputs as generated.  Covers the -inf fill (strided rows), the unit
kernel's stores, the fused top-k's unit kernel and selection, and
select_topk on the same strided rows."""
import numpy as np
import pytest
import torch

import parity
from gpu_util import announce, oracle, upload
from oracle import schedule_ref as sr
from oracle import topk as otk
from workloads import make_fp4, make_fp8

pytestmark = pytest.mark.gpu
pmqa = pytest.importorskip("paged_mqa_logits_amd")

FOUR_GIB = 1 << 32
LDO = 1 << 28          # floats per output row: row r starts r GiB into the buffer
GUARD_COLS = 8         # columns past max_context_len that no call may write
GUARD = 12345.0


def _relocated(d, dev):
    """Device kv_cache and block_table with every page id moved up by the
    first id whose bytes start past 4 GiB; the pages below hold 0xFF."""
    page_bytes = int(d["kv_cache"].shape[1])
    base = FOUR_GIB // page_bytes + 7
    n = int(d["kv_cache"].shape[0])
    assert base * page_bytes > FOUR_GIB and base + n < 2 ** 31
    big = torch.full((base + n, page_bytes), 0xFF, dtype=torch.uint8, device="cuda")
    big[base:] = dev["kv_cache"]
    return big, (dev["block_table"] + base).contiguous()


def _spaced_rows(rows, M):
    """[rows, M] view of rows LDO floats apart; columns [M, M + GUARD_COLS)
    of every row hold GUARD."""
    buf = torch.empty((rows, LDO), dtype=torch.float32, device="cuda")
    buf[:, M:M + GUARD_COLS] = GUARD
    return buf, buf[:, :M]


def _row_lengths(d):
    ctx, nn, M = d["context_lens"], int(d["next_n"]), int(d["max_context_len"])
    c = sr.units_per_row(np.maximum(ctx, 0))
    return np.array([otk.fused_row_length(ctx[r // nn], nn, r % nn, M, c[r // nn])
                     for r in range(len(ctx) * nn)])


@pytest.mark.timeout(300)
@pytest.mark.parametrize("variant,next_n", [("fp8", 1), ("fp8", 2), ("fp4", 1)])
def test_offsets_past_4gib(variant, next_n):
    announce(f"offsets past 4 GiB {variant} next_n={next_n}")
    ctx = [300, 0, 1000, 2049, 7000, 3000] if next_n == 1 else [1000, 7000, 2500]
    mk = make_fp8 if variant == "fp8" else make_fp4
    d = mk(ctx, next_n=next_n, max_context_len=7168, seed=91 + next_n)
    M, R = int(d["max_context_len"]), len(ctx) * next_n
    assert (R - 1) * LDO * 4 > FOUR_GIB
    ref = oracle(d)
    dev = upload(d)
    kv, bt = _relocated(d, dev)
    fp8 = variant == "fp8"
    vt = pmqa.VARIANT_FP8 if fp8 else pmqa.VARIANT_FP4
    sched = pmqa.compute_schedule(dev["context_lens"], variant=vt, next_n=next_n)
    buf, out = _spaced_rows(R, M)

    if fp8:
        pmqa.paged_mqa_logits_fp8(dev["q"], kv, dev["weights"], dev["context_lens"], bt, sched,
                                  M, out=out)
    else:
        pmqa.paged_mqa_logits_fp4(dev["q"], dev["q_scale"], kv, dev["weights"],
                                  dev["context_lens"], bt, sched, M, out=out)
    torch.cuda.synchronize()
    assert torch.all(buf[:, M:M + GUARD_COLS] == GUARD)
    stats = parity.check(out.cpu().numpy(), ref, f"{variant} logits past 4 GiB")
    print(f"[gpu-case] {stats['checked']} scores, {stats['masked']} masked entries compared",
          flush=True)

    lens = _row_lengths(d)
    lens_dev = torch.from_numpy(lens.astype(np.int32)).cuda()
    for k in (100, 2048):
        if fp8:
            idx, val = pmqa.paged_mqa_topk_fp8(dev["q"], kv, dev["weights"], dev["context_lens"],
                                               bt, sched, M, k, workspace=out)
        else:
            idx, val = pmqa.paged_mqa_topk_fp4(dev["q"], dev["q_scale"], kv, dev["weights"],
                                               dev["context_lens"], bt, sched, M, k,
                                               workspace=out)
        torch.cuda.synchronize()
        parity.check_topk(idx.cpu().numpy(), val.cpu().numpy(), ref, lens, k,
                          f"{variant} fused top-k past 4 GiB k={k}")
        # the selection alone, on the strided rows the fused step left behind
        i2, v2 = pmqa.select_topk(out, lens_dev, k, select_workspace=None)
        torch.cuda.synchronize()
        assert torch.equal(i2, idx) and torch.equal(v2.view(torch.int32), val.view(torch.int32))
    assert torch.all(buf[:, M:M + GUARD_COLS] == GUARD)
