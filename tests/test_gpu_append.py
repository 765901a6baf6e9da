"""quantize_append_fp8 / quantize_append_fp4 against the oracle producer,
byte for byte over the whole cache, and the appended cache read back by the
logits calls."""
import numpy as np
import pytest
import torch

import parity
from gpu_util import announce, oracle, run
from oracle import formats, quantize as qz

pytestmark = pytest.mark.gpu
pmqa = pytest.importorskip("paged_mqa_logits_amd")

E4M3 = formats.e4m3fn_table()


def _special_tokens():
    """Tokens that land on rounding ties and edge cases (fp32, D = 128)."""
    toks = []
    # fp8 ties: amax 448 makes the scale exactly 1, so x / scale = x; every
    # midpoint between adjacent finite E4M3 magnitudes, both signs
    mids = ((E4M3[:126] + E4M3[1:127]) / 2).astype(np.float32)
    for start in range(0, 126, 63):
        t = np.zeros(128, np.float32)
        t[0] = 448.0
        m = mids[start:start + 63]
        t[1:1 + len(m)] = m
        t[64:64 + len(m)] = -m
        toks.append(t)
    # MXFP4 ties: a block with amax 4 has exponent 0, so values are rounded
    # as they are
    t = np.zeros(128, np.float32)
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 4.0, -0.25, -0.75, -1.25, -5.0]
    for blk in range(4):
        t[32 * blk:32 * blk + len(ties)] = np.array(ties, np.float32) * np.float32(2.0 ** (blk - 1))
    toks.append(t)
    toks.append(np.zeros(128, np.float32))                      # all zero
    t = np.zeros(128, np.float32)
    t[::2] = -0.0                                               # negative zeros
    t[5] = 3.0
    t[7] = -1e-30                                               # rounds to -0
    toks.append(t)
    t = (np.random.default_rng(5).standard_normal(128) * 1e-20).astype(np.float32)
    toks.append(t)                                              # tiny but normal
    t = np.float32(7.9) * np.ones(128, np.float32)              # saturates in MXFP4
    t[64:] = -t[64:]
    toks.append(t)
    t = np.logspace(-6, 6, 128).astype(np.float32)              # wide dynamic range
    toks.append(t)
    return np.stack(toks)


def _case(n, pages, seed):
    rng = np.random.default_rng(seed)
    k = (rng.standard_normal((n, 128)) * 10.0 ** rng.uniform(-3, 3, (n, 1))).astype(np.float32)
    sp = _special_tokens()
    k[:len(sp)] = sp
    slots = rng.permutation(pages * 64)[:n].astype(np.int64)
    slots[rng.random(n) < 0.05] = -1                            # skipped
    slots[3] = pages * 64 + 17                                  # past the pool: skipped
    return k, slots


@pytest.mark.parametrize("variant", ["fp8", "fp4"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n,pages", [(1, 1), (37, 3), (5000, 120)])
def test_append_matches_oracle(variant, dtype, n, pages):
    announce(f"append {variant} {dtype} n={n} pages={pages}")
    k, slots = _case(max(n, 16), pages, seed=100 + n)
    k, slots = k[:n], slots[:n]
    if n == 1:
        slots[:] = 42
    kt = torch.from_numpy(k).cuda()
    if dtype == "bf16":
        kt = kt.to(torch.bfloat16)
        k = kt.float().cpu().numpy()            # the values the kernel sees, exactly
    page_bytes = pmqa.FP8_PAGE_BYTES if variant == "fp8" else pmqa.FP4_PAGE_BYTES
    poison = np.full((pages, page_bytes), 0xA7, np.uint8)
    cache = torch.from_numpy(poison).cuda()
    fn = pmqa.quantize_append_fp8 if variant == "fp8" else pmqa.quantize_append_fp4
    fn(kt.contiguous(), torch.from_numpy(slots).cuda(), cache)
    torch.cuda.synchronize()
    got = cache.cpu().numpy()
    keep = slots.copy()
    keep[keep >= pages * 64] = -1
    want = (qz.append_fp8 if variant == "fp8" else qz.append_fp4)(poison, k, keep)
    bad = np.argwhere(got != want)
    assert len(bad) == 0, f"{len(bad)} bytes differ, first at page/byte {bad[:5].tolist()}"


def test_append_empty_is_a_no_op():
    announce("append n=0")
    cache = torch.full((2, pmqa.FP8_PAGE_BYTES), 3, dtype=torch.uint8, device="cuda")
    pmqa.quantize_append_fp8(torch.empty((0, 128), device="cuda"),
                             torch.empty((0,), dtype=torch.int64, device="cuda"), cache)
    torch.cuda.synchronize()
    assert bool((cache == 3).all())


def test_validate_mode_rejects_bad_and_duplicate_slots(monkeypatch):
    announce("append validate")
    cache = torch.zeros((2, pmqa.FP8_PAGE_BYTES), dtype=torch.uint8, device="cuda")
    k = torch.ones((3, 128), device="cuda")
    monkeypatch.setenv("PMQA_VALIDATE_INPUTS", "1")
    pmqa.quantize_append_fp8(k, torch.tensor([0, -1, 127], device="cuda"), cache)
    for slots in ([0, 128, 5], [4, 9, 4]):
        with pytest.raises(pmqa.PmqaError) as ei:
            pmqa.quantize_append_fp8(k, torch.tensor(slots, device="cuda"), cache)
        assert ei.value.status_name == "PMQA_ERR_INVALID_VALUE"
    torch.cuda.synchronize()


@pytest.mark.parametrize("variant", ["fp8", "fp4"])
def test_appended_cache_scores_like_the_oracle(variant):
    """Fill a cache token by token with the append kernel (a decode-style
    stream: one token per row per call), then score it: the logits must match
    the oracle run on the oracle-appended cache."""
    announce(f"append then score {variant}")
    from workloads import make_fp4, make_fp8
    rng = np.random.default_rng(7)
    ctx = np.array([0, 70, 300, 129, 1], np.int32)
    mk = make_fp8 if variant == "fp8" else make_fp4
    d = mk(ctx, max_context_len=320, seed=7)
    B = len(ctx)
    raw = rng.standard_normal((B, 320, 128)).astype(np.float32)
    P, bt = d["kv_cache"].shape[0], d["block_table"]
    dev_cache = torch.from_numpy(np.zeros_like(d["kv_cache"])).cuda()
    want = np.zeros_like(d["kv_cache"])
    fn = pmqa.quantize_append_fp8 if variant == "fp8" else pmqa.quantize_append_fp4
    ref_fn = qz.append_fp8 if variant == "fp8" else qz.append_fp4
    all_k, all_s = [], []
    for t in range(int(ctx.max())):
        rows = np.nonzero(ctx > t)[0]
        slots = (bt[rows, t // 64].astype(np.int64) * 64 + t % 64)
        fn(torch.from_numpy(raw[rows, t]).cuda(), torch.from_numpy(slots).cuda(), dev_cache)
        all_k.append(raw[rows, t])
        all_s.append(slots)
    want = ref_fn(want, np.concatenate(all_k), np.concatenate(all_s))
    got_cache = dev_cache.cpu().numpy()
    assert np.array_equal(got_cache, want)
    d2 = dict(d, kv_cache=want)
    lg, _ = run(d2)
    parity.check(lg, oracle(d2), f"append+score {variant}")
