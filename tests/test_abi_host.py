"""Host-side checks of the C ABI: the library loads, exports every declared
symbol and rejects bad arguments before touching a device (runs without GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pmqa.h")

pmqa = pytest.importorskip("paged_mqa_logits_amd",
                           reason="libpmqa.so not built (python paged_mqa_logits_amd/build.py)")


def _declared_functions(header=HEADER):
    with open(header) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s+\*?([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    assert set(names) == set(pmqa.EXPORTS), names


def test_library_exports_every_declared_symbol():
    lib = pmqa.library()
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_ceiling_library_exports_its_header():
    """The measurement library beside the logits library (streaming ceiling
    kernels timed by bench.py) exports what include/pmqa_ceiling.h declares."""
    names = _declared_functions(os.path.join(ROOT, "include", "pmqa_ceiling.h"))
    assert names == ["pmqa_ceiling_fill", "pmqa_ceiling_gather"]
    lib = ctypes.CDLL(os.path.join(ROOT, "paged_mqa_logits_amd", "libpmqa_ceiling.so"))
    for name in names:
        assert hasattr(lib, name), name
    # argument checks return 1 before any launch
    p = ctypes.c_void_p
    lib.pmqa_ceiling_gather.argtypes = [p, ctypes.c_int64, ctypes.c_int32, p, ctypes.c_int64,
                                        ctypes.c_int32, ctypes.c_int32, p, p]
    lib.pmqa_ceiling_fill.argtypes = [p, ctypes.c_int64, ctypes.c_float, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_int32, p]
    fake = 0x10000
    assert lib.pmqa_ceiling_gather(p(fake), 10, 8448, p(fake), 5, 4, 3, p(fake), p(0)) == 1
    assert lib.pmqa_ceiling_gather(p(fake), 10, 4000, p(fake), 5, 4, 2, p(fake), p(0)) == 1
    assert lib.pmqa_ceiling_gather(p(0), 10, 8448, p(fake), 5, 4, 2, p(fake), p(0)) == 1
    assert lib.pmqa_ceiling_fill(p(fake), 6, 0.0, 4, 256, 1, p(0)) == 1
    assert lib.pmqa_ceiling_fill(p(fake + 4), 8, 0.0, 4, 256, 1, p(0)) == 1
    assert lib.pmqa_ceiling_fill(p(fake), 8, 0.0, 4, 96, 1, p(0)) == 1      # threads
    assert lib.pmqa_ceiling_fill(p(fake), 8, 0.0, 4, 128, 2, p(0)) == 1     # stores per round


def test_schedule_bytes():
    assert pmqa.schedule_bytes(4, 3) == 4 * (8 + 2 * 4 + 4 + 1)
    assert pmqa.schedule_bytes(2048, 3072) == 4 * (8 + 2 * 3073 + 2049)
    assert pmqa.schedule_bytes(0, 3) == 0
    assert pmqa.schedule_bytes(3, 0) == 0


def test_schedule_size_is_exact_in_the_binding():
    """The binding's schedule buffers have exactly the size for their worker
    count, so the worker count the logits wrappers infer from a length is
    the one the schedule was built for."""
    for B, W in [(4, 8), (4, 16), (2048, 1024), (1, 1)]:
        words = pmqa.schedule_bytes(B, W) // 4
        pmqa.check_schedule_words(words, B, W)
        assert pmqa.sched_workers(words, B) == W
        assert pmqa.sched_workers(words, B, num_workers=3) == 3
    # a buffer sized for 16 workers offered for 8 is refused
    with pytest.raises(ValueError, match="needs exactly"):
        pmqa.check_schedule_words(pmqa.schedule_bytes(4, 16) // 4, 4, 8)
    with pytest.raises(ValueError, match="needs exactly"):
        pmqa.check_schedule_words(pmqa.schedule_bytes(4, 8) // 4 - 1, 4, 8)
    with pytest.raises(ValueError, match="invalid schedule size"):
        pmqa.check_schedule_words(10, 0, 8)
    with pytest.raises(ValueError, match="does not fit"):
        pmqa.sched_workers(pmqa.schedule_bytes(4, 8) // 4 + 1, 4)


FAKE = 0x10000  # aligned, never dereferenced: every call below fails first


def _fp8(lib, **kw):
    args = dict(q=FAKE, kv=FAKE, w=FAKE, ctx=FAKE, bt=FAKE, sched=FAKE, out=FAKE, batch=2,
                next_n=1, heads=64, dim=128, page=64, num_pages=10, bt_stride=4, max_ctx=256,
                ldo=256, workers=8)
    args.update(kw)
    p = ctypes.c_void_p
    return lib.paged_mqa_logits_fp8(
        p(args["q"]), p(args["kv"]), p(args["w"]), p(args["ctx"]), p(args["bt"]),
        p(args["sched"]), p(args["out"]), args["batch"], args["next_n"], args["heads"],
        args["dim"], args["page"], args["num_pages"], args["bt_stride"], args["max_ctx"],
        args["ldo"], args["workers"], p(0))


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=0), 1, "q is null"),
    (dict(kv=0), 1, "kv_cache is null"),
    (dict(w=0), 1, "weights is null"),
    (dict(ctx=0), 1, "context_lens is null"),
    (dict(bt=0), 1, "block_table is null"),
    (dict(sched=0), 1, "schedule is null"),
    (dict(out=0), 1, "logits is null"),
    (dict(q=FAKE + 4), 1, "q must be 16-byte aligned"),
    (dict(out=FAKE + 8), 1, "logits must be 16-byte aligned"),
    (dict(ctx=FAKE + 2), 1, "4-byte aligned"),
    (dict(batch=0), 1, "batch"),
    (dict(heads=48), 2, "not compiled"),
    (dict(dim=64), 2, "not compiled"),
    (dict(page=16), 2, "not compiled"),
    (dict(next_n=3), 2, "next_n = 3"),
    (dict(num_pages=0), 1, "num_pages"),
    (dict(bt_stride=0), 1, "block_table_stride"),
    (dict(max_ctx=0), 1, "max_context_len"),
    (dict(ldo=100), 1, "logits_stride"),
    (dict(ldo=258), 1, "multiple of 4"),
    (dict(workers=0), 1, "num_workers"),
])
def test_fp8_argument_checks(kw, status, needle):
    lib = pmqa.library()
    st = _fp8(lib, **kw)
    assert st == status, (st, pmqa.last_error())
    assert needle in pmqa.last_error()


def test_fp4_null_q_scale():
    lib = pmqa.library()
    p = ctypes.c_void_p
    st = lib.paged_mqa_logits_fp4(p(FAKE), p(0), p(FAKE), p(FAKE), p(FAKE), p(FAKE), p(FAKE),
                                  p(FAKE), 2, 1, 64, 128, 64, 10, 4, 256, 256, 8, p(0))
    assert st == 1 and "q_scale is null" in pmqa.last_error()


@pytest.mark.parametrize("args,needle", [
    ((0, 4, 8, FAKE), "context_lens is null"),
    ((FAKE, 4, 8, 0), "schedule is null"),
    ((FAKE, 0, 8, FAKE), "batch"),
    ((FAKE, 4, 0, FAKE), "num_workers"),
    ((FAKE + 1, 4, 8, FAKE), "aligned"),
])
@pytest.mark.parametrize("entry", ["compute_schedule", "compute_schedule_linear",
                                   "refresh_schedule"])
def test_schedule_argument_checks(args, needle, entry):
    lib = pmqa.library()
    p = ctypes.c_void_p
    ctx, B, W, out = args
    extra = (p(0),) if entry == "refresh_schedule" else ()
    st = getattr(lib, entry)(p(ctx), B, W, p(out), *extra, p(0))
    assert st == 1 and needle in pmqa.last_error()


def test_refresh_schedule_flag_alignment():
    lib = pmqa.library()
    p = ctypes.c_void_p
    st = lib.refresh_schedule(p(FAKE), 4, 8, p(FAKE), p(FAKE + 2), p(0))
    assert st == 1 and "recomputed" in pmqa.last_error()


def test_num_workers_without_a_usable_device_returns_minus_one():
    """pmqa_num_workers reports failure as -1 with a message (here: no GPU, or
    none with the requested index)."""
    lib = pmqa.library()
    assert lib.pmqa_num_workers(1 << 20) == -1
    assert pmqa.last_error() != ""


def test_default_num_workers_argument_checks():
    lib = pmqa.library()
    out = ctypes.c_int32(0)
    assert lib.pmqa_default_num_workers(0, 5, 1, 64, ctypes.byref(out)) == 1
    assert lib.pmqa_default_num_workers(0, 0, 3, 64, ctypes.byref(out)) == 2
    assert lib.pmqa_default_num_workers(0, 0, 1, 48, ctypes.byref(out)) == 2
    assert lib.pmqa_default_num_workers(0, 0, 1, 64, None) == 1


def test_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros((1, 1, 64, 128), dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU tensor"):
        pmqa.paged_mqa_logits_fp8(q, q, q, q, q, q, 16)


def test_select_workspace_bytes():
    """Sections of whole 256-byte blocks: a 64-word header, the chunk list
    (16 words per row), map, lengths and thresholds (one word per row each),
    chunk counts (16 words per row), keys and columns (6272 words per row
    each: 1.5 x 3840 list slots plus 32 per chunk)."""
    def words(n):
        return (n + 63) // 64 * 64

    for rows in (1, 5, 100, 512):
        want = 4 * (64 + 3 * words(rows) + 2 * words(16 * rows) + 2 * words(6272 * rows))
        assert pmqa.select_workspace_bytes(rows, 600000, 2048) == want, rows
    assert pmqa.select_workspace_bytes(0, 600000, 2048) == 0
    assert pmqa.select_workspace_bytes(513, 600000, 2048) == 0    # no split beyond 512 rows
    # rows of at most 524288 columns are selected without splitting
    assert pmqa.select_workspace_bytes(64, 524288, 16) == 0
    assert pmqa.select_workspace_bytes(64, 131072, 2048) == 0
    assert pmqa.select_workspace_bytes(64, 600000, 600000) == 0   # every row has <= k candidates
    assert pmqa.select_workspace_bytes(64, 524289, 16) > 0


def _select(lib, ws, ws_bytes, rows=4, k=8):
    p = ctypes.c_void_p
    return lib.select_topk(p(FAKE), 600000, rows, 600000, p(FAKE), k, p(FAKE), p(FAKE), 8, p(ws),
                           ws_bytes, p(0))


def test_select_workspace_argument_checks():
    lib = pmqa.library()
    need = pmqa.select_workspace_bytes(4, 600000, 8)
    assert need > 0
    assert _select(lib, FAKE, need - 1) == 1
    assert "select_workspace_bytes" in pmqa.last_error()
    assert _select(lib, FAKE + 8, need) == 1
    assert "16-byte aligned" in pmqa.last_error()
    assert _select(lib, FAKE, need, k=0) == 1 and "k = 0" in pmqa.last_error()
