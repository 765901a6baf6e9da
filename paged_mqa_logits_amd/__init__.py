"""Python binding of the MI355X paged MQA logits library (``libpmqa.so``).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/pmqa.h``.  torch provides
device memory and the current stream; tensors are passed as raw pointers.
There is no fallback: importing this package fails if the library has not
been built (``python paged_mqa_logits_amd/build.py``).

Entry points (same names as the C ABI):

    compute_schedule(context_lens, num_workers=None, out=None) -> schedule
    compute_schedule_linear(context_lens, num_workers=None, out=None) -> schedule
    refresh_schedule(context_lens, schedule, num_workers=None, recomputed=None)
    paged_mqa_logits_fp8(q, kv_cache, weights, context_lens, block_table,
                         schedule, max_context_len, out=None) -> logits
    paged_mqa_logits_fp4(q, q_scale, kv_cache, weights, context_lens,
                         block_table, schedule, max_context_len, out=None)
    select_topk(logits, lengths, k) -> (indices, values)
    select_workspace_bytes(rows, max_context_len, k)
    select_topk_noalloc(logits, lengths, k) -> (indices, values)
    paged_mqa_topk_fp8(q, kv_cache, weights, context_lens, block_table,
                       schedule, max_context_len, k) -> (indices, values)
    paged_mqa_topk_fp4(q, q_scale, kv_cache, ..., k) -> (indices, values)
    quantize_append_fp8(k, slot_mapping, kv_cache) -> kv_cache
    quantize_append_fp4(k, slot_mapping, kv_cache) -> kv_cache
    num_workers(device=None)
    default_num_workers(variant, next_n=1, device=None)
    schedule_bytes(batch, num_workers)
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpmqa.so")

NUM_HEADS = 64
HEAD_DIM = 128
PAGE_SIZE = 64
UNIT_TOKENS = 256
FP8_PAGE_BYTES = 8448
FP4_PAGE_BYTES = 4352
SCHED_HEADER = 8
SCHED_MAGIC = 0x41514D50

VARIANT_FP8 = 0
VARIANT_FP4 = 1

STATUS = {0: "PMQA_OK", 1: "PMQA_ERR_INVALID_ARGUMENT", 2: "PMQA_ERR_UNSUPPORTED",
          3: "PMQA_ERR_INVALID_VALUE", 4: "PMQA_ERR_STALE_SCHEDULE",
          5: "PMQA_ERR_CAPTURING", 6: "PMQA_ERR_HIP"}

EXPORTS = ("pmqa_last_error", "pmqa_num_workers", "pmqa_default_num_workers",
           "pmqa_schedule_bytes",
           "compute_schedule", "compute_schedule_linear", "refresh_schedule",
           "paged_mqa_logits_fp8", "paged_mqa_logits_fp4", "quantize_append_fp8",
           "quantize_append_fp4", "select_topk", "paged_mqa_topk_fp8", "paged_mqa_topk_fp4",
           "pmqa_select_workspace_bytes", "select_topk_noalloc")


class PmqaError(RuntimeError):
    """A library call returned a status other than PMQA_OK."""

    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.status_name = STATUS.get(status, str(status))


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python paged_mqa_logits_amd/build.py` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)
_i32, _i64, _p, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t

_lib.pmqa_last_error.restype = ctypes.c_char_p
_lib.pmqa_last_error.argtypes = []
_lib.pmqa_schedule_bytes.restype = ctypes.c_size_t
_lib.pmqa_schedule_bytes.argtypes = [_i32, _i32]
_lib.pmqa_num_workers.restype = ctypes.c_int
_lib.pmqa_num_workers.argtypes = [ctypes.c_int]
_lib.pmqa_default_num_workers.restype = ctypes.c_int
_lib.pmqa_default_num_workers.argtypes = [ctypes.c_int, _i32, _i32, _i32, ctypes.POINTER(_i32)]
_lib.compute_schedule.restype = ctypes.c_int
_lib.compute_schedule.argtypes = [_p, _i32, _i32, _p, _p]
_lib.compute_schedule_linear.restype = ctypes.c_int
_lib.compute_schedule_linear.argtypes = [_p, _i32, _i32, _p, _p]
_lib.refresh_schedule.restype = ctypes.c_int
_lib.refresh_schedule.argtypes = [_p, _i32, _i32, _p, _p, _p]
_lib.paged_mqa_logits_fp8.restype = ctypes.c_int
_lib.paged_mqa_logits_fp8.argtypes = [_p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32,
                                      _i64, _i32, _i32, _i64, _i32, _p]
_lib.select_topk.restype = ctypes.c_int
_lib.select_topk.argtypes = [_p, _i64, _i32, _i32, _p, _i32, _p, _p, _i64, _p, _sz, _p]
_lib.select_topk_noalloc.restype = ctypes.c_int
_lib.select_topk_noalloc.argtypes = [_p, _i64, _i32, _i32, _p, _i32, _p, _p, _i64, _p]
_lib.pmqa_select_workspace_bytes.restype = _sz
_lib.pmqa_select_workspace_bytes.argtypes = [_i32, _i32, _i32]
_lib.paged_mqa_topk_fp8.restype = ctypes.c_int
_lib.paged_mqa_topk_fp8.argtypes = [_p, _p, _p, _p, _p, _p, _p, _i32, _p, _p, _i64, _p, _sz,
                                    _i32, _i32, _i32, _i32, _i32, _i64, _i32, _i32, _i64, _i32,
                                    _p]
_lib.paged_mqa_topk_fp4.restype = ctypes.c_int
_lib.paged_mqa_topk_fp4.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _i32, _p, _p, _i64, _p, _sz,
                                    _i32, _i32, _i32, _i32, _i32, _i64, _i32, _i32, _i64, _i32,
                                    _p]
_lib.quantize_append_fp8.restype = ctypes.c_int
_lib.quantize_append_fp8.argtypes = [_p, _i32, _i64, _i32, _p, _p, _i64, _p]
_lib.quantize_append_fp4.restype = ctypes.c_int
_lib.quantize_append_fp4.argtypes = [_p, _i32, _i64, _i32, _p, _p, _i64, _p]
_lib.paged_mqa_logits_fp4.restype = ctypes.c_int
_lib.paged_mqa_logits_fp4.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32,
                                      _i32, _i64, _i32, _i32, _i64, _i32, _p]


def library():
    """The loaded ctypes library (for tests of the raw ABI)."""
    return _lib


def last_error():
    return _lib.pmqa_last_error().decode()


def _check(status):
    if status != 0:
        raise PmqaError(status, last_error())


def _stream_ptr(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, name, dtypes, ndim=None, contiguous=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}; expected one of {dtypes}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_BYTE = (torch.uint8, torch.float8_e4m3fn, torch.int8)


def schedule_bytes(batch, num_workers):
    return int(_lib.pmqa_schedule_bytes(int(batch), int(num_workers)))


def num_workers(device=None):
    """Persistent-grid size of the fp8 batch-decode kernel (next_n 1, 64 heads)."""
    dev = torch.cuda.current_device() if device is None else int(device)
    w = int(_lib.pmqa_num_workers(dev))
    if w < 1:
        raise RuntimeError(f"pmqa_num_workers({dev}) failed: {last_error()}")
    return w


def default_num_workers(variant=VARIANT_FP8, next_n=1, device=None, num_heads=NUM_HEADS):
    dev = torch.cuda.current_device() if device is None else int(device)
    out = _i32(0)
    _check(_lib.pmqa_default_num_workers(dev, int(variant), int(next_n), int(num_heads),
                                         ctypes.byref(out)))
    return int(out.value)


def check_schedule_words(words, batch, num_workers):
    """Raise ValueError unless a schedule tensor of `words` int32 words is
    exactly the size for (batch, num_workers).  The logits and top-k wrappers
    infer num_workers from a schedule's length, so every schedule buffer the
    binding writes must have exactly that length: a larger one would be read
    as a schedule for more workers, which the kernels then reject by
    scoring nothing."""
    need = schedule_bytes(batch, num_workers) // 4
    if need == 0:
        raise ValueError(f"invalid schedule size: batch {batch}, num_workers {num_workers}")
    if words != need:
        raise ValueError(f"schedule buffer has {words} words; batch {batch} with "
                         f"{num_workers} workers needs exactly {need}")


def _schedule_buffer(context_lens, num_workers, out, variant, next_n, num_heads=NUM_HEADS):
    _need(context_lens, "context_lens", (torch.int32,), ndim=1)
    B = context_lens.shape[0]
    W = (default_num_workers(variant, next_n, num_heads=num_heads) if num_workers is None
         else int(num_workers))
    words = schedule_bytes(B, W) // 4
    if out is None:
        out = torch.empty(words, dtype=torch.int32, device=context_lens.device)
    else:
        _need(out, "out", (torch.int32,), ndim=1)
        check_schedule_words(out.numel(), B, W)
    return B, W, out


def compute_schedule(context_lens, num_workers=None, out=None, variant=VARIANT_FP8, next_n=1,
                     stream=None, num_heads=NUM_HEADS):
    """Schedule (int32 tensor) of the persistent workers for these lengths
    (default worker count: that of the logits kernel for variant, next_n and
    num_heads)."""
    B, W, out = _schedule_buffer(context_lens, num_workers, out, variant, next_n, num_heads)
    _check(_lib.compute_schedule(_ptr(context_lens), B, W, _ptr(out), _stream_ptr(stream)))
    return out


def compute_schedule_linear(context_lens, num_workers=None, out=None, variant=VARIANT_FP8,
                            next_n=1, stream=None):
    """The same schedule, worker starts found by a linear scan (for timing)."""
    B, W, out = _schedule_buffer(context_lens, num_workers, out, variant, next_n)
    _check(_lib.compute_schedule_linear(_ptr(context_lens), B, W, _ptr(out),
                                        _stream_ptr(stream)))
    return out


def refresh_schedule(context_lens, schedule, num_workers=None, recomputed=None,
                     variant=VARIANT_FP8, next_n=1, stream=None):
    """Rebuild `schedule` in place on the device only if it no longer matches
    these lengths; `recomputed` (optional int32 device tensor, 1 element)
    receives 1 after a rebuild, 0 otherwise.  Returns `schedule`."""
    B, W, schedule = _schedule_buffer(context_lens, num_workers, schedule, variant, next_n)
    if recomputed is not None:
        _need(recomputed, "recomputed", (torch.int32,))
    _check(_lib.refresh_schedule(_ptr(context_lens), B, W, _ptr(schedule), _ptr(recomputed),
                                 _stream_ptr(stream)))
    return schedule


def schedule_workers(schedule):
    """num_workers recorded in a schedule tensor's header (reads the device)."""
    return int(schedule[2].item())


def _logits_out(out, rows, max_context_len, device):
    if out is None:
        ldo = (max_context_len + 3) // 4 * 4
        buf = torch.empty((rows, ldo), dtype=torch.float32, device=device)
        return buf[:, :max_context_len], ldo, buf
    _need(out, "out", (torch.float32,), ndim=2, contiguous=False)
    if out.shape[0] != rows or out.shape[1] < max_context_len or out.stride(1) != 1:
        raise ValueError(f"out must be [{rows}, >= {max_context_len}] with unit column stride")
    return out, out.stride(0), out


def _fp8_shapes(q, kv_cache, weights, context_lens, block_table, schedule):
    _need(q, "q", _BYTE, ndim=4)
    _need(kv_cache, "kv_cache", _BYTE, ndim=2)
    _need(weights, "weights", (torch.float32,), ndim=2)
    _need(context_lens, "context_lens", (torch.int32,), ndim=1)
    _need(block_table, "block_table", (torch.int32,), ndim=2)
    _need(schedule, "schedule", (torch.int32,), ndim=1)
    B, NN, H, D = q.shape
    if kv_cache.shape[1] != FP8_PAGE_BYTES:
        raise ValueError(f"kv_cache rows must be {FP8_PAGE_BYTES} bytes, got {kv_cache.shape[1]}")
    if tuple(weights.shape) != (B * NN, H):
        raise ValueError(f"weights must be [{B * NN}, {H}], got {tuple(weights.shape)}")
    if context_lens.shape[0] != B or block_table.shape[0] != B:
        raise ValueError("context_lens and block_table must have one row per batch row")
    return B, NN, H, D


def _fp4_shapes(q, q_scale, kv_cache, weights, context_lens, block_table, schedule):
    _need(q, "q", _BYTE, ndim=4)
    _need(q_scale, "q_scale", (torch.uint8, torch.float8_e8m0fnu), ndim=4)
    _need(kv_cache, "kv_cache", _BYTE, ndim=2)
    _need(weights, "weights", (torch.float32,), ndim=2)
    _need(context_lens, "context_lens", (torch.int32,), ndim=1)
    _need(block_table, "block_table", (torch.int32,), ndim=2)
    _need(schedule, "schedule", (torch.int32,), ndim=1)
    B, NN, H, Dh = q.shape
    if tuple(q_scale.shape) != (B, NN, H, 2 * Dh // 32):
        raise ValueError(f"q_scale must be [{B}, {NN}, {H}, {2 * Dh // 32}]")
    if kv_cache.shape[1] != FP4_PAGE_BYTES:
        raise ValueError(f"kv_cache rows must be {FP4_PAGE_BYTES} bytes, got {kv_cache.shape[1]}")
    if tuple(weights.shape) != (B * NN, H):
        raise ValueError(f"weights must be [{B * NN}, {H}], got {tuple(weights.shape)}")
    if context_lens.shape[0] != B or block_table.shape[0] != B:
        raise ValueError("context_lens and block_table must have one row per batch row")
    return B, NN, H, 2 * Dh


def paged_mqa_logits_fp8(q, kv_cache, weights, context_lens, block_table, schedule,
                         max_context_len, out=None, num_workers=None, stream=None):
    """fp8 paged MQA logits; returns fp32 [batch*next_n, max_context_len]."""
    B, NN, H, D = _fp8_shapes(q, kv_cache, weights, context_lens, block_table, schedule)
    W = _sched_workers(schedule, B, num_workers)
    view, ldo, buf = _logits_out(out, B * NN, int(max_context_len), q.device)
    _check(_lib.paged_mqa_logits_fp8(
        _ptr(q), _ptr(kv_cache), _ptr(weights), _ptr(context_lens), _ptr(block_table),
        _ptr(schedule), _ptr(buf), B, NN, H, D, PAGE_SIZE, kv_cache.shape[0],
        block_table.shape[1], int(max_context_len), ldo, W, _stream_ptr(stream)))
    return view


def paged_mqa_logits_fp4(q, q_scale, kv_cache, weights, context_lens, block_table, schedule,
                         max_context_len, out=None, num_workers=None, stream=None):
    """MXFP4 paged MQA logits; returns fp32 [batch*next_n, max_context_len]."""
    B, NN, H, D = _fp4_shapes(q, q_scale, kv_cache, weights, context_lens, block_table, schedule)
    W = _sched_workers(schedule, B, num_workers)
    view, ldo, buf = _logits_out(out, B * NN, int(max_context_len), q.device)
    _check(_lib.paged_mqa_logits_fp4(
        _ptr(q), _ptr(q_scale), _ptr(kv_cache), _ptr(weights), _ptr(context_lens),
        _ptr(block_table), _ptr(schedule), _ptr(buf), B, NN, H, D, PAGE_SIZE,
        kv_cache.shape[0], block_table.shape[1], int(max_context_len), ldo, W,
        _stream_ptr(stream)))
    return view


def _topk_out(indices, values, rows, k, want_values, device):
    """Output buffers [rows, >= k] sharing one row stride."""
    if indices is None:
        indices = torch.empty((rows, k), dtype=torch.int32, device=device)
    _need(indices, "indices", (torch.int32,), ndim=2, contiguous=False)
    if indices.shape[0] != rows or indices.shape[1] < k or indices.stride(1) != 1:
        raise ValueError(f"indices must be [{rows}, >= {k}] with unit column stride")
    if values is None and want_values:
        values = torch.empty((rows, indices.stride(0)), dtype=torch.float32,
                             device=device)[:, :indices.shape[1]]
    if values is not None:
        _need(values, "values", (torch.float32,), ndim=2, contiguous=False)
        if tuple(values.shape) != tuple(indices.shape) or values.stride() != indices.stride():
            raise ValueError("values must have the shape and strides of indices")
    return indices, values, indices.stride(0)


def select_workspace_bytes(rows, max_context_len, k):
    """Bytes of the optional top-k split workspace (0: none would be used)."""
    return int(_lib.pmqa_select_workspace_bytes(int(rows), int(max_context_len), int(k)))


def _select_ws(select_workspace, rows, max_context_len, k, device):
    """(pointer, bytes) of the top-k split workspace: "auto" allocates one,
    None passes none, a uint8 tensor is used as given."""
    if select_workspace is None:
        return None, 0
    if isinstance(select_workspace, str):
        if select_workspace != "auto":
            raise ValueError('select_workspace must be "auto", None or a tensor')
        n = select_workspace_bytes(rows, max_context_len, k)
        if n == 0:
            return None, 0
        select_workspace = torch.empty(n, dtype=torch.uint8, device=device)
    _need(select_workspace, "select_workspace", (torch.uint8,), ndim=1)
    return select_workspace, select_workspace.numel()


def select_topk(logits, lengths, k, indices=None, values=None, want_values=True,
                select_workspace="auto", stream=None):
    """Top k of each row's first lengths[r] columns, ascending column order;
    returns (indices int32 [rows, k], values fp32 [rows, k] or None).
    select_workspace: "auto" (allocated here), None (single-kernel path) or a
    uint8 tensor of at least select_workspace_bytes(rows, max_context_len, k)
    bytes."""
    _need(logits, "logits", (torch.float32,), ndim=2, contiguous=False)
    _need(lengths, "lengths", (torch.int32,), ndim=1)
    rows, M = logits.shape
    if logits.stride(1) != 1:
        raise ValueError("logits must have unit column stride")
    if lengths.shape[0] != rows:
        raise ValueError("lengths must have one entry per row")
    indices, values, ldk = _topk_out(indices, values, rows, int(k), want_values, logits.device)
    ws, ws_bytes = _select_ws(select_workspace, rows, M, int(k), logits.device)
    _check(_lib.select_topk(_ptr(logits), logits.stride(0), rows, M, _ptr(lengths), int(k),
                            _ptr(indices), _ptr(values), ldk, _ptr(ws), ws_bytes,
                            _stream_ptr(stream)))
    return indices[:, :k], None if values is None else values[:, :k]


def select_topk_noalloc(logits, lengths, k, indices=None, values=None, want_values=True,
                        stream=None):
    """select_topk with the split workspace in the library's static scratch
    (the C call allocates nothing; pass indices / values to allocate nothing
    here either).  Calls overlapping on one device race on the scratch."""
    _need(logits, "logits", (torch.float32,), ndim=2, contiguous=False)
    _need(lengths, "lengths", (torch.int32,), ndim=1)
    rows, M = logits.shape
    if logits.stride(1) != 1:
        raise ValueError("logits must have unit column stride")
    if lengths.shape[0] != rows:
        raise ValueError("lengths must have one entry per row")
    indices, values, ldk = _topk_out(indices, values, rows, int(k), want_values, logits.device)
    _check(_lib.select_topk_noalloc(_ptr(logits), logits.stride(0), rows, M, _ptr(lengths),
                                    int(k), _ptr(indices), _ptr(values), ldk,
                                    _stream_ptr(stream)))
    return indices[:, :k], None if values is None else values[:, :k]


def paged_mqa_topk_fp8(q, kv_cache, weights, context_lens, block_table, schedule,
                       max_context_len, k, workspace=None, indices=None, values=None,
                       want_values=True, num_workers=None, select_workspace="auto",
                       stream=None):
    """The fp8 indexer step: logits of every scheduled unit into `workspace`
    (no -inf fill), then the top k per output row; returns (indices, values).
    select_workspace as in select_topk."""
    B, NN, H, D = _fp8_shapes(q, kv_cache, weights, context_lens, block_table, schedule)
    W = _sched_workers(schedule, B, num_workers)
    _, ldo, buf = _logits_out(workspace, B * NN, int(max_context_len), q.device)
    indices, values, ldk = _topk_out(indices, values, B * NN, int(k), want_values, q.device)
    ws, ws_bytes = _select_ws(select_workspace, B * NN, int(max_context_len), int(k), q.device)
    _check(_lib.paged_mqa_topk_fp8(
        _ptr(q), _ptr(kv_cache), _ptr(weights), _ptr(context_lens), _ptr(block_table),
        _ptr(schedule), _ptr(buf), int(k), _ptr(indices), _ptr(values), ldk, _ptr(ws), ws_bytes,
        B, NN, H, D,
        PAGE_SIZE, kv_cache.shape[0], block_table.shape[1], int(max_context_len), ldo, W,
        _stream_ptr(stream)))
    return indices[:, :k], None if values is None else values[:, :k]


def paged_mqa_topk_fp4(q, q_scale, kv_cache, weights, context_lens, block_table, schedule,
                       max_context_len, k, workspace=None, indices=None, values=None,
                       want_values=True, num_workers=None, select_workspace="auto",
                       stream=None):
    """The MXFP4 indexer step (see paged_mqa_topk_fp8)."""
    B, NN, H, D = _fp4_shapes(q, q_scale, kv_cache, weights, context_lens, block_table, schedule)
    W = _sched_workers(schedule, B, num_workers)
    _, ldo, buf = _logits_out(workspace, B * NN, int(max_context_len), q.device)
    indices, values, ldk = _topk_out(indices, values, B * NN, int(k), want_values, q.device)
    ws, ws_bytes = _select_ws(select_workspace, B * NN, int(max_context_len), int(k), q.device)
    _check(_lib.paged_mqa_topk_fp4(
        _ptr(q), _ptr(q_scale), _ptr(kv_cache), _ptr(weights), _ptr(context_lens),
        _ptr(block_table), _ptr(schedule), _ptr(buf), int(k), _ptr(indices), _ptr(values), ldk,
        _ptr(ws), ws_bytes, B, NN, H, D, PAGE_SIZE, kv_cache.shape[0], block_table.shape[1],
        int(max_context_len), ldo, W, _stream_ptr(stream)))
    return indices[:, :k], None if values is None else values[:, :k]


def sched_workers(words, batch, num_workers=None):
    """Worker count of a schedule of `words` int32 words for `batch` rows (no
    device read): `num_workers` when given, else the one count whose exact
    schedule size is `words` (the binding writes schedules of exactly that
    size, see check_schedule_words)."""
    if num_workers is not None:
        return int(num_workers)
    w2 = words - SCHED_HEADER - 2 - batch - 1        # = 2 * num_workers
    if w2 < 2 or w2 % 2:
        raise ValueError(f"schedule of {words} words does not fit batch {batch}; "
                         "pass num_workers explicitly")
    return w2 // 2


def _sched_workers(schedule, batch, num_workers):
    return sched_workers(schedule.numel(), batch, num_workers)


DTYPE_F32 = 0
DTYPE_BF16 = 1


def _append(fn, k, slot_mapping, kv_cache, page_bytes, stream):
    _need(k, "k", (torch.float32, torch.bfloat16), ndim=2)
    _need(slot_mapping, "slot_mapping", (torch.int64,), ndim=1)
    _need(kv_cache, "kv_cache", _BYTE, ndim=2)
    if kv_cache.shape[1] != page_bytes:
        raise ValueError(f"kv_cache rows must be {page_bytes} bytes, got {kv_cache.shape[1]}")
    if slot_mapping.shape[0] != k.shape[0]:
        raise ValueError("slot_mapping must have one entry per token of k")
    dtype = DTYPE_F32 if k.dtype == torch.float32 else DTYPE_BF16
    _check(fn(_ptr(k), dtype, k.shape[0], k.shape[1], _ptr(slot_mapping), _ptr(kv_cache),
              kv_cache.shape[0], _stream_ptr(stream)))
    return kv_cache


def quantize_append_fp8(k, slot_mapping, kv_cache, stream=None):
    """Quantize K tokens [n, 128] (fp32 or bf16) to E4M3 + fp32 scale and
    write them into the fp8 paged cache at slot_mapping (page*64 + row)."""
    return _append(_lib.quantize_append_fp8, k, slot_mapping, kv_cache, FP8_PAGE_BYTES, stream)


def quantize_append_fp4(k, slot_mapping, kv_cache, stream=None):
    """Quantize K tokens [n, 128] (fp32 or bf16) to MXFP4 and write them into
    the fp4 paged cache at slot_mapping (page*64 + row)."""
    return _append(_lib.quantize_append_fp4, k, slot_mapping, kv_cache, FP4_PAGE_BYTES, stream)
