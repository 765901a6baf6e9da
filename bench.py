"""Benchmark: fp8 paged MQA logits at batch-2048 decode on one MI355X.

One step is the whole hot path for one decode batch: compute_schedule
followed by paged_mqa_logits_fp8, replayed from a captured HIP graph, with all
inputs resident in HBM.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Workload (seeded, synthetic; see workloads/synth.py): B = 2048 rows, next_n 1,
64 heads, head_dim 128, 64-token pages; context lengths lognormal (median
4096, sigma 1) clipped to [1, 65536] with 10% of rows empty; output width
65536.

Reported beside the step rate:
  roofline      the paged_mqa_logits_fp8 call alone (its two kernels: the -inf
                fill and the unit kernel), timed with HIP events on the stream
                it is launched on: algorithmic bytes per call / mean call
                duration, against the 8 TB/s HBM peak; ``traffic`` is read from
                the rocprofv3 counter summary in profiles/ when that summary was
                taken on the current kernel sources, else null;
  mfma_busy_pct the unit kernel's MFMA busy share from the committed
                rocprofv3 counter summary (same rule), a secondary figure;
  decode_drift  a graph of [every non-empty row += 1 token, refresh_schedule,
                logits call] replayed step after step: the schedule is rebuilt
                on the device whenever a row crosses a 256-token boundary;
  ceiling       the practical HBM ceiling of the call on the same box: two
                hand-written streaming kernels (libpmqa_ceiling.so) move
                the call's bytes with no arithmetic, a gather that loads every
                page the call reads (16-byte non-temporal buffer loads, in
                the call's row order) and a non-temporal store sweep the size
                of the output; each is swept over waves per SIMD (and pages in
                flight) and the fastest shape kept.  copy_gbps = their bytes
                over their summed time, frac_of_copy = achieved / copy_gbps;
                torch_copy_gbps is a plain 1 GiB device copy, for reference;
  cpu_baseline  the fp64 CPU oracle on a fixed subset of the same rows.

Workloads moving less than 512 MB per call (mid_fp8) would fit the 256 MB
MALL between repeated calls; for them a 512 MB scrub write runs before each
timed call, outside its timed interval (mall_scrub: true).
"""
import argparse
import hashlib
import json
import re
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV tokens scored/s + achieved HBM GB/s, fp8 paged MQA logits, B=2048 decode"
HBM_PEAK_GBPS = 8000.0
WORKLOAD = "large_fp8"
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "logits_fp8_large_fp8_traffic.txt")
MFMA_SUMMARY = os.path.join(ROOT, "profiles", "logits_mfma_busy.txt")
# Sources (under paged_mqa_logits_amd/) that determine the timed kernels,
# compile flags included.
KERNEL_SOURCES = ["csrc/logits_kernel.hpp", "csrc/logits_fp8.hip", "csrc/tail_fill.hip",
                  "csrc/pmqa_internal.h", "csrc/api.cpp", "build.py"]


def strip_comments(text, python=False):
    """Source text without its comments and blank lines, so that editing a
    comment keeps the hash (the sources here hold no comment markers inside
    string literals)."""
    if python:
        text = re.sub(r"(?m)^\s*#.*$", "", text)
    else:
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash():
    """Hash of the sources that determine the timed kernels (code only)."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_mqa_logits_amd", name)) as f:
            h.update(strip_comments(f.read(), name.endswith(".py")).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(ctx, next_n, max_ctx, heads, dim, page, sched_bytes, variant="fp8"):
    """Bytes the method must move for one logits call (partial pages not counted).

    fp8: 128 E4M3 bytes + a 4-byte scale per KV token, q 128 B + weight 4 B
    per head.  fp4: 64 packed bytes + 4 E8M0 scales per KV token, q 64 B + 4
    scales + weight 4 B per head.  K is counted once per batch row, up to
    max_ctx tokens (later tokens are truncated, never read)."""
    ctx = np.clip(ctx.astype(np.int64), 0, max_ctx)
    B = len(ctx)
    per_tok = dim + 4 if variant == "fp8" else dim // 2 + dim // 32
    per_head = dim + 4 if variant == "fp8" else dim // 2 + dim // 32 + 4
    k_stream = per_tok * int(ctx.sum())
    table = 4 * int(((ctx + page - 1) // page).sum())      # block-table entries read
    qw = B * next_n * heads * per_head                      # q (+ scales) + fp32 weights
    out = 4 * B * next_n * max_ctx                          # every logit, -inf included
    return k_stream + table + qw + 4 * B + out + sched_bytes


def scored_tokens(ctx, next_n, max_ctx):
    lim = np.repeat(ctx.astype(np.int64), next_n) - next_n + 1 + np.tile(np.arange(next_n), len(ctx))
    return int(np.clip(lim, 0, max_ctx).sum())


def read_traffic(expected_hash, launches_bytes):
    """HBM bytes per launch from the committed counter summary, or None."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    vals = {}
    with open(TRAFFIC_SUMMARY) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_hash") != expected_hash:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_mfma_busy(expected_hash, workload):
    """MFMA busy % of the workload's unit kernel from the committed counter
    summary (a secondary figure), or None when it is missing or stale."""
    if not os.path.exists(MFMA_SUMMARY):
        return None
    ok, val = False, None
    with open(MFMA_SUMMARY) as f:
        for line in f:
            if line.startswith("# kernel source hash"):
                ok = line.rsplit(":", 1)[1].strip() == expected_hash
            elif not line.startswith("#") and line.startswith(workload + ","):
                try:
                    val = float(line.split(",")[3])
                except (IndexError, ValueError):
                    val = None
    return val if ok else None


def cpu_baseline(data, n_rows, seed):
    """Time the fp64 oracle on a fixed random subset of batch rows."""
    from oracle import reference
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = len(os.sched_getaffinity(0))
    B = len(data["context_lens"])
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(B, size=min(n_rows, B), replace=False))
    nn = data["next_n"]
    out_rows = [int(b) * nn + j for b in rows for j in range(nn)]
    t0 = time.perf_counter()
    if data["variant"] == "fp8":
        reference.paged_mqa_logits_fp8(data["q"], data["kv_cache"], data["weights"],
                                       data["context_lens"], data["block_table"],
                                       data["max_context_len"], rows=out_rows)
    else:
        reference.paged_mqa_logits_fp4(data["q"], data["q_scale"], data["kv_cache"],
                                       data["weights"], data["context_lens"],
                                       data["block_table"], data["max_context_len"],
                                       rows=out_rows)
    dt = time.perf_counter() - t0
    toks = scored_tokens(data["context_lens"][rows], nn, data["max_context_len"])
    return {"value": toks / dt, "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"{len(rows)} of {B} rows (seeded), {toks} KV tokens, {dt:.1f} s",
            "cpu": cpu_model(), "blas": blas_name()}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def blas_name():
    try:
        from threadpoolctl import threadpool_info
        libs = [f"{p.get('internal_api')} {p.get('version')}" for p in threadpool_info()
                if p.get("user_api") == "blas"]
        return ", ".join(libs) or None
    except Exception:
        return None


def measure_append(pmqa, torch, batch, reps=20):
    """quantize_append_fp8/fp4 with bf16 input: one token per batch row (a
    decode step) and 2^20 tokens into whole pages placed at random (a
    prefill).  Algorithmic bytes per token: 256 in + 8 slot + the page bytes
    of one token (132 fp8, 68 fp4)."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    out = {}
    stream = torch.cuda.current_stream()
    for variant, page_bytes, fn in (("fp8", pmqa.FP8_PAGE_BYTES, pmqa.quantize_append_fp8),
                                    ("fp4", pmqa.FP4_PAGE_BYTES, pmqa.quantize_append_fp4)):
        for label, n in (("decode", batch), ("prefill", 1 << 20)):
            pages = (n + 63) // 64
            cache = torch.zeros((pages, page_bytes), dtype=torch.uint8, device="cuda")
            k = torch.randn((n, 128), generator=gen, device="cuda").to(torch.bfloat16)
            perm = torch.randperm(pages, generator=gen, device="cuda")
            idx = torch.arange(n, device="cuda")
            slots = perm[idx // 64] * 64 + idx % 64
            fn(k, slots, cache)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn(k, slots, cache)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / reps * 1e3
            alg = n * (256 + 8 + page_bytes // 64)
            out[f"{variant}_{label}"] = {"tokens": n, "us": round(us, 2),
                                         "gbps": round(alg / (us * 1e-6) / 1e9, 1)}
            del cache, k, perm, idx, slots
    return out


def pages_read(ctx, block_table, max_ctx, page):
    """Page ids the logits call reads, in row order: the first
    ceil(min(ctx_b, max_ctx) / page) block-table entries of every row."""
    n = (np.clip(ctx.astype(np.int64), 0, max_ctx) + page - 1) // page
    mask = np.arange(block_table.shape[1])[None, :] < n[:, None]
    return np.ascontiguousarray(block_table[mask].astype(np.int32))


def measure_ceiling(torch, kv_cache, page_bytes, pages, out, reps=10):
    """Streaming ceiling of one call's bytes: the fastest gather of `pages`
    and the fastest non-temporal sweep over `out`, each timed with HIP events
    on the current stream (mean per launch over `reps` back-to-back
    launches)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "paged_mqa_logits_amd", "libpmqa_ceiling.so"))
    lib.pmqa_ceiling_gather.restype = ctypes.c_int
    lib.pmqa_ceiling_gather.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.pmqa_ceiling_fill.restype = ctypes.c_int
    lib.pmqa_ceiling_fill.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_float,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    pg = torch.from_numpy(pages).cuda()
    sink = torch.empty((8 * cus * 256 * 4,), dtype=torch.int32, device="cuda")

    def per_launch_us(fn):
        if fn() != 0:
            raise RuntimeError("ceiling kernel launch refused its arguments")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    g_bytes = int(len(pages)) * page_bytes
    gather = {}
    # waves per SIMD on every compute unit (1-4), and one wave per SIMD on
    # three quarters of them (the fp8 decode kernel's grid)
    for label, blocks in [("0.75w", max(1, 3 * cus // 4))] + [(f"{w}w", cus * w) for w in (1, 2, 3, 4)]:
        for fl in (2, 4):
            us = per_launch_us(lambda: lib.pmqa_ceiling_gather(
                ctypes.c_void_p(kv_cache.data_ptr()), kv_cache.shape[0], page_bytes,
                ctypes.c_void_p(pg.data_ptr()), len(pages), blocks, fl,
                ctypes.c_void_p(sink.data_ptr()), sp))
            gather[f"{label}_{fl}p"] = round(g_bytes / (us * 1e-6) / 1e9, 1)
    f_bytes = out.numel() * 4
    fill = {}
    # (workgroups, threads, stores per round): 1-8 workgroups of 256 threads
    # per compute unit, one store each per round; and fewer writers with 4
    # stores each (one workgroup of 128 threads per 4 compute units is the
    # shape of the library's flat -inf fill)
    shapes = [(cus * w, 256, 1) for w in (1, 2, 4, 8)] + \
             [(max(1, cus // 4), 128, 4), (max(1, 3 * cus // 8), 64, 4), (max(1, cus // 2), 64, 4)]
    for blocks, threads, stores in shapes:
        us = per_launch_us(lambda: lib.pmqa_ceiling_fill(
            ctypes.c_void_p(out.data_ptr()), out.numel(), float("-inf"), blocks, threads, stores,
            sp))
        fill[f"{blocks}b_{threads}t_{stores}s"] = round(f_bytes / (us * 1e-6) / 1e9, 1)
    g_best = max(gather, key=gather.get)
    f_best = max(fill, key=fill.get)
    t = g_bytes / (gather[g_best] * 1e9) + f_bytes / (fill[f_best] * 1e9)
    del pg, sink
    return {"gbps": (g_bytes + f_bytes) / t / 1e9, "us": round(t * 1e6, 1),
            "gather_bytes": g_bytes, "fill_bytes": f_bytes,
            "gather_gbps": gather, "gather_best": g_best,
            "fill_gbps": fill, "fill_best": f_best}


def describe(cfg):
    if cfg.ctx_kind == "lognormal":
        dist = (f"ctx lognormal(median {cfg.ctx_median:g}, sigma {cfg.ctx_sigma:g}) clipped "
                f"[{cfg.ctx_lo}, {cfg.ctx_hi}]")
    else:
        dist = f"ctx uniform [{cfg.ctx_lo}, {cfg.ctx_hi}]"
    zeros = f", {cfg.zero_frac:.0%} empty rows" if cfg.zero_frac else ""
    return (f"{cfg.name}: B={cfg.batch} decode, next_n={cfg.next_n}, {cfg.variant}, "
            f"{cfg.num_heads} heads, "
            f"head_dim 128, 64-token pages, {dist}{zeros}, logits [{cfg.batch * cfg.next_n}, "
            f"{cfg.max_context_len}] fp32; step = graph replay of compute_schedule + "
            f"paged_mqa_logits_{cfg.variant}")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-rows", type=int, default=2048,
                    help="rows of the workload timed on the CPU oracle")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default=WORKLOAD,
                    help="workload name (default: the B=2048 fp8 decode the metric is quoted on)")
    ap.add_argument("--logits-only", action="store_true",
                    help="time only the graph step and the logits call (for profiling runs)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this size "
                         "(reference kernel for rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_mqa_logits_amd as pmqa
    from workloads import CONFIGS, make_workload

    cfg = CONFIGS[args.workload]
    print(f"[bench] generating {args.workload}", file=sys.stderr, flush=True)
    data = make_workload(args.workload)
    fp8 = data["variant"] == "fp8"
    variant = pmqa.VARIANT_FP8 if fp8 else pmqa.VARIANT_FP4
    ctx_np = data["context_lens"]
    M = data["max_context_len"]
    NN = data["next_n"]
    B = len(ctx_np)
    torch.cuda.set_device(0)
    keys = ("q", "kv_cache", "weights", "context_lens", "block_table") + (() if fp8 else ("q_scale",))
    dev = {k: torch.from_numpy(np.ascontiguousarray(data[k])).cuda() for k in keys}
    H = int(data["q"].shape[2])
    W = pmqa.default_num_workers(variant, NN, num_heads=H)
    sched = torch.empty(pmqa.schedule_bytes(B, W) // 4, dtype=torch.int32, device="cuda")
    out = torch.empty((B * NN, M), dtype=torch.float32, device="cuda")

    def logits_call():
        if fp8:
            pmqa.paged_mqa_logits_fp8(dev["q"], dev["kv_cache"], dev["weights"],
                                      dev["context_lens"], dev["block_table"], sched, M, out=out,
                                      num_workers=W)
        else:
            pmqa.paged_mqa_logits_fp4(dev["q"], dev["q_scale"], dev["kv_cache"], dev["weights"],
                                      dev["context_lens"], dev["block_table"], sched, M, out=out,
                                      num_workers=W)

    def step():
        pmqa.compute_schedule(dev["context_lens"], num_workers=W, out=sched)
        logits_call()

    step()
    torch.cuda.synchronize()
    print("[bench] eager step ok; capturing graph", file=sys.stderr, flush=True)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            step()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()

    # A call moving less than 512 MB could be served from the 256 MB MALL on
    # repeat: then a 512 MB scrub write runs between timed calls (outside the
    # timed intervals) so that every call starts from HBM.
    stream = torch.cuda.current_stream()
    sbytes_alg = algorithmic_bytes(ctx_np, NN, M, H, pmqa.HEAD_DIM, pmqa.PAGE_SIZE,
                                   pmqa.schedule_bytes(B, W), data["variant"])
    scrub = (torch.empty((128 << 20,), dtype=torch.float32, device="cuda")
             if sbytes_alg < (512 << 20) else None)

    def timed(fn, n):
        """Per-call durations (ms) of n calls of fn on the stream (after 5
        untimed calls)."""
        for _ in range(5):
            fn()
        if scrub is None:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
            for i in range(n):
                ev[2 * i].record(stream)
                fn()
                ev[2 * i + 1].record(stream)
        else:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
            for i in range(n):
                scrub.fill_(float(i))
                ev[2 * i].record(stream)
                fn()
                ev[2 * i + 1].record(stream)
        torch.cuda.synchronize()
        return np.array([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(n)])

    # The GPU is brought to its working clocks before anything is timed: 50
    # untimed logits calls (~17 ms; a serving loop runs warm).  Measured on
    # MI355X: after the capture's idle sync, whatever was timed first ran
    # 2-3% slow with only the 5 warm-up replays before it (its p90 up to 10%).
    for _ in range(50):
        logits_call()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    if scrub is None:
        # back to back: the steady decode loop, the K replays bracketed by one
        # event on each side (an event recorded between replays costs the
        # stream 5-10 us per replay on MI355X: measured 339 against 345-351 us)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_step = e0.elapsed_time(e1) / args.steps
        # the spread of single steps, from a second pass with an event
        # between replays (each interval includes one event's cost)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        evs[0].record(stream)
        for i in range(args.steps):
            graph.replay()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        step_ms = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    else:
        step_ms = timed(graph.replay, args.steps)
        ms_step = float(step_ms.mean())
    print(f"[bench] graph step {ms_step * 1e3:.1f} us", file=sys.stderr, flush=True)

    # the logits call alone (fill + unit kernel), events on the stream it is launched on
    n_calls = max(args.steps, 50)  # at least 50 timed calls of each measured call
    k_ms = timed(logits_call, n_calls)
    k_mean = float(k_ms.mean())

    # schedule calls alone, back to back on the stream (us per call): the
    # binary search, the linear scan it replaced, and refresh_schedule keeping
    # a fresh schedule or rebuilding a stale one (header word cleared first)
    def per_call_us(fn, n=n_calls):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(5):
            fn()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3

    def extras():
        """Everything beside the graph step and the logits call: schedule
        calls, appends, the top-k step, the decode-drift graph, the streaming
        ceiling and a plain copy."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        spare = torch.empty_like(sched)
        ctx_dev = dev["context_lens"]
        poke = lambda: spare[:1].fill_(0)
        sched_us = {
            "binary": per_call_us(lambda: pmqa.compute_schedule(ctx_dev, num_workers=W, out=spare)),
            "linear": per_call_us(lambda: pmqa.compute_schedule_linear(ctx_dev, num_workers=W,
                                                                       out=spare)),
            "refresh_keep": per_call_us(lambda: pmqa.refresh_schedule(ctx_dev, spare, num_workers=W)),
        }
        sched_us["refresh_rebuild"] = per_call_us(
            lambda: (poke(), pmqa.refresh_schedule(ctx_dev, spare, num_workers=W))) - per_call_us(poke)

        append = measure_append(pmqa, torch, B)

        # the indexer step: logits of the scheduled units, then the top k per row
        # (no -inf fill), and the selection alone on this step's logits
        K_TOP = 2048
        ws = torch.empty_like(out)
        tk_idx = torch.empty((B * NN, K_TOP), dtype=torch.int32, device="cuda")
        tk_val = torch.empty((B * NN, K_TOP), dtype=torch.float32, device="cuda")
        sel_bytes = pmqa.select_workspace_bytes(B * NN, M, K_TOP)
        sel_ws = torch.empty(sel_bytes, dtype=torch.uint8, device="cuda") if sel_bytes else None

        def topk_call():
            if fp8:
                pmqa.paged_mqa_topk_fp8(dev["q"], dev["kv_cache"], dev["weights"],
                                        dev["context_lens"], dev["block_table"], sched, M, K_TOP,
                                        workspace=ws, indices=tk_idx, values=tk_val, num_workers=W,
                                        select_workspace=sel_ws)
            else:
                pmqa.paged_mqa_topk_fp4(dev["q"], dev["q_scale"], dev["kv_cache"], dev["weights"],
                                        dev["context_lens"], dev["block_table"], sched, M, K_TOP,
                                        workspace=ws, indices=tk_idx, values=tk_val, num_workers=W,
                                        select_workspace=sel_ws)

        pmqa.compute_schedule(dev["context_lens"], num_workers=W, out=sched)
        # the schedule and append timings before this leave the GPU nearly
        # idle for ~10 ms: 50 untimed steps bring it back to its working
        # clocks (measured on MI355X, large_fp8: 291-296 us per step right
        # after them, 280-281 us after a run of logits calls)
        for _ in range(50):
            topk_call()
        torch.cuda.synchronize()
        lengths = torch.from_numpy(np.clip(ctx_np.astype(np.int64).repeat(NN) - NN + 1 +
                                           np.tile(np.arange(NN), B), 0, M).astype(np.int32)).cuda()
        topk = {"k": K_TOP,
                "fused_call_us": round(per_call_us(topk_call), 2),
                "select_only_us": round(per_call_us(
                    lambda: pmqa.select_topk(out, lengths, K_TOP, indices=tk_idx, values=tk_val,
                                             select_workspace=sel_ws)), 2),
                "select_single_kernel_us": round(per_call_us(
                    lambda: pmqa.select_topk(out, lengths, K_TOP, indices=tk_idx, values=tk_val,
                                             select_workspace=None)), 2),
                "select_workspace_mb": round(sel_bytes / 2**20, 1)}
        # the selection's algorithmic bytes: every candidate logit read once
        # (4 B) and k index + value pairs written per row (8 B each)
        sel_alg = 4 * int(lengths.to(torch.int64).sum().item()) + 8 * K_TOP * B * NN
        topk["select_algorithmic_bytes"] = sel_alg
        topk["select_frac_of_8tbps"] = round(
            sel_alg / (topk["select_single_kernel_us"] * 1e-6) / (HBM_PEAK_GBPS * 1e9), 4)

        # decode drift: every non-empty row grows by one token per step, so rows
        # cross 256-token boundaries as decoding goes on; the graph refreshes the
        # schedule on the device (rebuilding it when a unit count changed) before
        # the logits call
        ctx_d = dev["context_lens"].clone()
        grow = (ctx_d > 0).to(torch.int32)
        sched_d = torch.empty_like(sched)
        flag = torch.zeros(1, dtype=torch.int32, device="cuda")
        rebuilds = torch.zeros(1, dtype=torch.int32, device="cuda")
        pmqa.compute_schedule(ctx_d, num_workers=W, out=sched_d)

        def drift_step():
            ctx_d.add_(grow)
            pmqa.refresh_schedule(ctx_d, sched_d, num_workers=W, recomputed=flag)
            if fp8:
                pmqa.paged_mqa_logits_fp8(dev["q"], dev["kv_cache"], dev["weights"], ctx_d,
                                          dev["block_table"], sched_d, M, out=ws, num_workers=W)
            else:
                pmqa.paged_mqa_logits_fp4(dev["q"], dev["q_scale"], dev["kv_cache"], dev["weights"],
                                          ctx_d, dev["block_table"], sched_d, M, out=ws,
                                          num_workers=W)
            rebuilds.add_(flag)

        torch.cuda.synchronize()
        dgraph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(dgraph, stream=cap):
                drift_step()
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        for _ in range(5):  # untimed replays (the rows keep growing)
            dgraph.replay()
        torch.cuda.synchronize()
        rebuilds.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            dgraph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        drift = {"steps": args.steps, "us_per_step": round(e0.elapsed_time(e1) / args.steps * 1e3, 1),
                 "schedule_rebuilds": int(rebuilds.item())}
        del dgraph

        # the practical ceiling: the call's page reads and output writes alone
        # (the sweep writes the top-k workspace, an output-sized buffer: `out`
        # keeps the last logits call's result for the parity check below)
        ceiling = measure_ceiling(torch, dev["kv_cache"],
                                  pmqa.FP8_PAGE_BYTES if fp8 else pmqa.FP4_PAGE_BYTES,
                                  pages_read(ctx_np, data["block_table"], M, pmqa.PAGE_SIZE), ws)
        print(f"[bench] ceiling {ceiling['gbps']:.0f} GB/s ({ceiling['us']} us)", file=sys.stderr,
              flush=True)

        # a plain device-to-device copy of 1 GiB on the same box (bytes read + written)
        src = torch.ones((1 << 28,), dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        e0.record(stream)
        for _ in range(5):
            dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        copy_gbps = 2 * src.numel() * 4 / (e0.elapsed_time(e1) / 5 * 1e-3) / 1e9
        del src, dst
        return sched_us, append, topk, drift, ceiling, copy_gbps

    if args.logits_only:
        sched_us = append = topk = drift = ceiling = copy_gbps = None
    else:
        sched_us, append, topk, drift, ceiling, copy_gbps = extras()

    if args.calibration_copy_mib:
        n = args.calibration_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # sampled parity of the last output against the oracle
    from oracle import reference
    bs = [int(np.argmax(ctx_np)), int(np.nonzero(ctx_np == 0)[0][0]) if (ctx_np == 0).any() else 0, 1, B - 1]
    rows = [b * NN + j for b in bs for j in range(NN)]
    if fp8:
        ref = reference.paged_mqa_logits_fp8(data["q"], data["kv_cache"], data["weights"], ctx_np,
                                             data["block_table"], M, rows=rows, want_tol=True)
    else:
        ref = reference.paged_mqa_logits_fp4(data["q"], data["q_scale"], data["kv_cache"],
                                             data["weights"], ctx_np, data["block_table"], M,
                                             rows=rows, want_tol=True)
    got = out[rows].cpu().numpy()
    masked = np.isneginf(ref["logits"])
    ok = bool(np.all(got.view(np.uint32)[masked] == np.uint32(0xFF800000)) and
              np.all(np.abs(got[~masked].astype(np.float64) - ref["logits"][~masked]) <= ref["tol"][~masked]))

    tokens = scored_tokens(ctx_np, NN, M)
    sbytes = pmqa.schedule_bytes(B, W)
    alg = algorithmic_bytes(ctx_np, NN, M, H, pmqa.HEAD_DIM, pmqa.PAGE_SIZE, sbytes,
                            data["variant"])
    achieved = alg / (k_mean * 1e-3) / 1e9
    src_hash = kernel_source_hash()
    traffic = read_traffic(src_hash, alg) if args.workload == WORKLOAD else None

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(data, args.cpu_rows, seed=cfg.seed)

    res = {
        "metric": METRIC,
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": data["variant"],
        "data": "synthetic",
        "config": {
            "workload": describe(cfg),
            "batch": B, "next_n": NN, "max_context_len": M, "kv_tokens_per_step": tokens,
            "num_workers": W, "graph": True,
        },
        "unique_kv_tokens_per_s": (int(np.clip(ctx_np.astype(np.int64), 0, M).sum()) /
                                   (ms_step * 1e-3)) if NN > 1 else None,
        "gbps": alg / (ms_step * 1e-3) / 1e9,
        "mall_scrub": scrub is not None,
        "algorithmic_bytes_per_step": alg,
        "graph_step_us": {"mean": ms_step * 1e3,
                          "evented_mean": float(step_ms.mean()) * 1e3,
                          "median": float(np.median(step_ms)) * 1e3,
                          "p10": float(np.percentile(step_ms, 10)) * 1e3,
                          "p90": float(np.percentile(step_ms, 90)) * 1e3},
        "logits_call_us": {"mean": k_mean * 1e3, "median": float(np.median(k_ms)) * 1e3,
                             "p10": float(np.percentile(k_ms, 10)) * 1e3,
                             "p90": float(np.percentile(k_ms, 90)) * 1e3},
        "decode_drift": drift,
        "schedule_us": {k: round(v, 2) for k, v in sched_us.items()} if sched_us else None,
        "append": append,
        "topk": topk,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": (f"paged_mqa_logits_{data['variant']} = {'neg_inf_fill_flat_kernel' if M % 4 == 0 else 'neg_inf_fill_kernel'} + "
                                f"logits_kernel<{'Fp8' if fp8 else 'Fp4'}Format, {NN}, {H // 16}>"),
                     "kernel_source_hash": src_hash,
                     "copy_gbps": ceiling["gbps"] if ceiling else None,
                     "frac_of_copy": achieved / ceiling["gbps"] if ceiling else None,
                     "torch_copy_gbps": copy_gbps},
        "ceiling": ceiling,
        "mfma_busy_pct": read_mfma_busy(src_hash, args.workload),
        "sampled_parity": ok,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
