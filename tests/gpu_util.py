"""Helpers for the GPU tests: upload seeded inputs, call the library through
its Python binding (which calls the C ABI), and bring results back."""
import numpy as np
import torch

import paged_mqa_logits_amd as pmqa


def upload(data):
    dev = {}
    for k in ("q", "q_scale", "kv_cache", "weights", "context_lens", "block_table"):
        if k in data:
            dev[k] = torch.from_numpy(np.ascontiguousarray(data[k])).cuda()
    return dev


# Bit pattern every output element holds before a call: a NaN no kernel
# writes, so a column that no kernel covers fails the comparison.
POISON_BITS = 0x7FC0DEAD


def poisoned_out(rows, max_context_len):
    """[rows, max_context_len] view (row stride rounded up to 4) full of POISON_BITS."""
    ldo = (max_context_len + 3) // 4 * 4
    buf = torch.full((rows, ldo), POISON_BITS, dtype=torch.int32, device="cuda")
    return buf.view(torch.float32)[:, :max_context_len]


def run(data, dev=None, num_workers=None, out=None, schedule=None):
    """Schedule + logits on the GPU; returns (logits float32 numpy, schedule).
    Without `out` the output starts out poisoned."""
    dev = upload(data) if dev is None else dev
    variant = pmqa.VARIANT_FP8 if data["variant"] == "fp8" else pmqa.VARIANT_FP4
    nn = int(data["next_n"])
    if schedule is None:
        schedule = pmqa.compute_schedule(dev["context_lens"], num_workers=num_workers,
                                         variant=variant, next_n=nn,
                                         num_heads=int(data["q"].shape[2]))
    M = int(data["max_context_len"])
    if out is None:
        out = poisoned_out(len(data["context_lens"]) * nn, M)
    if variant == pmqa.VARIANT_FP8:
        lg = pmqa.paged_mqa_logits_fp8(dev["q"], dev["kv_cache"], dev["weights"],
                                       dev["context_lens"], dev["block_table"], schedule, M,
                                       out=out)
    else:
        lg = pmqa.paged_mqa_logits_fp4(dev["q"], dev["q_scale"], dev["kv_cache"],
                                       dev["weights"], dev["context_lens"], dev["block_table"],
                                       schedule, M, out=out)
    torch.cuda.synchronize()
    return lg.cpu().numpy(), schedule


def oracle(data, rows=None):
    from oracle import reference
    if data["variant"] == "fp8":
        return reference.paged_mqa_logits_fp8(data["q"], data["kv_cache"], data["weights"],
                                              data["context_lens"], data["block_table"],
                                              data["max_context_len"], rows=rows, want_tol=True)
    return reference.paged_mqa_logits_fp4(data["q"], data["q_scale"], data["kv_cache"],
                                          data["weights"], data["context_lens"],
                                          data["block_table"], data["max_context_len"],
                                          rows=rows, want_tol=True)


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
