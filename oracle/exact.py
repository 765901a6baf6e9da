"""Rational brute force for paged MQA logits on tiny inputs.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

This is a second, deliberately different way of computing the definition in
``oracle/reference.py`` (page "[flashinfer] ... Paged MQA Logits ...",
introduction: head scores passed through ReLU, weighted and summed), used to pin that
module.  It shares none of its code:

* element decoding goes through torch's ``float8_e4m3fn`` / ``float8_e8m0fnu``
  casts (a library) and, for E2M1, through the magnitude table printed in the
  OCP Microscaling Formats v1.0 specification (0, 0.5, 1, 1.5, 2, 3, 4, 6);
* every token is located on its own (page = block_table[b, t // page_size],
  slot = t % page_size) instead of concatenating pages;
* all arithmetic is exact ``fractions.Fraction`` arithmetic, summed in plain
  Python loops.

It also gives, for every scored entry, the exact magnitude sum
``sum_h |w_h| * |scale_t * q_h . k_t|`` on which the per-entry parity bound
of the reference rests (the bound is 2e-3 times it plus 1e-6).

Cost is O(rows * tokens * H * D) Python operations: keep inputs tiny.
"""
from fractions import Fraction

import numpy as np
import torch

_E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)  # OCP MX v1.0


def _fp8_values(codes) -> list:
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(codes, np.uint8)).reshape(-1))
    return [Fraction(float(v)) for v in t.view(torch.float8_e4m3fn).float().tolist()]


def _e8m0_values(codes) -> list:
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(codes, np.uint8)).reshape(-1))
    return [Fraction(float(v)) for v in t.view(torch.float8_e8m0fnu).float().tolist()]


def _e2m1_value(nib: int) -> Fraction:
    mag = Fraction(_E2M1_MAGNITUDES[nib & 7])
    return -mag if nib & 8 else mag


def _fp4_row_values(packed, scales, D) -> list:
    """Values of one D-element MXFP4 vector given its D/2 bytes and D/32 scales."""
    sc = _e8m0_values(scales)
    vals = []
    for d in range(D):
        byte = int(packed[d // 2])
        nib = byte & 0xF if d % 2 == 0 else byte >> 4
        vals.append(_e2m1_value(nib) * sc[d // 32])
    return vals


def _score(row_q, k_vals, scale, w_row):
    """(logit, magnitude sum) of one entry, both exact."""
    total = Fraction(0)
    mag = Fraction(0)
    for h, qh in enumerate(row_q):
        dot = Fraction(0)
        for a, b in zip(qh, k_vals):
            dot += a * b
        x = scale * dot
        wh = Fraction(float(w_row[h]))
        if x > 0:
            total += wh * x
        mag += abs(wh) * abs(x)
    return total, mag


def _limit(ctx, next_n, j, M):
    return min(ctx - next_n + 1 + j, M)


def entries_fp8(q, kv_cache, weights, context_lens, block_table, max_context_len,
                page_size=64):
    """Exact (logit, magnitude sum) pairs (list of lists; None marks a -inf
    entry) for the fp8 variant."""
    B, NN, H, D = q.shape
    out = []
    for b in range(B):
        L = int(context_lens[b])
        for j in range(NN):
            r = b * NN + j
            qrow = [_fp8_values(q[b, j, h]) for h in range(H)]
            lim = _limit(L, NN, j, max_context_len)
            row = []
            for t in range(max_context_len):
                if t >= lim:
                    row.append(None)
                    continue
                page = kv_cache[int(block_table[b, t // page_size])]
                slot = t % page_size
                kv = _fp8_values(page[slot * D:(slot + 1) * D])
                off = page_size * D + 4 * slot
                scale = Fraction(float(np.frombuffer(page[off:off + 4].tobytes(), "<f4")[0]))
                row.append(_score(qrow, kv, scale, weights[r]))
            out.append(row)
    return out


def entries_fp4(q, q_scale, kv_cache, weights, context_lens, block_table,
                max_context_len, page_size=64):
    """Exact (logit, magnitude sum) pairs (list of lists; None marks -inf)
    for the MXFP4 variant."""
    B, NN, H, Dh = q.shape
    D = 2 * Dh
    nblk = D // 32
    vbytes = page_size * Dh
    out = []
    for b in range(B):
        L = int(context_lens[b])
        for j in range(NN):
            r = b * NN + j
            qrow = [_fp4_row_values(q[b, j, h], q_scale[b, j, h], D) for h in range(H)]
            lim = _limit(L, NN, j, max_context_len)
            row = []
            for t in range(max_context_len):
                if t >= lim:
                    row.append(None)
                    continue
                page = kv_cache[int(block_table[b, t // page_size])]
                slot = t % page_size
                kv = _fp4_row_values(page[slot * Dh:(slot + 1) * Dh],
                                     page[vbytes + slot * nblk:vbytes + (slot + 1) * nblk], D)
                row.append(_score(qrow, kv, Fraction(1), weights[r]))
            out.append(row)
    return out


def _part(rows, i):
    return [[None if e is None else e[i] for e in row] for row in rows]


def logits_fp8(*args, **kw):
    """Exact logits (list of lists; None marks a -inf entry) for the fp8 variant."""
    return _part(entries_fp8(*args, **kw), 0)


def bounds_fp8(*args, **kw):
    """Exact sum_h |w_h| |scale_t q_h . k_t| per scored entry (None where masked)."""
    return _part(entries_fp8(*args, **kw), 1)


def logits_fp4(*args, **kw):
    """Exact logits (list of lists; None marks -inf) for the MXFP4 variant."""
    return _part(entries_fp4(*args, **kw), 0)


def bounds_fp4(*args, **kw):
    """Exact sum_h |w_h| |q_h . k_t| per scored entry of the MXFP4 variant."""
    return _part(entries_fp4(*args, **kw), 1)
