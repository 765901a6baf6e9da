"""Reference quantize-and-append of new K tokens into the paged cache.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The page on paged MQA logits consumes a paged K cache in two formats (its
introduction names an fp8 and an fp4 kernel) but does not say how the cache
is written.  The readings used here, the plainest that the consumer's
formats support:

fp8 page (per token, head_dim values):
    amax  = max_i |x_i|                               (fp32, exact)
    scale = amax / 448                                (fp32 division, rounded
                                                        to nearest even)
    code_i = the E4M3fn byte nearest to v_i = x_i / scale (fp32 division),
             |v_i| first clamped to 448, ties to the even code; the sign bit
             follows the sign of v_i (a negative value that rounds to zero is
             the byte 0x80)
    a token with amax = 0 gets scale 0 and every code 0.

MXFP4 page (per block of 32 consecutive values, OCP MX rule):
    e      = floor(log2 amax) - 2   (2 = the largest E2M1 exponent),
             clamped to [-127, 127]; the E8M0 scale byte is e + 127
    code_i = the E2M1 magnitude nearest to |x_i| * 2^-e (exact), ties to the
             even code, saturating at 6; the sign bit is set for a negative
             value with a non-zero magnitude code
    an all-zero block gets scale byte 0 and every code 0.
    Element 2i of a block row is the low nibble of byte i.

Page layouts (the ones the logits kernels read): an fp8 page is 64 tokens x
head_dim E4M3 bytes followed by 64 little-endian fp32 scales; an fp4 page is
64 tokens x head_dim/2 packed bytes followed by 64 x head_dim/32 E8M0 bytes.
A token goes to page slot // 64, row slot % 64; a negative slot is skipped.

Rounding here is a nearest-value search over the decoded code tables of
``formats``, not bit manipulation.  Pins: ``tests/test_oracle_quantize.py``.
"""
import math

import numpy as np

from .formats import e2m1_table, e4m3fn_table

PAGE_TOKENS = 64
FP8_MAX = 448.0

_E4M3_MAG = e4m3fn_table()[:127]          # codes 0..126: every finite magnitude
_E2M1_MAG = e2m1_table()[:8]              # codes 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6


def _nearest_even(mags, a):
    """Index of the magnitude nearest to a (a >= 0, mags ascending), ties to
    the even index; a above the last magnitude maps to the last index."""
    a = np.asarray(a, dtype=np.float64)
    hi = np.clip(np.searchsorted(mags, a, side="left"), 1, len(mags) - 1)
    lo = hi - 1
    dlo = a - mags[lo]
    dhi = mags[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    out = np.where(pick_hi, hi, lo)
    return np.where(a >= mags[-1], len(mags) - 1, out)


def quantize_fp8_token(x):
    """One token's float32 values -> (uint8 codes [D], float32 scale)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    scale = np.float32(amax / np.float32(FP8_MAX))
    if amax == 0:
        return np.zeros(x.shape, dtype=np.uint8), np.float32(0)
    v = (x / scale).astype(np.float32)
    mag = np.minimum(np.abs(v).astype(np.float64), FP8_MAX)
    code = _nearest_even(_E4M3_MAG, mag).astype(np.uint8)
    code |= (np.signbit(v).astype(np.uint8) << 7)
    return code, scale


def mx_scale_exponent(amax):
    """floor(log2 amax) - 2 clamped to [-127, 127]; None for amax == 0."""
    if amax == 0:
        return None
    _, ex = math.frexp(float(amax))      # amax = m * 2^ex, m in [0.5, 1)
    return max(-127, min(127, ex - 1 - 2))


def quantize_mxfp4_token(x):
    """One token's float32 values (D multiple of 32) -> (packed uint8 [D/2],
    E8M0 uint8 [D/32])."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[0]
    codes = np.zeros(D, dtype=np.uint8)
    scales = np.zeros(D // 32, dtype=np.uint8)
    for blk in range(D // 32):
        v = x[32 * blk:32 * blk + 32].astype(np.float64)
        e = mx_scale_exponent(np.max(np.abs(v)))
        if e is None:
            continue
        scales[blk] = e + 127
        mag = _nearest_even(_E2M1_MAG, np.abs(v) * 2.0 ** (-e))
        c = mag.astype(np.uint8)
        c |= ((v < 0) & (c > 0)).astype(np.uint8) << 3
        codes[32 * blk:32 * blk + 32] = c
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    return packed, scales


def append_fp8(kv_cache, k, slots):
    """Write tokens k [n, D] (float32) into a copy of kv_cache
    [pages, 64*D + 4*64] at the given slots; returns the new cache."""
    out = np.array(kv_cache, dtype=np.uint8, copy=True)
    k = np.asarray(k, dtype=np.float32)
    D = k.shape[1]
    for i, slot in enumerate(np.asarray(slots, dtype=np.int64)):
        if slot < 0:
            continue
        page, row = divmod(int(slot), PAGE_TOKENS)
        code, scale = quantize_fp8_token(k[i])
        out[page, row * D:(row + 1) * D] = code
        base = PAGE_TOKENS * D + 4 * row
        out[page, base:base + 4] = np.frombuffer(np.float32(scale).tobytes(), dtype=np.uint8)
    return out


def append_fp4(kv_cache, k, slots):
    """Write tokens k [n, D] (float32) into a copy of kv_cache
    [pages, 64*D/2 + 64*D/32] at the given slots; returns the new cache."""
    out = np.array(kv_cache, dtype=np.uint8, copy=True)
    k = np.asarray(k, dtype=np.float32)
    D = k.shape[1]
    for i, slot in enumerate(np.asarray(slots, dtype=np.int64)):
        if slot < 0:
            continue
        page, row = divmod(int(slot), PAGE_TOKENS)
        packed, scales = quantize_mxfp4_token(k[i])
        out[page, row * (D // 2):(row + 1) * (D // 2)] = packed
        base = PAGE_TOKENS * (D // 2) + row * (D // 32)
        out[page, base:base + D // 32] = scales
    return out
