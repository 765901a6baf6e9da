"""Exact decoders for the low-precision element formats, built from bit fields.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The page on paged MQA logits (introduction) names an fp8 kernel and an fp4
kernel but does not define the encodings.  The readings used here are the
standard ones for those names:

* fp8 = OCP FP8 E4M3 "fn" variant: 1 sign, 4 exponent (bias 7), 3 mantissa
  bits, no infinities, S.1111.111 is NaN, largest finite value 448.
* fp4 = OCP MX E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit, no
  infinities or NaN, magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* block scale = OCP MX E8M0: an unsigned biased exponent, value 2^(c-127),
  code 255 is NaN.

Every table holds fp64 values, which represent all of these exactly.

Pins: ``tests/test_oracle_formats.py`` compares every code against torch's
``float8_e4m3fn`` / ``float8_e8m0fnu`` casts (an independent library) and
maps each E2M1 code to the E4M3 code with the same value through torch.
"""
import numpy as np


def e4m3fn_value(code: int) -> float:
    """Value of one E4M3 "fn" byte (sign s, exponent e, mantissa m)."""
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    sign = -1.0 if s else 1.0
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:  # subnormal: m * 2^-3 * 2^(1-7)
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e2m1_value(nibble: int) -> float:
    """Value of one E2M1 nibble (sign s, exponent e, mantissa m)."""
    s = (nibble >> 3) & 1
    e = (nibble >> 1) & 0x3
    m = nibble & 0x1
    sign = -1.0 if s else 1.0
    if e == 0:  # subnormal: m * 2^-1 * 2^(1-1)
        return sign * m * 0.5
    return sign * (1.0 + m / 2.0) * 2.0 ** (e - 1)


def e8m0_value(code: int) -> float:
    """Value of one E8M0 byte: 2^(code-127), or NaN for 255."""
    if code == 0xFF:
        return float("nan")
    return 2.0 ** (code - 127)


def e4m3fn_table() -> np.ndarray:
    """fp64[256]: decoded value of every E4M3fn byte."""
    return np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def e2m1_table() -> np.ndarray:
    """fp64[16]: decoded value of every E2M1 nibble."""
    return np.array([e2m1_value(n) for n in range(16)], dtype=np.float64)


def e8m0_table() -> np.ndarray:
    """fp64[256]: decoded value of every E8M0 byte."""
    return np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """Decode an array of E4M3fn bytes (any shape) to fp64."""
    return e4m3fn_table()[np.asarray(codes, dtype=np.uint8)]


def decode_e2m1_packed(packed: np.ndarray) -> np.ndarray:
    """Decode packed E2M1 bytes [..., n] to fp64 [..., 2n].

    Element 2i is the low nibble of byte i, element 2i+1 the high nibble.
    """
    packed = np.asarray(packed, dtype=np.uint8)
    lut = e2m1_table()
    lo = lut[packed & 0x0F]
    hi = lut[packed >> 4]
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.float64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def decode_e8m0(codes: np.ndarray) -> np.ndarray:
    """Decode an array of E8M0 bytes to fp64."""
    return e8m0_table()[np.asarray(codes, dtype=np.uint8)]
