"""Pins for oracle/formats.py: exhaustive comparison with independent decoders."""
import numpy as np
import pytest
import torch

from oracle import formats


def _torch_decode(codes, dtype):
    t = torch.tensor(codes, dtype=torch.uint8)
    return t.view(dtype).float().double().numpy()


def test_e4m3fn_exhaustive_matches_torch():
    mine = formats.e4m3fn_table()
    ref = _torch_decode(list(range(256)), torch.float8_e4m3fn)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(mine[~nan], ref[~nan])
    # signed zero is kept
    assert np.signbit(mine[0x80]) and not np.signbit(mine[0x00])


def test_e4m3fn_anchors():
    t = formats.e4m3fn_table()
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0       # largest finite
    assert t[0x01] == 2.0 ** -9                          # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9                      # largest subnormal
    assert t[0x08] == 2.0 ** -6                          # smallest normal
    assert t[0x38] == 1.0 and t[0xB8] == -1.0
    assert t[0x44] == 3.0 and t[0x30] == 0.5


def test_e8m0_exhaustive_matches_torch():
    mine = formats.e8m0_table()
    ref = _torch_decode(list(range(256)), torch.float8_e8m0fnu)
    assert np.isnan(mine[255]) and np.isnan(ref[255])
    assert np.array_equal(mine[:255], ref[:255])
    assert mine[127] == 1.0 and mine[0] == 2.0 ** -127 and mine[254] == 2.0 ** 127


def test_e2m1_matches_e4m3_through_torch():
    """Each E2M1 code re-encoded as the E4M3 code of the same value (sign kept,
    exponent re-biased from 1 to 7, mantissa bit moved to the top of the 3-bit
    field) must decode to the same number through torch's float8_e4m3fn."""
    mine = formats.e2m1_table()
    for n in range(16):
        s, e, m = n >> 3, (n >> 1) & 3, n & 1
        if e == 0 and m == 0:
            code = s << 7                                 # signed zero
        elif e == 0:
            code = (s << 7) | (6 << 3)                    # 0.5 = 2^-1
        else:
            code = (s << 7) | ((e + 6) << 3) | (m << 2)
        ref = _torch_decode([code], torch.float8_e4m3fn)[0]
        assert mine[n] == ref, (n, mine[n], ref)


def test_e2m1_table_is_the_ocp_magnitude_list():
    t = formats.e2m1_table()
    assert list(t[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(t[8:]) == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_e2m1_packed_nibble_order():
    # byte 0x21: low nibble 1 (0.5) is element 0, high nibble 2 (1.0) element 1
    out = formats.decode_e2m1_packed(np.array([[0x21, 0xF7]], np.uint8))
    assert out.tolist() == [[0.5, 1.0, 6.0, -6.0]]


@pytest.mark.parametrize("code", [0x00, 0x55, 0x7E, 0x80, 0xC1])
def test_decode_array_shape(code):
    a = np.full((2, 3), code, np.uint8)
    assert formats.decode_e4m3fn(a).shape == (2, 3)
