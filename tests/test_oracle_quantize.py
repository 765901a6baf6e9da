"""Pins of oracle/quantize.py (the cache producer) against things other than
itself: torch's float8_e4m3fn cast, the input generator's torch-bucketize MX
quantizer, hand-computed ties and saturation, an error bound, and the page
layout the logits oracle decodes."""
import numpy as np
import pytest
import torch

from oracle import formats, quantize as qz
from oracle import reference
from workloads.synth import quantize_mxfp4

E4M3 = formats.e4m3fn_table()


def _torch_e4m3(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_fp8_codes_match_torch_cast():
    rng = np.random.default_rng(0)
    for i in range(200):
        x = (rng.standard_normal(128) * 10.0 ** rng.uniform(-6, 6)).astype(np.float32)
        if i % 7 == 0:
            x[rng.integers(0, 128, 5)] *= -1000.0       # one dominant value
        code, scale = qz.quantize_fp8_token(x)
        assert scale == np.float32(np.max(np.abs(x)) / np.float32(448.0))
        v = np.clip((x / scale).astype(np.float32), -448.0, 448.0)
        assert np.array_equal(code, _torch_e4m3(v)), i


def test_fp8_midpoints_round_to_even_code():
    """Every midpoint between adjacent finite magnitudes, both signs."""
    mids = ((E4M3[:126] + E4M3[1:127]) / 2).astype(np.float32)
    assert np.array_equal((mids.astype(np.float64) * 2), E4M3[:126] + E4M3[1:127])  # exact
    got = qz._nearest_even(E4M3[:127], mids.astype(np.float64))
    want = _torch_e4m3(mids)
    assert np.array_equal(got, want)
    assert np.all(got % 2 == 0)
    assert np.array_equal(_torch_e4m3(-mids), want | 0x80)


def test_fp8_special_tokens():
    code, scale = qz.quantize_fp8_token(np.zeros(128, np.float32))
    assert scale == 0 and not code.any()
    x = np.zeros(128, np.float32)
    x[3] = -2.5
    x[9] = 1e-30                       # rounds to +0
    x[10] = -1e-30                     # rounds to -0: byte 0x80
    code, scale = qz.quantize_fp8_token(x)
    assert scale == np.float32(2.5) / np.float32(448.0)
    assert code[3] == 0xFE             # -448
    assert code[9] == 0x00 and code[10] == 0x80 and code[0] == 0x00


def test_fp8_error_within_half_quantum():
    rng = np.random.default_rng(1)
    for _ in range(50):
        x = rng.standard_normal(128).astype(np.float32) * np.float32(rng.uniform(0.01, 100))
        code, scale = qz.quantize_fp8_token(x)
        v = (x / scale).astype(np.float64)
        deq = E4M3[code]
        mag = np.abs(v)
        # quantum at |v|: 2^-9 below 2^-6, else 2^(floor(log2|v|) - 3)
        q = np.where(mag < 2.0 ** -6, 2.0 ** -9,
                     2.0 ** (np.floor(np.log2(np.maximum(mag, 2.0 ** -6))) - 3))
        assert np.all(np.abs(deq - np.clip(v, -448, 448)) <= q / 2 + 1e-12)
        assert np.max(np.abs(deq)) == 448.0        # the amax element lands on 448


def test_mxfp4_matches_generator_quantizer():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((300, 128)) * 10.0 ** rng.uniform(-8, 8, (300, 1))).astype(np.float32)
    x[5, :32] = 0.0                     # an all-zero block
    x[6, 32:64] = -0.0
    x[7, 64:96] = 6.0 * 2.0 ** -140     # subnormal fp32 values, exponent clamped
    packed_ref, sc_ref = quantize_mxfp4(x)
    for i in range(len(x)):
        packed, sc = qz.quantize_mxfp4_token(x[i])
        assert np.array_equal(sc, sc_ref[i]), i
        assert np.array_equal(packed, packed_ref[i]), i


def test_mxfp4_hand_ties_and_saturation():
    # a block whose amax is 4 (exponent floor(log2 4) - 2 = 0, scale byte 127)
    # so every value is rounded as is
    vals = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 4.0, -0.25, -0.75, -5.0, 0.1]
    want = [0, 2, 2, 4, 4, 6, 6, 6, 0, 0xA, 0xE, 0]      # ties to even, -0.25 -> +0
    x = np.zeros(128, np.float32)
    x[:len(vals)] = vals
    packed, sc = qz.quantize_mxfp4_token(x)
    assert sc[0] == 127 and sc[1] == 0
    codes = np.empty(128, np.uint8)
    codes[0::2], codes[1::2] = packed & 0xF, packed >> 4
    assert codes[:len(vals)].tolist() == want
    # amax 7.9: exponent 0, 7.9 saturates at 6 (code 7); amax 8: exponent 1
    x = np.zeros(128, np.float32)
    x[0], x[32] = 7.9, 8.0
    packed, sc = qz.quantize_mxfp4_token(x)
    assert sc.tolist() == [127, 128, 0, 0]
    assert packed[0] & 0xF == 7 and packed[16] & 0xF == 6    # 8 / 2 = 4


def test_page_writers_place_tokens_where_the_logits_oracle_reads_them():
    """Append three tokens (one skipped), then read them back through the
    logits oracle's own page gathers."""
    rng = np.random.default_rng(3)
    k = rng.standard_normal((3, 128)).astype(np.float32)
    slots = np.array([65, -1, 2], np.int64)          # page 1 row 1, skipped, page 0 row 2
    poison8 = np.full((3, qz.PAGE_TOKENS * 132), 0xA5, np.uint8)
    c8 = qz.append_fp8(poison8, k, slots)
    changed = np.argwhere(c8 != poison8)
    assert set(map(int, np.unique(changed[:, 0]))) <= {0, 1}
    for i, slot in ((0, 65), (2, 2)):
        code, scale = qz.quantize_fp8_token(k[i])
        page, row = divmod(slot, 64)
        vals, sc = reference.gather_fp8_tokens(c8, np.array([page]), row + 1, 64, 128)
        assert np.array_equal(vals[row], formats.decode_e4m3fn(code))
        assert sc[row] == scale
    assert (c8[2] == 0xA5).all()
    poison4 = np.full((3, qz.PAGE_TOKENS * 68), 0x5A, np.uint8)
    c4 = qz.append_fp4(poison4, k, slots)
    for i, slot in ((0, 65), (2, 2)):
        packed, sc = qz.quantize_mxfp4_token(k[i])
        page, row = divmod(slot, 64)
        assert np.array_equal(c4[page, row * 64:(row + 1) * 64], packed)
        assert np.array_equal(c4[page, 4096 + 4 * row:4096 + 4 * row + 4], sc)
        vals = reference.gather_fp4_tokens(c4, np.array([page]), row + 1, 64, 128)
        deq = formats.decode_e2m1_packed(packed) * np.repeat(formats.decode_e8m0(sc), 32)
        assert np.array_equal(vals[row], deq)
    assert (c4[2] == 0x5A).all()


@pytest.mark.parametrize("bad", [np.nan])
def test_fp8_nan_input_is_not_silently_finite(bad):
    """NaN input is outside the producer's contract; the oracle must not
    invent a finite scale for it (the GPU kernel's behaviour is checked only
    on finite inputs)."""
    x = np.ones(128, np.float32)
    x[0] = bad
    _, scale = qz.quantize_fp8_token(x)
    assert np.isnan(scale)
