"""Pins for the oracle's number formats (CPU only).

e4m3fn and E8M0 decoding are checked code by code against torch's float8
conversions (a library routine) and against hand values; BF16 rounding against
torch's float32 -> bfloat16 conversion, constructed ties, the subnormal range
and the overflow threshold.
"""

import math

import numpy as np
import pytest
import torch

from oracle import codecs


def test_e4m3_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = codecs.decode_e4m3(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    assert np.array_equal(ref[~nan], ours[~nan])
    # The sign of zero is part of the code.
    assert math.copysign(1.0, ours[0x80]) == -1.0


@pytest.mark.parametrize(
    "code,value",
    [(0x38, 1.0), (0x7E, 448.0), (0x01, 2.0**-9), (0x07, 7 * 2.0**-9),
     (0x08, 2.0**-6), (0xB8, -1.0), (0xC0, -2.0), (0x39, 1.125), (0x00, 0.0)],
)
def test_e4m3_hand_values(code, value):
    assert codecs.e4m3_value(code) == value


def test_e8m0_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    ours = codecs.decode_e8m0(np.arange(256, dtype=np.uint8))
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ref[:255], ours[:255])
    assert codecs.e8m0_value(127) == 1.0
    assert codecs.e8m0_value(0) == 2.0**-127
    assert codecs.e8m0_value(254) == 2.0**127


def _torch_bf16_bits(f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(f32.astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_rne_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(1)
    parts = [
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(5000) * 1e-39).astype(np.float32),  # FP32 subnormals
        (rng.standard_normal(5000) * 1e37).astype(np.float32),
        rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ]
    f32 = np.concatenate(parts)
    f32 = f32[np.isfinite(f32)]
    ours = codecs.bf16_rne_bits(f32.astype(np.float64))
    ref = _torch_bf16_bits(f32)
    assert np.array_equal(ours, ref)


def test_bf16_ties_go_to_even():
    one = 1.0
    step = 2.0**-7
    # 1 + step/2 lies halfway between 1 (even) and 1 + step (odd).
    assert codecs.bf16_rne_bits(np.array([one + step / 2]))[0] == 0x3F80
    # 1 + 3 step/2 lies halfway between 1 + step (odd) and 1 + 2 step (even).
    assert codecs.bf16_rne_bits(np.array([one + 1.5 * step]))[0] == 0x3F82
    # Just above a tie rounds up, just below rounds down (float64 resolution).
    assert codecs.bf16_rne_bits(np.array([one + step / 2 + 2.0**-40]))[0] == 0x3F81
    assert codecs.bf16_rne_bits(np.array([one + 1.5 * step - 2.0**-40]))[0] == 0x3F81
    # Negative ties mirror.
    assert codecs.bf16_rne_bits(np.array([-(one + step / 2)]))[0] == 0xBF80


def test_bf16_subnormals_and_underflow():
    q = 2.0**-133
    cases = {q: 0x0001, 2 * q: 0x0002, 0.5 * q: 0x0000, 1.5 * q: 0x0002,
             2.5 * q: 0x0002, 0.25 * q: 0x0000, -0.5 * q: 0x8000, -q: 0x8001,
             2.0**-126: 0x0080, 2.0**-136: 0x0000, -(2.0**-134): 0x8000}
    v = np.array(list(cases))
    assert list(codecs.bf16_rne_bits(v)) == list(cases.values())


def test_bf16_overflow_threshold():
    top = (2.0 - 2.0**-7) * 2.0**127  # largest finite BF16
    thr = codecs.BF16_OVERFLOW
    bits = codecs.bf16_rne_bits(np.array([top, thr - 2.0**100, thr, -thr, 2.0**128]))
    assert list(bits) == [0x7F7F, 0x7F7F, 0x7F80, 0xFF80, 0x7F80]


def test_bf16_rounds_once_from_float64():
    # A value whose float32 rounding lands exactly on a BF16 tie, while the
    # exact value lies above it: rounding through float32 would go down.
    v = 1.0 + 2.0**-8 + 2.0**-30
    assert np.float32(v) == np.float32(1.0 + 2.0**-8)
    assert codecs.bf16_rne_bits(np.array([v]))[0] == 0x3F81


def test_bf16_decode_roundtrip():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    vals = codecs.bf16_to_f64(bits)
    finite = np.isfinite(vals)
    back = codecs.bf16_rne_bits(vals[finite])
    assert np.array_equal(back, bits[finite])


def test_clear_negative_zero():
    bits = np.array([0x8000, 0x0000, 0x8001, 0x3F80, 0x8000], dtype=np.uint16)
    assert list(codecs.clear_negative_zero(bits)) == [0, 0, 0x8001, 0x3F80, 0]
