"""Pins of the BF16 activation quantizer in the oracle (oracle.quant.quantize_bf16)
against closed forms, torch's float8 conversion and the inverse property."""

import math

import numpy as np
import pytest

from oracle import codecs, quant

torch = pytest.importorskip("torch")


def _bf16(values) -> np.ndarray:
    """uint16 BF16 bits of float values that BF16 holds exactly."""
    f = np.asarray(values, dtype=np.float32)
    b = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    assert np.array_equal(quant.bf16_bits_to_f64(b), f.astype(np.float64)), "not exact in BF16"
    return b


def test_every_finite_bf16_value_as_block_maximum():
    """Each finite BF16 magnitude as the largest of its block: the scale is
    ceil(log2(amax / 448)) clamped to [-127, 127] (from a float64 logarithm,
    not the oracle's integer search) and the code is torch's e4m3fn conversion
    of amax / 2^e (round to nearest even)."""
    mags = np.arange(0x0001, 0x7F80, dtype=np.uint16)  # positive finite, no zero
    mags = mags[::7]  # 4660 values spread over every exponent
    blocks = np.zeros((mags.size, 32), dtype=np.uint16)
    blocks[:, 5] = mags
    blocks[:, 9] = mags | np.uint16(0x8000)  # the negative twin
    codes, scales = quant.quantize_bf16(blocks.reshape(1, -1))
    codes = codes.reshape(mags.size, 32)
    vals = quant.bf16_bits_to_f64(mags)
    e = np.array([max(-127, min(127, math.ceil(math.log2(v / 448.0)))) for v in vals])
    assert np.array_equal(scales[0].astype(int), e + 127)
    y = torch.tensor(np.ldexp(vals, -e), dtype=torch.float64)
    want = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes[:, 5], want)
    assert np.array_equal(codes[:, 9], want | 0x80)
    others = np.delete(codes, [5, 9], axis=1)
    assert not others.any()  # +0 elements stay code 0


def test_scale_boundaries():
    """amax = 448 * 2^k gives e = k; the next BF16 value above gives k + 1."""
    for k in (-20, -3, 0, 1, 7, 60):
        top = 448.0 * 2.0**k
        above = quant.bf16_bits_to_f64(_bf16([top]) + np.uint16(1))[0]
        assert above > top
        for amax, want in ((top, k), (above, k + 1)):
            blk = np.zeros((1, 32), dtype=np.float32)
            blk[0, 0] = amax
            b = (blk.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
            _, s = quant.quantize_bf16(b)
            assert int(s[0, 0]) == want + 127, (k, amax)


def test_mxfp8_values_come_back_unchanged():
    """Inverse property: values that are exactly MXFP8 (codes times 2^e with
    every block holding a code of magnitude >= 256, so that its amax lies in
    (224, 448] * 2^e) are exact in BF16 and quantize back to the same codes and
    scales, the signs of zeros included."""
    rng = np.random.default_rng(11)
    rows, k = 4, 256
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    codes = rng.choice(finite, size=(rows, k)).astype(np.uint8)
    big = rng.integers(0x78, 0x7F, size=(rows, k // 32)).astype(np.uint8)  # 256..448
    pos = rng.integers(0, 32, size=(rows, k // 32))
    sign = rng.integers(0, 2, size=(rows, k // 32)).astype(np.uint8) << 7
    for r in range(rows):
        for b in range(k // 32):
            codes[r, 32 * b + pos[r, b]] = big[r, b] | sign[r, b]
    scales = rng.integers(127 - 40, 127 + 40, size=(rows, k // 32)).astype(np.uint8)
    vals = np.array([[codecs.e4m3_value(int(c)) for c in row] for row in codes])
    vals = vals * np.repeat(2.0 ** (scales.astype(np.int64) - 127), 32, axis=1)
    bits = _bf16(vals.astype(np.float32))
    got_c, got_s = quant.quantize_bf16(bits)
    assert np.array_equal(got_s, scales)
    assert np.array_equal(got_c, codes)


def test_ties_go_to_even():
    """A value halfway between two e4m3 neighbours rounds to the even code.
    In a block of amax 448 (e = 0): 17 lies between 16 (0x58) and 18 (0x59)
    and becomes 16; 19 lies between 18 and 20 (0x5A) and becomes 20."""
    blk = np.zeros((1, 32), dtype=np.float32)
    blk[0, :4] = [448.0, 17.0, 19.0, -17.0]
    c, s = quant.quantize_bf16(_bf16(blk))
    assert int(s[0, 0]) == 127
    assert list(c[0, :4]) == [0x7E, 0x58, 0x5A, 0xD8]


def test_zero_and_negative_zero():
    blk = np.zeros((1, 64), dtype=np.uint16)
    blk[0, 3] = 0x8000
    blk[0, 40] = _bf16([1.0])[0]
    blk[0, 41] = _bf16([-2.0**-30])[0]  # rounds to zero with its sign
    c, s = quant.quantize_bf16(blk)
    assert int(s[0, 0]) == 0  # an all-zero block: e = -127
    assert c[0, 3] == 0x80 and not np.delete(c[0, :32], 3).any()
    assert int(s[0, 1]) == 127 - 8  # amax 1 -> e = ceil(log2(1/448)) = -8
    assert c[0, 41] == 0x80


def test_subnormal_bf16_inputs_keep_their_value():
    """BF16 subnormals in a block of small amax: e = -127 and the codes are
    the e4m3 values of v * 2^127 (torch's conversion)."""
    mags = np.arange(1, 0x80, dtype=np.uint16)  # every positive BF16 subnormal
    blk = np.zeros((1, 128), dtype=np.uint16)
    blk[0, :mags.size] = mags
    c, s = quant.quantize_bf16(blk)
    assert list(s[0]) == [0, 0, 0, 0]
    y = torch.tensor(np.ldexp(quant.bf16_bits_to_f64(mags), 127), dtype=torch.float64)
    assert np.array_equal(c[0, :mags.size], y.to(torch.float8_e4m3fn).view(torch.uint8).numpy())


def test_non_finite_blocks():
    blk = np.zeros((1, 96), dtype=np.uint16)
    blk[0, 0] = 0x7F80  # +inf
    blk[0, 1] = _bf16([-3.0])[0]
    blk[0, 40] = 0xFFC1  # a negative NaN
    blk[0, 70] = _bf16([5.0])[0]
    c, s = quant.quantize_bf16(blk)
    assert list(s[0]) == [0xFF, 0xFF, 127 - 6]
    assert c[0, 0] == 0x7F and c[0, 1] == 0xFF and c[0, 2] == 0x7F
    assert c[0, 40] == 0xFF and c[0, 41] == 0x7F
