"""The per-32 MXFP8 quantizer, element by element.

Test infrastructure only (see the package docstring).

The pages hand the GEMM activations and weights that are already MXFP8
(publishing_gemm page: ``PublishingMxfp8Linear.__call__`` takes a quantized
activation; the weight carries ``weight_scale``). How the bytes were produced
is not on the pages; the synthetic workloads quantize float32 values this way,
one E8M0 scale per 32 consecutive elements along K:

* e = the smallest integer with amax <= 448 * 2^e, where amax is the block's
  largest magnitude (this is ceil(log2(amax / 448)) computed without a
  floating-point logarithm); an all-zero block takes e = -127; e is clamped to
  [-127, 127] and the scale byte is e + 127.
* every element becomes the e4m3fn value nearest to v / 2^e, ties to even,
  with gradual underflow (subnormal spacing 2^-9). |v / 2^e| <= 448 by the
  choice of e, so no element saturates. The sign of a value that rounds to
  zero is kept (code 0x80 for negative values).

This module loops in pure Python and is meant for small arrays; it pins the
vectorized input generator bit for bit.

``quantize_bf16`` is the activation quantizer in front of the GEMM
(publishing_gemm page, ``PublishingMxfp8Linear.__call__``: the activation is
an MXFP8 QuantizedActivation whose original dtype is BF16). The pages do not
print the quantizer; it applies the rule above to the BF16 values, which are
exact in float64. Reading for what the rule leaves open: a block whose largest
magnitude is infinite or NaN gets scale byte 0xFF (the E8M0 NaN) and every
code of the block is the e4m3fn NaN 0x7F with the element's sign bit.
"""

from __future__ import annotations

import math

import numpy as np

from .codecs import E4M3_MAX, e4m3_value

BLOCK = 32

# value -> code for every finite e4m3fn code (both zeros kept apart by sign).
_CODE_OF = {}
for _c in range(256):
    _v = e4m3_value(_c)
    if not math.isnan(_v):
        _CODE_OF[(_v, math.copysign(1.0, _v))] = _c


def block_exponent(amax: float) -> int:
    """Smallest integer e with amax <= 448 * 2^e, clamped to [-127, 127]."""
    if amax < 0 or math.isnan(amax) or math.isinf(amax):
        raise ValueError("amax must be a finite magnitude")
    if amax == 0.0:
        return -127
    _, p = math.frexp(amax)  # amax = f 2^p, 0.5 <= f < 1, so 2^(p-1) <= amax < 2^p
    e = p - 9  # 448 2^(p-9) = 0.875 2^p is within a factor of two of amax
    while E4M3_MAX * math.ldexp(1.0, e) < amax:
        e += 1
    while E4M3_MAX * math.ldexp(1.0, e - 1) >= amax:
        e -= 1
    return max(-127, min(127, e))


def e4m3_round(y: float) -> int:
    """e4m3fn code of the value nearest to y (ties to even); |y| <= 448."""
    if math.isnan(y) or abs(y) > E4M3_MAX:
        raise ValueError("value outside the e4m3fn range")
    a = abs(y)
    if a < 2.0**-6:
        quantum = 2.0**-9  # subnormal spacing, also the spacing of [2^-6, 2^-5)
    else:
        _, p = math.frexp(a)  # 2^(p-1) <= a < 2^p
        quantum = math.ldexp(1.0, (p - 1) - 3)
    steps = a / quantum  # exact: power-of-two scaling
    n = math.floor(steps)
    frac = steps - n
    if frac > 0.5 or (frac == 0.5 and n % 2 == 1):
        n += 1
    r = math.copysign(n * quantum, y)
    return _CODE_OF[(r, math.copysign(1.0, r))]


def quantize_mxfp8(values: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Quantize a [rows, K] float array (K a multiple of 32) to e4m3fn codes
    [rows, K] and E8M0 scale bytes [rows, K/32]."""
    values = np.asarray(values)
    rows, k = values.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 32")
    codes = np.zeros((rows, k), dtype=np.uint8)
    scales = np.zeros((rows, k // BLOCK), dtype=np.uint8)
    for r in range(rows):
        for b in range(k // BLOCK):
            block = [float(v) for v in values[r, b * BLOCK : (b + 1) * BLOCK]]
            e = block_exponent(max(abs(v) for v in block))
            scales[r, b] = e + 127
            for j, v in enumerate(block):
                codes[r, b * BLOCK + j] = e4m3_round(math.ldexp(v, -e))
    return codes, scales


E8M0_NAN = 0xFF
E4M3_NAN = 0x7F


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """float64 values of uint16 BF16 bit patterns (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # NaN patterns widen to NaN
        return b.view(np.float32).astype(np.float64)


def quantize_bf16(bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Quantize a [rows, K] array of BF16 bit patterns (uint16) to e4m3fn codes
    [rows, K] and E8M0 scale bytes [rows, K/32]: finite blocks as
    quantize_mxfp8, non-finite blocks as the reading in the module docstring."""
    bits = np.asarray(bits, dtype=np.uint16)
    rows, k = bits.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 32")
    vals = bf16_bits_to_f64(bits)
    codes = np.zeros((rows, k), dtype=np.uint8)
    scales = np.zeros((rows, k // BLOCK), dtype=np.uint8)
    for r in range(rows):
        for b in range(k // BLOCK):
            sl = slice(b * BLOCK, (b + 1) * BLOCK)
            if np.all(np.isfinite(vals[r, sl])):
                c, sc = quantize_mxfp8(vals[r:r + 1, sl])
                codes[r, sl] = c[0]
                scales[r, b] = sc[0, 0]
            else:
                sign = (bits[r, sl] >> np.uint16(8)).astype(np.uint8) & np.uint8(0x80)
                codes[r, sl] = sign | np.uint8(E4M3_NAN)
                scales[r, b] = E8M0_NAN
    return codes, scales
