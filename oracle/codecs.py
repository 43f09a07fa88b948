"""Number formats of the publishing GEMM, written out from their definitions.

Test infrastructure only (see the package docstring).

* e4m3fn data and E8M0 per-32 scales: the publishing_gemm page passes the weight
  and the activation as Float8E4M3FN bytes with Float8E8M0FNU scales, one scale
  per 32 elements along K (``PublishingMxfp8Linear.__call__`` and ``_compile``,
  ``sf_vec_size=32``). The values follow the OCP MX formats: e4m3fn has one
  sign bit, four exponent bits with bias 7, three mantissa bits, subnormals at
  exponent field 0, no infinities, and NaN only at S.1111.111; E8M0 is a
  biased power of two, 2^(s-127), with 255 as NaN.
* BF16 output: the epilogue rounds every FP32 result to BF16 (publishing_gemm
  page, module docstring and ``epilog_warp``). Round-to-nearest-even is the
  rounding; the oracle rounds the exact float64 value once.
* Negative-zero clearing: every published BF16 value has negative zero cleared
  (publishing_gemm page, module docstring; ``publish_value`` sanitizes each pack
  before the store). A BF16 half equal to 0x8000 becomes 0x0000, which also
  means no published 32-bit word can equal the Lamport sentinel 0x80000000
  (all_gather page, module docstring, step 1).
"""

from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0
SENTINEL_U32 = 0x80000000
BF16_NEG_ZERO = 0x8000


def e4m3_value(code: int) -> float:
    """Exact value of one e4m3fn byte (float64; NaN for 0x7F / 0xFF)."""
    if not 0 <= code <= 255:
        raise ValueError("an e4m3 code is one byte")
    sign = -1.0 if code >> 7 else 1.0
    exponent = (code >> 3) & 0xF
    mantissa = code & 0x7
    if exponent == 0xF and mantissa == 0x7:
        return math.nan
    if exponent == 0:
        return sign * mantissa * 2.0**-9
    return sign * (1.0 + mantissa / 8.0) * 2.0 ** (exponent - 7)


def e8m0_value(code: int) -> float:
    """Exact value of one E8M0 scale byte, 2^(code-127) (NaN for 255)."""
    if not 0 <= code <= 255:
        raise ValueError("an E8M0 code is one byte")
    if code == 255:
        return math.nan
    return math.ldexp(1.0, code - 127)


# Lookup tables built from the scalar closed forms above.
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E8M0_TABLE = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """float64 values of an array of e4m3fn bytes."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError("e4m3 codes must be uint8")
    return E4M3_TABLE[codes]


def decode_e8m0(codes: np.ndarray) -> np.ndarray:
    """float64 values of an array of E8M0 scale bytes."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError("E8M0 codes must be uint8")
    return E8M0_TABLE[codes]


# ---------------------------------------------------------------------------
# BF16: 1 sign bit, 8 exponent bits (bias 127), 7 mantissa bits.
# Normal numbers (1 + M/128) 2^E for E in [-126, 127]; subnormals M 2^-133.
# ---------------------------------------------------------------------------

BF16_MIN_EXP = -126
BF16_MANT_BITS = 7
BF16_OVERFLOW = (2.0 - 2.0**-8) * 2.0**127  # halfway between max finite and 2^128


def bf16_quantum(v: np.ndarray) -> np.ndarray:
    """Spacing of BF16 numbers at |v|: 2^(max(floor(log2|v|), -126) - 7).

    For v == 0 this is the subnormal spacing 2^-133.
    """
    v = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(v)  # v = f 2^e with 0.5 <= f < 1, so floor(log2 v) = e - 1
    floor_log2 = np.where(v == 0.0, BF16_MIN_EXP, e - 1)
    return np.ldexp(1.0, np.maximum(floor_log2, BF16_MIN_EXP) - BF16_MANT_BITS)


def bf16_round_value(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest BF16 number, ties to even.

    Returns float64 values that are exactly BF16-representable (+-inf on
    overflow). The division by the quantum is a power-of-two scaling and
    ``np.rint`` rounds half to even, so every step is exact.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("the oracle rounds finite values only")
    q = bf16_quantum(v)
    r = np.rint(v / q) * q
    # Rounding can carry into the next binade; that result is still exact.
    big = np.abs(v) >= BF16_OVERFLOW
    r = np.where(big, np.copysign(np.inf, v), r)
    # Keep the sign of values that round to zero (IEEE rounding keeps it).
    return np.copysign(r, v)


def bf16_bits_from_value(r: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float64 values that are exact BF16 numbers."""
    r = np.asarray(r, dtype=np.float64)
    f32 = r.astype(np.float32)
    if not np.array_equal(f32.astype(np.float64), r, equal_nan=True):
        raise ValueError("value is not exactly representable in BF16")
    bits = f32.view(np.uint32)
    if np.any(bits & 0xFFFF):
        raise ValueError("value is not exactly representable in BF16")
    return (bits >> 16).astype(np.uint16)


def bf16_rne_bits(v: np.ndarray) -> np.ndarray:
    """BF16 bits of round-to-nearest-even(v), rounded once from float64."""
    return bf16_bits_from_value(bf16_round_value(v))


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """float64 values of uint16 BF16 bit patterns."""
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("BF16 bits must be uint16")
    with np.errstate(invalid="ignore"):  # NaN payloads stay NaN
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def clear_negative_zero(bits: np.ndarray) -> np.ndarray:
    """BF16 bits with every 0x8000 (negative zero) replaced by 0x0000."""
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("BF16 bits must be uint16")
    return np.where(bits == BF16_NEG_ZERO, np.uint16(0), bits).astype(np.uint16)
