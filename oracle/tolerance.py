"""Acceptance bound for BF16 results of the GEMM.

Test infrastructure only (see the package docstring).

The pages fix no tolerance. The device accumulates in FP32 (publishing_gemm
page, ``_compile``: ``acc_dtype=Float32``) and rounds once to BF16; the oracle
holds the exact result in float64. A device value passes when

    |device - exact| <= ulp_bf16(exact) + 1e-6 * sum_k |W[n,k] x[t,k]|

where ulp_bf16(v) = 2^(max(floor(log2|v|), -126) - 7) and ulp_bf16(0) = 2^-133.
The first term covers the final rounding (half an ulp, doubled to allow for an
FP32 sum that crosses a binade boundary); the second covers FP32 accumulation
in any order, whose error is of order 2^-24 sqrt(K) times the partial sums
and stays well below 1e-6 of the magnitude sum for K <= 2^16. Values are
compared as numbers, so +0 and -0 are equal.
"""

from __future__ import annotations

import numpy as np

from .codecs import bf16_quantum, bf16_to_f64

REL_ABS_SUM = 1e-6


def bound(exact: np.ndarray, abs_sum: np.ndarray) -> np.ndarray:
    """Per-element bound ulp_bf16(exact) + 1e-6 abs_sum."""
    return bf16_quantum(exact) + REL_ABS_SUM * np.asarray(abs_sum, dtype=np.float64)


def excess(device_bits: np.ndarray, exact: np.ndarray, abs_sum: np.ndarray) -> np.ndarray:
    """|device - exact| / bound, per element (<= 1 passes; inf/nan fail)."""
    dev = bf16_to_f64(np.asarray(device_bits, dtype=np.uint16))
    err = np.abs(dev - np.asarray(exact, dtype=np.float64))
    ratio = err / bound(exact, abs_sum)
    return np.where(np.isfinite(ratio), ratio, np.inf)


def within(device_bits: np.ndarray, exact: np.ndarray, abs_sum: np.ndarray) -> bool:
    """Whether every device BF16 value is within the bound."""
    return bool(np.all(excess(device_bits, exact, abs_sum) <= 1.0))
