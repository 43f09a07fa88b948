"""The block-scaled GEMM the publishing kernel computes, in float64.

Test infrastructure only (see the package docstring).

publishing_gemm page, module docstring, "GEMM structure": the kernel computes
C[n, m] = sum_k W[n, k] x[m, k] with the weight W [N, K] as the wide operand and
at most 8 activation rows x [m, K]; both are MXFP8 (e4m3fn bytes and one E8M0
scale per 32 consecutive K). The result goes out as BF16 with negative zero
cleared (same docstring, second paragraph). Split-K only changes the order of
the FP32 additions, so it does not appear here.

The oracle is that definition written out:

    C[t, n] = sum_k dec(W[n,k]) 2^(Ws[n,k/32]-127) dec(x[t,k]) 2^(xs[t,k/32]-127)

accumulated in float64 (every product is exact in float64: 4-bit mantissas
and exponents far inside the float64 range), then rounded once to BF16 with
ties to even, then 0x8000 -> 0x0000. The output is laid out [m, N], token-major,
as the linear's output ``out`` of shape (m, n) on the publishing_gemm page
(``PublishingMxfp8Linear.__call__``).
"""

from __future__ import annotations

import numpy as np

from .codecs import (
    bf16_rne_bits,
    clear_negative_zero,
    decode_e4m3,
    decode_e8m0,
)

BLOCK = 32
MAX_ROWS = 8  # at most 8 activation rows (publishing_gemm page, "GEMM structure")


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float64 [rows, K] values of e4m3fn codes [rows, K] with E8M0 scales
    [rows, K/32]: dec(code) * 2^(scale-127)."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    rows, k = codes.shape
    if k % BLOCK or scales.shape != (rows, k // BLOCK):
        raise ValueError("scales must be [rows, K/32]")
    values = decode_e4m3(codes)
    factor = np.repeat(decode_e8m0(scales), BLOCK, axis=1)
    out = values * factor  # exact: a power-of-two scaling
    if not np.all(np.isfinite(out)):
        raise ValueError("the oracle takes finite MXFP8 inputs only")
    return out


def check_shapes(w, ws, x, xs) -> tuple[int, int, int]:
    """(m, N, K) of well-formed operands."""
    n, k = w.shape
    m, kx = x.shape
    if kx != k:
        raise ValueError("W and x disagree on K")
    if not 1 <= m <= MAX_ROWS:
        raise ValueError("the low-batch GEMM takes 1..8 activation rows")
    if ws.shape != (n, k // BLOCK) or xs.shape != (m, k // BLOCK):
        raise ValueError("scale shapes must be [rows, K/32]")
    return m, n, k


def gemm_f64(w, ws, x, xs) -> tuple[np.ndarray, np.ndarray]:
    """(C, abs_sum), both float64 [m, N].

    C[t, n] = sum_k Wd[n, k] xd[t, k] and abs_sum[t, n] = sum_k |Wd[n, k] xd[t, k]|,
    with Wd, xd the dequantized operands. The contraction is a float64 matrix
    product (a library routine); its rounding error is below 2^-53 K abs_sum.
    """
    check_shapes(w, ws, x, xs)
    wd = dequantize(w, ws)
    xd = dequantize(x, xs)
    c = xd @ wd.T
    abs_sum = np.abs(xd) @ np.abs(wd).T
    return c, abs_sum


def published_bits(c: np.ndarray) -> np.ndarray:
    """uint16 [m, N] BF16 bits the epilogue publishes for exact results c:
    round to nearest even once, then clear negative zero."""
    return clear_negative_zero(bf16_rne_bits(c))


def gemm_publish_bits(w, ws, x, xs) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(bits, C, abs_sum): the published BF16 bits [m, N] and the float64
    result and magnitude sum they come from."""
    c, abs_sum = gemm_f64(w, ws, x, xs)
    return published_bits(c), c, abs_sum
