"""Pins for the oracle GEMM (CPU only).

Brute force with exact rationals on tiny shapes, closed forms (identity-like W,
all-ones x, a single nonzero pair), invariants (scale shift, negation, K-block
permutation, zero rows) and the hand-worked example under tests/golden/.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import codecs, gemm
from workloads import generate

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _exact(w, ws, x, xs):
    """(C, S): C[t][n] = sum of the products and S[t][n] = sum of their
    magnitudes, as exact Fractions summed term by term."""
    m, k = x.shape
    n = w.shape[0]
    out = [[Fraction(0)] * n for _ in range(m)]
    mag = [[Fraction(0)] * n for _ in range(m)]
    for t in range(m):
        for j in range(n):
            acc = Fraction(0)
            acc_abs = Fraction(0)
            for kk in range(k):
                a = Fraction(codecs.e4m3_value(int(w[j, kk]))) * Fraction(
                    codecs.e8m0_value(int(ws[j, kk // 32])))
                b = Fraction(codecs.e4m3_value(int(x[t, kk]))) * Fraction(
                    codecs.e8m0_value(int(xs[t, kk // 32])))
                acc += a * b
                acc_abs += abs(a * b)
            out[t][j] = acc
            mag[t][j] = acc_abs
    return out, mag


@pytest.mark.parametrize("m,n,k,seed", [(1, 8, 32, 1), (3, 16, 64, 2), (8, 16, 128, 3),
                                        (5, 8, 256, 4), (2, 16, 96, 5)])
def test_brute_force_exact_rationals(m, n, k, seed):
    p = generate.random_problem(seed, m, n, k)
    c, abs_sum = gemm.gemm_f64(p.w, p.ws, p.x, p.xs)
    exact, mag = _exact(p.w, p.ws, p.x, p.xs)
    ex = np.array([[float(v) for v in row] for row in exact])
    ex_abs = np.array([[float(v) for v in row] for row in mag])
    assert c.shape == (m, n) and abs_sum.shape == (m, n)
    assert np.all(np.abs(c - ex) <= 2.0**-50 * ex_abs + 1e-300)
    # The magnitude sum the acceptance bound is scaled by.
    assert np.all(np.abs(abs_sum - ex_abs) <= 2.0**-50 * ex_abs)
    # Rounding the correctly rounded float64 of the exact value gives the
    # oracle's BF16 bits.
    assert np.array_equal(gemm.published_bits(c), gemm.published_bits(ex))


def test_identity_like_weight():
    p = generate.random_problem(8, 4, 64, 128)
    w = np.zeros((64, 128), dtype=np.uint8)
    w[np.arange(64), np.arange(64)] = 0x38  # 1.0
    ws = np.full((64, 4), 127, dtype=np.uint8)
    c, _ = gemm.gemm_f64(w, ws, p.x, p.xs)
    xd = codecs.decode_e4m3(p.x) * np.repeat(codecs.decode_e8m0(p.xs), 32, axis=1)
    assert np.array_equal(c, xd[:, :64])


def test_all_ones_activation():
    p = generate.random_problem(9, 1, 32, 256)
    x = np.full((2, 256), 0x38, dtype=np.uint8)
    xs = np.full((2, 8), 127, dtype=np.uint8)
    c, _ = gemm.gemm_f64(p.w, p.ws, x, xs)
    wd = codecs.decode_e4m3(p.w) * np.repeat(codecs.decode_e8m0(p.ws), 32, axis=1)
    rowsum = np.array([float(sum(Fraction(v) for v in row)) for row in wd])
    assert np.allclose(c[0], rowsum, rtol=0, atol=1e-12 * np.abs(wd).sum(1).max())
    assert np.array_equal(c[0], c[1])


@pytest.mark.parametrize("wn,wk,tk,wc,xc,wsb,xsb", [
    (3, 40, 0, 0x44, 0xB9, 120, 131),
    (0, 0, 0, 0x38, 0x38, 127, 127),
    (15, 127, 3, 0x7E, 0xFE, 100, 160),
    (9, 64, 7, 0x01, 0x08, 127, 127),
])
def test_single_nonzero_pair(wn, wk, tk, wc, xc, wsb, xsb):
    n, k, m = 16, 128, 8
    w = np.zeros((n, k), dtype=np.uint8)
    x = np.zeros((m, k), dtype=np.uint8)
    ws = np.full((n, k // 32), 127, dtype=np.uint8)
    xs = np.full((m, k // 32), 127, dtype=np.uint8)
    w[wn, wk] = wc
    x[tk, wk] = xc
    ws[wn, wk // 32] = wsb
    xs[tk, wk // 32] = xsb
    bits, c, _ = gemm.gemm_publish_bits(w, ws, x, xs)
    prod = (codecs.e4m3_value(wc) * 2.0 ** (wsb - 127)
            * codecs.e4m3_value(xc) * 2.0 ** (xsb - 127))
    expect = np.zeros((m, n))
    expect[tk, wn] = prod
    assert np.array_equal(c, expect)
    # One product of two 4-bit significands has at most 8 significant bits,
    # so it is exact in BF16.
    assert codecs.bf16_to_f64(bits)[tk, wn] == prod
    others = np.ones((m, n), dtype=bool)
    others[tk, wn] = False
    assert np.all(bits[others] == 0)


def test_scale_shift_and_negation():
    p = generate.random_problem(10, 4, 32, 256)
    c, _ = gemm.gemm_f64(p.w, p.ws, p.x, p.xs)
    ws2 = p.ws.copy()
    ws2[5] += 3
    ws2[9] -= 2
    c2, _ = gemm.gemm_f64(p.w, ws2, p.x, p.xs)
    expect = c.copy()
    expect[:, 5] *= 8
    expect[:, 9] /= 4
    assert np.array_equal(c2, expect)
    c3, _ = gemm.gemm_f64(p.w, p.ws, p.x ^ np.uint8(0x80), p.xs)
    assert np.array_equal(c3, -c)


def test_kblock_permutation_changes_only_rounding():
    p = generate.random_problem(12, 3, 16, 512)
    c, abs_sum = gemm.gemm_f64(p.w, p.ws, p.x, p.xs)
    perm = np.random.default_rng(0).permutation(16)
    cols = (perm[:, None] * 32 + np.arange(32)[None, :]).reshape(-1)
    c2, _ = gemm.gemm_f64(p.w[:, cols], p.ws[:, perm], p.x[:, cols], p.xs[:, perm])
    assert np.all(np.abs(c2 - c) <= 512 * 2.0**-53 * abs_sum)


def test_zero_rows_publish_positive_zero():
    p = generate.random_problem(13, 8, 64, 128, dist="stress")
    bits, c, _ = gemm.gemm_publish_bits(p.w, p.ws, p.x, p.xs)
    zr = np.r_[p.meta["zero_rows_pos"], p.meta["zero_rows_neg"]]
    assert np.all(c[:, zr] == 0)
    assert np.all(bits[:, zr] == 0x0000)
    assert not np.any(bits == 0x8000)


def test_published_bits_round_once_then_clear():
    """The epilogue's bits of exact results, worked by hand: one rounding from
    the exact value (not through FP32), ties to even, and negative zero
    cleared after the rounding (a negative result too small for BF16 rounds
    to -0 and is published as +0)."""
    c = np.array([[1.0 + 2.0**-8 + 2.0**-30,   # above a tie: up (FP32 first would tie down)
                   -(1.0 + 2.0**-8),            # a tie: to the even -1
                   1.5 * 2.0**-133,             # between subnormal steps 1 and 2: even 2
                   -(2.0**-140),                # rounds to -0, published as +0
                   0.0, -3.0, 2.0**-126, 448.0]])
    want = [0x3F81, 0xBF80, 0x0002, 0x0000, 0x0000, 0xC040, 0x0080, 0x43E0]
    assert list(gemm.published_bits(c)[0]) == want


def test_shapes_rejected():
    p = generate.random_problem(14, 2, 16, 64)
    with pytest.raises(ValueError):
        gemm.gemm_f64(p.w, p.ws, p.x[:, :32], p.xs[:, :1])
    x9 = np.zeros((9, 64), dtype=np.uint8)
    with pytest.raises(ValueError):
        gemm.gemm_f64(p.w, p.ws, x9, np.zeros((9, 2), dtype=np.uint8))


def _golden_operands(g):
    m, n, k = g["m"], g["n"], g["k"]
    w = np.zeros((n, k), dtype=np.uint8)
    for e in g["w_nonzero"]:
        w[e["row"], e["col"]] = int(e["code"], 16)
    ws = np.array(g["w_scale_bytes"], dtype=np.uint8).reshape(n, 1)
    x = np.array([[int(c, 16)] * k for c in g["x_code_per_token"]], dtype=np.uint8)
    xs = np.array(g["x_scale_per_token"], dtype=np.uint8).reshape(m, 1)
    return w, ws, x, xs


def test_hand_worked_example():
    with open(os.path.join(GOLDEN, "hand_worked_pack.json")) as f:
        g = json.load(f)
    w, ws, x, xs = _golden_operands(g)
    bits, c, _ = gemm.gemm_publish_bits(w, ws, x, xs)
    rounded = codecs.bf16_rne_bits(c)
    expect_r = np.array([[int(v, 16) for v in row] for row in g["rounded_bf16"]],
                        dtype=np.uint16)
    free = np.zeros_like(rounded, dtype=bool)
    for t, j in g["sign_free"]:
        free[t, j] = True
    assert np.array_equal(rounded[~free], expect_r[~free])
    assert np.all((rounded[free] & 0x7FFF) == 0)
    expect_p = np.array([[int(v, 16) for v in row] for row in g["published_bf16"]],
                        dtype=np.uint16)
    assert np.array_equal(bits, expect_p)


# Single products at the ends of the E8M0 range, worked out by hand:
# (W code, W scale byte, x code, x scale byte, product, BF16 bits as rounded).
#   0x01 = 2^-9 (smallest subnormal), 0x09 = 1.125 * 2^-6, 0x38 = 1.0,
#   0x30 = 0.5, 0x78 = 256, 0x7E = 448, 0xB8 = -1.0; scale byte s = 2^(s-127).
EXTREME_PRODUCTS = [
    (0x01, 0, 0x38, 254, 2.0**-9, 0x3B00),            # 2^-136 * 2^127
    (0x09, 0, 0x38, 254, 1.125 * 2.0**-6, 0x3C90),    # 1.125 * 2^-133 * 2^127
    (0x7E, 247, 0x38, 0, 3.5, 0x4060),                # 448 * 2^120 * 2^-127
    (0x78, 247, 0x30, 10, 1024.0, 0x4480),            # 2^128 * 2^-118
    (0x38, 1, 0x38, 253, 2.0**0, 0x3F80),             # 2^-126 * 2^126
    (0xB8, 57, 0x38, 57, -(2.0**-140), 0x8000),       # rounds to -0
    (0x7E, 254, 0x7E, 254, 448.0**2 * 2.0**254, 0x7F80),  # beyond BF16: +inf
]


@pytest.mark.parametrize("wc,wsb,xc,xsb,value,bits", EXTREME_PRODUCTS)
def test_extreme_scale_single_products(wc, wsb, xc, xsb, value, bits):
    """The oracle decodes every scale byte exactly: one product at the E8M0
    extremes has the value and the rounded bits worked out by hand, and the
    published word clears a negative zero."""
    w = np.zeros((8, 64), np.uint8)
    x = np.zeros((1, 64), np.uint8)
    ws = np.full((8, 2), 127, np.uint8)
    xs = np.full((1, 2), 127, np.uint8)
    w[3, 40], ws[3, 1], x[0, 40], xs[0, 1] = wc, wsb, xc, xsb
    c, abs_sum = gemm.gemm_f64(w, ws, x, xs)
    assert c[0, 3] == value and abs_sum[0, 3] == abs(value)
    assert codecs.bf16_rne_bits(c)[0, 3] == bits
    assert gemm.published_bits(c)[0, 3] == (0 if bits == 0x8000 else bits)
    assert np.count_nonzero(c) == 1
