"""Pins of the acceptance bound (oracle.tolerance) and the BF16 spacing it is
built on (oracle.codecs.bf16_quantum), from outside their own formulas:
numpy's float32 spacing, closed forms at the subnormal end, and what the bound
must accept and reject."""

import numpy as np
import pytest

from oracle import codecs, gemm, tolerance


def test_quantum_is_float32_spacing_times_2_16():
    """For normal values a BF16 step is 2^16 float32 steps (BF16 keeps the top
    16 bits of float32): checked against numpy's spacing on many magnitudes."""
    rng = np.random.default_rng(1)
    v = np.ldexp(rng.uniform(1.0, 2.0, 4000), rng.integers(-120, 120, 4000)).astype(np.float32)
    v[::2] *= -1
    want = np.abs(np.spacing(v.astype(np.float32))).astype(np.float64) * 2.0**16
    assert np.array_equal(codecs.bf16_quantum(v.astype(np.float64)), want)


def test_quantum_at_zero_and_subnormals():
    """Below 2^-126 BF16 is subnormal with a fixed step 2^-133, and zero takes it."""
    for v in (0.0, 2.0**-140, 2.0**-130, -2.0**-127, 2.0**-126 - 2.0**-133):
        assert codecs.bf16_quantum(np.array([v]))[0] == 2.0**-133
    assert codecs.bf16_quantum(np.array([2.0**-126]))[0] == 2.0**-133
    assert codecs.bf16_quantum(np.array([1.0]))[0] == 2.0**-7
    assert codecs.bf16_quantum(np.array([1.999]))[0] == 2.0**-7
    assert codecs.bf16_quantum(np.array([2.0]))[0] == 2.0**-6


def _neighbours(exact):
    """The BF16 values just below and just above each exact float64 value."""
    bits = codecs.bf16_rne_bits(exact)
    val = codecs.bf16_to_f64(bits)
    lo = np.where(val <= exact, bits, bits - np.where(exact > 0, 1, -1).astype(np.int64))
    hi = np.where(val >= exact, bits, bits + np.where(exact > 0, 1, -1).astype(np.int64))
    return lo.astype(np.uint16), hi.astype(np.uint16)


def test_both_bf16_neighbours_pass():
    """Either BF16 value adjacent to the exact result is accepted even with no
    accumulation slack (reading A17: no single correct BF16 value)."""
    rng = np.random.default_rng(2)
    exact = rng.normal(size=2000) * np.exp2(rng.integers(-30, 30, 2000))
    exact = exact[np.abs(exact) > 2.0**-120]
    lo, hi = _neighbours(exact)
    zero = np.zeros_like(exact)
    assert tolerance.within(lo, exact, zero) and tolerance.within(hi, exact, zero)


def test_two_steps_off_fails_unless_the_sum_allows_it():
    """A value two BF16 steps beyond the exact result fails with a small
    Sigma|W x|, and passes once 1e-6 Sigma|W x| covers the extra step."""
    exact = np.array([1.0 + 2.0**-9, 3.0 + 2.0**-8, -5.0 - 2.0**-7])
    far = codecs.bf16_rne_bits(exact + 3 * np.sign(exact) * codecs.bf16_quantum(exact))
    assert not tolerance.within(far, exact, np.zeros(3))
    big = 1e6 * 4 * codecs.bf16_quantum(exact)
    assert tolerance.within(far, exact, big)
    ex = tolerance.excess(far, exact, np.zeros(3))
    assert np.all(ex > 2.0) and np.all(ex < 4.0)


def test_the_sum_term_is_one_millionth():
    """The slack is exactly 1e-6 Sigma|W x| on top of one step: a value three
    steps off passes once 1e-6 S reaches the error beyond one step, and fails
    for S a hair smaller."""
    exact = np.array([1.0 + 2.0**-9, -7.0 - 2.0**-6, 2.0**-100 * 1.3])
    far = codecs.bf16_rne_bits(exact + 3 * np.sign(exact) * codecs.bf16_quantum(exact))
    err = np.abs(codecs.bf16_to_f64(far) - exact)
    need = (err - codecs.bf16_quantum(exact)) / 1e-6
    assert np.all(need > 0)
    for i in range(exact.size):
        one = slice(i, i + 1)
        assert tolerance.within(far[one], exact[one], need[one] * (1 + 1e-9))
        assert not tolerance.within(far[one], exact[one], need[one] * (1 - 1e-9))


def test_non_finite_device_values_always_fail():
    exact = np.array([1.0, -2.0, 0.0])
    for bits in (0x7FC0, 0x7F80, 0xFF80):
        dev = np.full(3, bits, dtype=np.uint16)
        assert np.all(np.isinf(tolerance.excess(dev, exact, np.full(3, 1e30))))
        assert not tolerance.within(dev, exact, np.full(3, 1e30))


def test_zero_results_accept_both_signs():
    """Reading A7: +0 and -0 compare equal in c_out."""
    exact = np.zeros(4)
    assert tolerance.within(np.array([0x0000, 0x8000, 0x0000, 0x8000], dtype=np.uint16),
                            exact, np.zeros(4))


def test_check_shapes_rejects_malformed_operands():
    w = np.zeros((16, 64), np.uint8); ws = np.zeros((16, 2), np.uint8)
    x = np.zeros((2, 64), np.uint8); xs = np.zeros((2, 2), np.uint8)
    assert gemm.check_shapes(w, ws, x, xs) == (2, 16, 64)
    with pytest.raises(ValueError):
        gemm.check_shapes(w, ws, np.zeros((2, 32), np.uint8), np.zeros((2, 1), np.uint8))
    with pytest.raises(ValueError):
        gemm.check_shapes(w, ws, np.zeros((9, 64), np.uint8), np.zeros((9, 2), np.uint8))
    with pytest.raises(ValueError):
        gemm.check_shapes(w, np.zeros((16, 3), np.uint8), x, xs)
