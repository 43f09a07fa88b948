"""Pins of the all-reduce consumer in the oracle (oracle.mailbox.allreduce_bf16
and MailboxModel.collect_sum) against facts fixed outside its own formula:
identities, exact integer and rational sums, the FP32 order of additions, and
the mailbox invariants."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import codecs, mailbox


def _bits(values):
    """BF16 bits of exactly representable float values."""
    return codecs.bf16_bits_from_value(np.asarray(values, dtype=np.float64))


def test_one_rank_is_the_identity():
    rng = np.random.default_rng(1)
    v = codecs.bf16_round_value(rng.standard_normal(512) * 10.0 ** rng.integers(-6, 6, 512))
    h = _bits(v)
    assert np.array_equal(mailbox.allreduce_bf16(h[None, :]), h)


@pytest.mark.parametrize("ranks", [2, 3, 8])
def test_small_integers_sum_exactly(ranks):
    rng = np.random.default_rng(ranks)
    ints = rng.integers(-32, 33, size=(ranks, 256))
    h = np.stack([_bits(row.astype(np.float64)) for row in ints])
    got = codecs.bf16_to_f64(mailbox.allreduce_bf16(h))
    assert np.array_equal(got, ints.sum(axis=0).astype(np.float64))


def test_exact_rational_sum_rounded_once():
    """With the ranks' exponents within 12 of each other every FP32 partial
    sum of 8-bit significands is exact, so the result is the exact rational
    sum rounded once to BF16, computed here with Fractions and ties to even."""
    rng = np.random.default_rng(7)
    for _ in range(200):
        base = int(rng.integers(-20, 20))
        vals = []
        for _r in range(int(rng.integers(2, 9))):
            sig = int(rng.integers(128, 256)) * (1 if rng.random() < 0.5 else -1)
            vals.append(Fraction(sig) * Fraction(2) ** (base + int(rng.integers(0, 5)) - 7))
        exact = sum(vals, Fraction(0))
        h = np.stack([_bits([float(v)]) for v in vals])
        got = mailbox.allreduce_bf16(h)
        # Round the rational to BF16 by hand: 8 significant bits, ties to even.
        if exact == 0:
            want = 0.0
        else:
            mag = abs(exact)
            e = 0
            while mag >= 2:
                mag /= 2
                e += 1
            while mag < 1:
                mag *= 2
                e -= 1
            scaled = abs(exact) / Fraction(2) ** (e - 7)  # in [128, 256)
            fl = scaled.numerator // scaled.denominator
            rem = scaled - fl
            if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
                fl += 1
            want = float(fl) * 2.0 ** (e - 7) * (1 if exact > 0 else -1)
        assert codecs.bf16_to_f64(got)[0] == want, (vals, exact)


def test_fp32_order_of_additions():
    """2^24 + 1 - 2^24 in FP32, left to right: the 1 is lost in the first
    addition (the exact sum 1 would be the float64 answer)."""
    h = np.stack([_bits([2.0**24]), _bits([1.0]), _bits([-(2.0**24)])])
    assert codecs.bf16_to_f64(mailbox.allreduce_bf16(h))[0] == 0.0
    h2 = np.stack([_bits([1.0]), _bits([2.0**24]), _bits([-(2.0**24)])])
    assert codecs.bf16_to_f64(mailbox.allreduce_bf16(h2))[0] == 0.0
    h3 = np.stack([_bits([2.0**24]), _bits([-(2.0**24)]), _bits([1.0])])
    assert codecs.bf16_to_f64(mailbox.allreduce_bf16(h3))[0] == 1.0


def test_cancellation_gives_positive_zero():
    h = np.stack([_bits([3.5, -0.25]), _bits([-3.5, 0.25])])
    assert list(mailbox.allreduce_bf16(h)) == [0x0000, 0x0000]


def test_fp32_result_rounds_to_bf16_nearest_even():
    """1 + 2^-8 is exactly between BF16 1 and 1 + 2^-7 (ties to even: 1);
    1 + 3 * 2^-8 is between 1 + 2^-7 and 1 + 2^-6 (ties to even: 1 + 2^-6)."""
    h = np.stack([_bits([1.0, 1.0]), _bits([2.0**-8, 3 * 2.0**-8])])
    got = codecs.bf16_to_f64(mailbox.allreduce_bf16(h))
    assert list(got) == [1.0, 1.0 + 2.0**-6]


def test_collect_sum_resets_and_advances():
    mb = mailbox.MailboxModel(3, 64)
    a = _bits(np.arange(8, dtype=np.float64))
    mb.publish(0, a)
    mb.publish(1, a)
    with pytest.raises(mailbox.WouldSpin):
        mb.collect_sum(16)
    mb.publish(2, a)
    got = mb.collect_sum(16)
    assert np.array_equal(codecs.bf16_to_f64(got), 3 * np.arange(8, dtype=np.float64))
    assert mb.next == 1 and mb.idle()
