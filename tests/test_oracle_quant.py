"""Pins for the MXFP8 quantizer and the input generator (CPU only).

The oracle's element-by-element quantizer is checked against its defining
properties and against torch's float32 -> float8_e4m3fn conversion (a library
routine); the vectorized encoder in ``workloads`` must then agree with it bit
for bit.
"""

import math

import numpy as np
import pytest
import torch

from oracle import codecs, quant
from workloads import generate


def _blocks(seed):
    rng = np.random.default_rng(seed)
    rows = [
        rng.standard_normal(256),
        rng.standard_normal(256) * 0.02,
        rng.standard_normal(256) * 1e-30,
        rng.standard_normal(256) * 1e30,
        np.zeros(256),
        np.where(rng.random(256) < 0.5, 0.0, -0.0),
        np.r_[np.full(32, 448.0), np.full(32, -448.0), rng.standard_normal(192)],
        rng.standard_normal(256) * np.where(rng.random(256) < 0.05, 50.0, 1.0),
    ]
    return np.stack(rows).astype(np.float32)


def test_scale_is_the_smallest_power_of_two():
    vals = _blocks(3).astype(np.float64)
    codes, scales = quant.quantize_mxfp8(vals)
    for r in range(vals.shape[0]):
        for b in range(vals.shape[1] // 32):
            amax = np.max(np.abs(vals[r, 32 * b : 32 * b + 32]))
            e = int(scales[r, b]) - 127
            if amax == 0:
                assert e == -127
                continue
            assert amax <= 448.0 * 2.0**e
            assert e == -127 or amax > 448.0 * 2.0 ** (e - 1)


def test_elements_round_to_nearest_e4m3():
    vals = _blocks(4).astype(np.float64)
    codes, scales = quant.quantize_mxfp8(vals)
    deq = codecs.decode_e4m3(codes) * np.repeat(codecs.decode_e8m0(scales), 32, axis=1)
    # Every other e4m3 value, scaled the same way, is no closer.
    finite = codecs.E4M3_TABLE[~np.isnan(codecs.E4M3_TABLE)]
    for r in range(vals.shape[0]):
        for j in range(0, vals.shape[1], 7):
            s = 2.0 ** (int(scales[r, j // 32]) - 127)
            err = abs(deq[r, j] - vals[r, j])
            best = np.min(np.abs(finite * s - vals[r, j]))
            assert err == best


def test_e4m3_round_matches_torch():
    rng = np.random.default_rng(5)
    y = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(20000) * 2.0**-7,
        np.array([448.0, -448.0, 2.0**-10, -(2.0**-10), 3 * 2.0**-11, 0.0]),
    ]).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([quant.e4m3_round(float(v)) for v in y], dtype=np.uint8)
    # torch keeps -0 for negative values that round to zero, as the oracle does.
    assert np.array_equal(ours, ref)


def test_e4m3_ties_to_even():
    # 1 + 1/16 lies halfway between 1 (0x38, even) and 1.125 (0x39, odd).
    assert quant.e4m3_round(1.0 + 1 / 16) == 0x38
    # 1.125 + 1/16 lies halfway between 0x39 (odd) and 0x3A (even).
    assert quant.e4m3_round(1.125 + 1 / 16) == 0x3A
    # Subnormal tie: 1.5 * 2^-9 goes to 2 * 2^-9 (code 0x02).
    assert quant.e4m3_round(1.5 * 2.0**-9) == 0x02
    assert quant.e4m3_round(0.5 * 2.0**-9) == 0x00
    assert quant.e4m3_round(-0.5 * 2.0**-9) == 0x80


def test_representable_values_roundtrip():
    for c in range(256):
        v = codecs.e4m3_value(c)
        if math.isnan(v):
            continue
        assert quant.e4m3_round(v) == c


@pytest.mark.parametrize("seed", [6, 7])
def test_input_encoder_matches_oracle_quantizer(seed):
    vals = _blocks(seed)
    c_ref, s_ref = quant.quantize_mxfp8(vals)
    c_gen, s_gen = generate.quantize_mxfp8(vals)
    assert np.array_equal(s_gen, s_ref)
    assert np.array_equal(c_gen, c_ref)


def test_generated_problem_is_seeded_and_finite():
    a = generate.config_problem(0)
    b = generate.config_problem(0)
    assert a.seed == b.seed == generate.config_seed(0)
    assert np.array_equal(a.w, b.w) and np.array_equal(a.x, b.x)
    for codes in (a.w, a.x):
        assert not np.any((codes & 0x7F) == 0x7F)  # no NaN codes
    assert not np.any(a.ws == 255) and not np.any(a.xs == 255)
    assert a.w.shape == (256, 512) and a.x.shape == (1, 512)
    assert a.algorithmic_bytes() == 136208


def test_stress_structure():
    p = generate.random_problem(11, 8, 512, 256, 4, "stress")
    assert np.all(p.w[p.meta["zero_rows_pos"]] == 0x00)
    assert np.all(p.w[p.meta["zero_rows_neg"]] == 0x80)
    for r in p.meta["tiny_rows"]:
        assert np.count_nonzero(p.w[r] & 0x7F) == 1 and np.all(p.ws[r] == 0)
    for t in range(1, 8, 2):
        assert np.array_equal(p.x[t], p.x[t - 1] ^ 0x80)
        assert np.array_equal(p.xs[t], p.xs[t - 1])


@pytest.mark.parametrize("m", [1, 8])
def test_stress_tiny_rows_round_to_signed_zeros(m):
    """The stress recipe's tiny rows: every result is a single product that
    rounds to a BF16 zero, and some of them to negative zero, which the
    publish must clear."""
    from oracle import codecs, gemm

    p = generate.random_problem(13 + m, m, 512, 1024, 4, "stress")
    c, _ = gemm.gemm_f64(p.w, p.ws, p.x, p.xs)
    raw = codecs.bf16_rne_bits(c[:, p.meta["tiny_rows"]])
    assert np.all((raw & 0x7FFF) == 0)
    assert np.any(raw == 0x8000)
    assert np.all(gemm.published_bits(c[:, p.meta["tiny_rows"]]) == 0)


def test_peer_payloads_hold_sentinels_and_negative_zeros():
    bits = generate.peer_payloads(1, 4, 8, 4096)
    assert bits.shape == (3, 8, 4096) and bits.dtype == np.uint16
    words = bits.reshape(-1, 2)
    assert np.any((words[:, 0] == 0) & (words[:, 1] == 0x8000))
    assert np.count_nonzero(bits == 0x8000) >= bits.size // 100
