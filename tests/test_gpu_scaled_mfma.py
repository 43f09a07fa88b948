"""Why the GEMM does not use the block-scaled fp8 MFMA (needs an MI355X).

The publishing_gemm page's MXFP8 linear layer contracts e4m3 codes with one
E8M0 scale per 32 K values (PublishingMxfp8Linear._compile, sf_vec_size 32).
gfx950's instruction for that is v_mfma_scale_f32_16x16x128_f8f6f4. These tests
run it and the library's own arithmetic (each code times its scale converted
to an exact BF16 value, then v_mfma_f32_16x16x32_bf16) on the same operands
through mxg_probe_mfma, and compare both with the float64 oracle:

* the scaled instruction sums aligned groups of eight K values and drops a
  product below 2^-13 of the largest one in its group (2^-13 is kept, 2^-14
  lost), while the BF16 path keeps every product exactly;
* over K = 2048, blocks whose large products cancel leave a result made only of
  such small products: the scaled instruction misses it by far more than the
  acceptance bound (1 BF16 ulp + 1e-6 sum|W x|), the BF16 path is exact.

The inputs are fixed and small, so the numbers quoted for this deviation can be
checked by running this file.
"""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ONE = 0x38  # e4m3 1.0
TWO_M6 = 0x08  # e4m3 2^-6 (smallest normal)
TWO_M7 = 0x04  # e4m3 2^-7 (subnormal, 4 * 2^-9)
NEG_ONE = 0xB8


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    from mxfp8_decode_gemm_amd import binding as mx

    torch.cuda.set_device(0)
    return mx


def probe(mx, a, a_scale, b, b_scale, scaled):
    """C[16][16] (FP32) of the device's scaled (True) or BF16 (False) path."""
    k = a.shape[1]
    dev = [torch.from_numpy(np.ascontiguousarray(t)).cuda() for t in (a, a_scale, b, b_scale)]
    c = torch.zeros(256, dtype=torch.float32, device="cuda")
    mx.mxg_probe_mfma(dev[0], dev[1], dev[2], dev[3], k, scaled, c)
    torch.cuda.synchronize()
    return c.cpu().numpy().reshape(16, 16).astype(np.float64)


def oracle(a, a_scale, b, b_scale):
    """Exact C[row][col] = sum_k A[row][k] B[col][k] and its magnitude sum in
    float64: the oracle's GEMM with W = A and the columns of B as activation
    rows, eight at a time (it takes at most eight)."""
    from oracle import gemm

    parts = [gemm.gemm_f64(a, a_scale, b[h:h + 8], b_scale[h:h + 8]) for h in (0, 8)]
    c = np.concatenate([p[0] for p in parts], axis=0).T
    s = np.concatenate([p[1] for p in parts], axis=0).T
    return c, s


def operands(k):
    a = np.zeros((16, k), np.uint8)
    b = np.zeros((16, k), np.uint8)
    a_scale = np.full((16, k // 32), 127, np.uint8)
    b_scale = np.full((16, k // 32), 127, np.uint8)
    return a, a_scale, b, b_scale


@pytest.mark.parametrize("big", [0, 20, 77])
def test_small_products_dropped_in_the_group_of_eight(mx, big):
    """A product of 1 at K position `big` and one product p at every other
    position of a 128-wide step, one case per position (row 0, column 0). The
    scaled instruction sums aligned groups of eight K values: a p = 2^-14 in
    the eight-group of the large product is dropped (the sum stays 1), in any
    other group it is kept; p = 2^-13 is kept everywhere. The BF16 path is
    exact everywhere."""
    group = range(big // 8 * 8, big // 8 * 8 + 8)
    for small_a, small_b, p in [(TWO_M7, TWO_M7, 2.0 ** -14), (TWO_M6, TWO_M7, 2.0 ** -13)]:
        for pos in range(128):
            if pos == big:
                continue
            a, a_scale, b, b_scale = operands(128)
            a[0, big] = ONE
            b[0, big] = ONE
            a[0, pos] = small_a
            b[0, pos] = small_b
            exact, _ = oracle(a, a_scale, b, b_scale)
            assert exact[0, 0] == 1.0 + p
            bf = probe(mx, a, a_scale, b, b_scale, False)
            sc = probe(mx, a, a_scale, b, b_scale, True)
            assert bf[0, 0] == exact[0, 0], (pos, p)  # BF16 path: exact
            dropped = p < 2.0 ** -13 and pos in group
            assert sc[0, 0] == (1.0 if dropped else exact[0, 0]), (big, pos, p, sc[0, 0])
            assert not np.any(bf.ravel()[1:]) and not np.any(sc.ravel()[1:])


def test_group_truncation_counts(mx):
    """1 at K position 0 and n products of 2^-14 at positions 1..n: the seven
    that share the large product's eight-group are lost, the rest kept."""
    for n in range(1, 16):
        a, a_scale, b, b_scale = operands(128)
        a[0, 0] = ONE
        b[0, 0] = ONE
        a[0, 1:1 + n] = TWO_M7
        b[0, 1:1 + n] = TWO_M7
        exact, _ = oracle(a, a_scale, b, b_scale)
        assert exact[0, 0] == 1.0 + n * 2.0 ** -14
        sc = probe(mx, a, a_scale, b, b_scale, True)
        assert sc[0, 0] == 1.0 + max(0, n - 7) * 2.0 ** -14, (n, sc[0, 0])
        assert probe(mx, a, a_scale, b, b_scale, False)[0, 0] == exact[0, 0]


def test_cancelling_blocks_break_the_bound(mx):
    """K = 2048: in each of the 64 scale blocks one product of +1 or -1 (they
    cancel over the row) and 31 products of 2^-14. The exact result is
    64 * 31 * 2^-14 = 0.12109375, a BF16 value; sum|W x| = 64.12, so the
    acceptance bound is 2^-11 + 6.4e-5 = 5.52e-4. The scaled instruction loses
    the 7 small products that share an eight-group with the large one in
    every block and returns 64 * 24 * 2^-14 = 0.09375, 49.5 bounds off; the
    BF16 path returns the exact value."""
    from oracle import tolerance

    k = 2048
    a, a_scale, b, b_scale = operands(k)
    for j in range(k // 32):
        a[0, 32 * j] = ONE
        b[0, 32 * j] = ONE if j % 2 == 0 else NEG_ONE
        a[0, 32 * j + 1:32 * j + 32] = TWO_M7
        b[0, 32 * j + 1:32 * j + 32] = TWO_M7
    exact, abs_sum = oracle(a, a_scale, b, b_scale)
    assert exact[0, 0] == 64 * 31 * 2.0 ** -14
    bnd = float(tolerance.bound(exact[0, 0], abs_sum[0, 0]))
    bf = probe(mx, a, a_scale, b, b_scale, False)
    sc = probe(mx, a, a_scale, b, b_scale, True)
    print(f"exact {exact[0, 0]!r}  bf16 path {bf[0, 0]!r}  scaled fp8 MFMA {sc[0, 0]!r}  "
          f"bound {bnd!r}  scaled error / bound {abs(sc[0, 0] - exact[0, 0]) / bnd:.1f}", flush=True)
    assert bf[0, 0] == exact[0, 0]
    assert sc[0, 0] == 64 * 24 * 2.0 ** -14
    assert abs(sc[0, 0] - exact[0, 0]) > 40 * bnd


def test_random_operands_agree_when_products_are_alike(mx):
    """Sanity of the probe itself: codes of one binade (no product far below
    its block's largest) give the same sums on both paths, equal to the
    oracle's within FP32 accumulation."""
    rng = np.random.default_rng(5)
    k = 512
    a = (0x38 + rng.integers(0, 8, size=(16, k))).astype(np.uint8)  # 1.0 .. 1.875
    b = (0x38 + rng.integers(0, 8, size=(16, k))).astype(np.uint8)
    a_scale = rng.integers(120, 134, size=(16, k // 32)).astype(np.uint8)
    b_scale = rng.integers(120, 134, size=(16, k // 32)).astype(np.uint8)
    exact, abs_sum = oracle(a, a_scale, b, b_scale)
    for scaled in (False, True):
        got = probe(mx, a, a_scale, b, b_scale, scaled)
        assert np.all(np.abs(got - exact) <= 1e-6 * abs_sum), scaled
