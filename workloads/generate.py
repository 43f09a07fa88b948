"""Seeded generators for the five workloads of the low-batch MXFP8 GEMM.

The pages print no benchmark or dataset. The workload they describe is the
low-batch attention output projection of a decode step (publishing_gemm page,
module docstring: at most 8 activation rows, the weight as the wide operand,
optional split-K). These generators stand in for it with seeded Gaussian data:

* W and x are float32 Gaussians, quantized to MXFP8 along K (e4m3fn bytes, one
  E8M0 scale per 32 elements, scale exponent = ceil(log2(absmax / 448))).
* "outliers": 1 % of the K channels of x (round(0.01 K) distinct indices) are
  multiplied by 50 in every row before quantization.
* "stress": some W rows are zero (half +0 codes, half -0 codes), odd tokens of
  x are the even tokens with the sign bit flipped, and a few "tiny" W rows hold
  one smallest-subnormal e4m3 value (2^-9) with scale byte 0, in a K column
  where every token's value lies below 1.5 in magnitude, so that each of
  their results is one product below 2^-135 in magnitude, which rounds to
  a BF16 zero of the product's sign.
* Peer payloads for emulated rank slots are BF16 bit patterns of Gaussians
  with about 1 % of halves forced to 0x8000 and some 32-bit words forced to
  0x80000000 (the Lamport sentinel), which the publish must turn into 0.
* BF16 activations (for the in-GEMM quantizer) are the same Gaussians with
  outlier channels, rounded to BF16 (nearest even).
* All-gather payloads are uniform random 32-bit words with about 1 % set to
  the sentinel and 1 % to its near neighbours.

Seeds: 20261202 + 100 * config_index + variant, with variant = m + 16 * split_k
for the N=4096 sweep and 0 otherwise.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BLOCK = 32
SEED_BASE = 20261202


@dataclass
class Problem:
    """One GEMM call's operands (all uint8, row-major, K contiguous)."""

    name: str
    m: int
    n: int
    k: int
    split_k: int
    w: np.ndarray  # [N, K] e4m3fn codes
    ws: np.ndarray  # [N, K/32] E8M0 bytes
    x: np.ndarray  # [m, K] e4m3fn codes
    xs: np.ndarray  # [m, K/32] E8M0 bytes
    seed: int
    meta: dict = field(default_factory=dict)

    @property
    def out_bytes(self) -> int:
        return 2 * self.m * self.n

    def algorithmic_bytes(self) -> int:
        """W, W scales, x, x scales and the published BF16, each moved once."""
        n, k, m = self.n, self.k, self.m
        return n * k + n * k // BLOCK + m * k + m * k // BLOCK + 2 * m * n


# ---------------------------------------------------------------------------
# Vectorized MXFP8 encoder (the input side; the oracle holds its own
# element-by-element quantizer, which a CPU test compares with this one).
# ---------------------------------------------------------------------------


def quantize_mxfp8(values: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Encode a float array [rows, K] as e4m3fn codes [rows, K] and E8M0
    scale bytes [rows, K/32]."""
    v = np.asarray(values, dtype=np.float64)
    rows, k = v.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = v.reshape(rows, k // BLOCK, BLOCK)
    amax = np.max(np.abs(blocks), axis=2)
    _, p = np.frexp(amax)
    e = p.astype(np.int64) - 9
    for _ in range(2):
        e = np.where(448.0 * np.ldexp(1.0, e) < amax, e + 1, e)
    for _ in range(2):
        e = np.where(448.0 * np.ldexp(1.0, e - 1) >= amax, e - 1, e)
    e = np.where(amax == 0.0, -127, e)
    e = np.clip(e, -127, 127)
    scales = (e + 127).astype(np.uint8)

    y = np.ldexp(blocks, -e[:, :, None])
    a = np.abs(y)
    _, pa = np.frexp(a)
    q_exp = np.where(a < 2.0**-6, -9, pa.astype(np.int64) - 4)
    steps = np.rint(np.ldexp(a, -q_exp)).astype(np.int64)  # ties to even
    # steps is 0..8 below 2^-6 (subnormals and the first normal) and 8..16
    # otherwise; one formula gives the code in both ranges, carries included.
    mag = ((q_exp + 10) << 3) + steps - 8
    mag = np.where(steps == 0, 0, mag)
    codes = (mag | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)
    return codes.reshape(rows, k), scales


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

CONFIGS = {
    0: dict(name="tiny", n=256, k=512, m=1, split_k=1, ranks=1, capacity=512,
            dist="normal"),
    1: dict(name="n7168_k2048_m4", n=7168, k=2048, m=4, split_k=1, ranks=1,
            capacity=57344, dist="outliers"),
    2: dict(name="n7168_k8192_m8_s4", n=7168, k=8192, m=8, split_k=4, ranks=1,
            capacity=114688, dist="outliers"),
    3: dict(name="n4096_k16384_sweep", n=4096, k=16384, m=8, split_k=4, ranks=4,
            capacity=65536, dist="normal"),
    4: dict(name="stress_alternating", n=7168, k=4096, m=1, split_k=4, ranks=4,
            capacity=32768, dist="stress",
            sizes=((7168, 4096, 1), (2048, 8192, 8))),
}


def config_seed(index: int, variant: int = 0) -> int:
    return SEED_BASE + 100 * index + variant


def _gaussian(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def _operands(rng, n, k, m, dist):
    """(wq, ws, xq, xs, meta, x): the quantized operands and the float32
    activation they come from."""
    if dist == "outliers":
        w = _gaussian(rng, (n, k), 0.02)
        x = _gaussian(rng, (m, k), 1.0)
        channels = rng.choice(k, size=int(round(0.01 * k)), replace=False)
        x[:, channels] *= np.float32(50.0)
        meta = {"outlier_channels": np.sort(channels)}
    else:
        w = _gaussian(rng, (n, k), 1.0)
        x = _gaussian(rng, (m, k), 1.0)
        meta = {}
    wq, ws = quantize_mxfp8(w)
    xq, xs = quantize_mxfp8(x)
    return wq, ws, xq, xs, meta, x


def _stress(rng, wq, ws, xq, xs, xf):
    """Force exact zeros, negative zeros and BF16-underflowing results.
    xf is the float32 activation before quantization; odd tokens become
    copies of the even ones, so the even rows bound every token."""
    n, k = wq.shape
    m = xq.shape[0]
    rows = rng.choice(n, size=max(2, n // 64) + 8, replace=False)
    zero_rows, tiny_rows = rows[: len(rows) - 8], rows[len(rows) - 8 :]
    half = len(zero_rows) // 2
    wq[zero_rows[:half]] = 0x00
    wq[zero_rows[half:]] = 0x80
    # K columns whose activations all lie below 1.5 in magnitude (below
    # 1.625 once quantized), so that 2^-136 times them stays under 2^-134,
    # half of BF16's smallest step.
    calm = np.flatnonzero(np.max(np.abs(xf[0::2]), axis=0) < 1.5)
    for r in tiny_rows:
        wq[r] = 0x00
        k0 = int(calm[rng.integers(calm.size)])
        wq[r, k0] = 0x01 if rng.integers(2) else 0x81
        ws[r] = 0
    for t in range(1, m, 2):
        xq[t] = xq[t - 1] ^ np.uint8(0x80)
        xs[t] = xs[t - 1]
    return {"zero_rows_pos": np.sort(zero_rows[:half]),
            "zero_rows_neg": np.sort(zero_rows[half:]),
            "tiny_rows": np.sort(tiny_rows)}


def random_problem(seed: int, m: int, n: int, k: int, split_k: int = 1,
                   dist: str = "normal", name: str | None = None) -> Problem:
    """A seeded problem of any shape ("normal", "outliers" or "stress")."""
    rng = np.random.default_rng(seed)
    wq, ws, xq, xs, meta, xf = _operands(rng, n, k, m, "outliers" if dist == "outliers"
                                         else "normal")
    if dist == "stress":
        meta.update(_stress(rng, wq, ws, xq, xs, xf))
    return Problem(name or f"m{m}_n{n}_k{k}_s{split_k}_{dist}", m, n, k, split_k,
                   wq, ws, xq, xs, seed, meta)


EXTREME_SCALE_TARGETS = (0, 1, 2, 3, 127, 246, 247, 250, 254)


def extreme_scales(p: Problem, seed: int) -> Problem:
    """A copy of p with its scale bytes moved to the ends of the E8M0 range.
    Per 32-block column b, W's scale bytes lie at most 3 below a target that
    cycles through EXTREME_SCALE_TARGETS (clamped to 0) and x's within 2 of
    254 minus that target (clamped to 0..254), so each product is the codes'
    product times 2^-5 .. 2^2, finite and far inside the FP32 range, while
    both operands leave the range in which e4m3 * 2^(s-127) is a BF16 value."""
    import copy

    rng = np.random.default_rng(seed)
    q = copy.deepcopy(p)
    nb = p.k // BLOCK
    target = np.array([EXTREME_SCALE_TARGETS[b % len(EXTREME_SCALE_TARGETS)]
                       for b in range(nb)], dtype=np.int64)
    ws = target[None, :] - rng.integers(0, 4, size=(p.n, nb))
    xs = (254 - target)[None, :] + rng.integers(-2, 3, size=(p.m, nb))
    q.ws = np.clip(ws, 0, 254).astype(np.uint8)
    q.xs = np.clip(xs, 0, 254).astype(np.uint8)
    q.name = p.name + "_extreme_scales"
    return q


def config_problem(index: int, m: int | None = None, split_k: int | None = None,
                   size: int = 0, dist: str | None = None) -> Problem:
    """The problem of workload ``index``.

    index 3 takes ``m`` and ``split_k`` (the sweep point); index 4 takes
    ``size`` 0 or 1 (the two alternating shapes); index 2 takes ``dist``
    "outliers" (primary) or "normal" (secondary reading of its distribution).
    """
    cfg = CONFIGS[index]
    if index == 4:
        n, k, mm = cfg["sizes"][size]
        seed = config_seed(index, size)
        return random_problem(seed, mm, n, k, cfg["split_k"], "stress",
                              name=f"stress_{'AB'[size]}_n{n}_k{k}_m{mm}")
    mm = m if m is not None else cfg["m"]
    s = split_k if split_k is not None else cfg["split_k"]
    variant = mm + 16 * s if index == 3 else 0
    d = dist or cfg["dist"]
    if index == 2 and d == "normal":
        variant = 1
    seed = config_seed(index, variant)
    return random_problem(seed, mm, cfg["n"], cfg["k"], s, d,
                          name=f"{cfg['name']}_m{mm}_s{s}_{d}")


def peer_payloads(seed: int, ranks: int, m: int, n: int) -> np.ndarray:
    """uint16 BF16 payloads [ranks - 1, m, n] for emulated rank slots 1..R-1,
    with about 1 % negative-zero halves and some sentinel words."""
    rng = np.random.default_rng(seed ^ 0x5EED)
    count = max(ranks - 1, 0)
    vals = _gaussian(rng, (count, m, n), 1.0)
    bits = (vals.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    flat = bits.reshape(-1)
    if flat.size:
        negz = rng.choice(flat.size, size=max(1, flat.size // 100), replace=False)
        flat[negz] = 0x8000
        words = flat.reshape(-1, 2)
        sent = rng.choice(words.shape[0], size=max(1, words.shape[0] // 500),
                          replace=False)
        words[sent, 0] = 0x0000
        words[sent, 1] = 0x8000
    return bits


def word_payloads(seed: int, ranks: int, words: int) -> np.ndarray:
    """uint32 payloads [ranks, words] for an all-gather of arbitrary words:
    uniform random bits with about 1 % of the words set to the sentinel
    0x80000000 and about 1 % to neighbours of it (0x80000001, 0x7FFFFFFF,
    0x00008000, 0x80008000), so that the word rule meets both."""
    rng = np.random.default_rng(seed ^ 0xA11C)
    out = rng.integers(0, 2**32, size=(ranks, words), dtype=np.uint64).astype(np.uint32)
    flat = out.reshape(-1)
    hits = max(1, flat.size // 100)
    flat[rng.choice(flat.size, size=hits, replace=False)] = 0x80000000
    near = np.array([0x80000001, 0x7FFFFFFF, 0x00008000, 0x80008000], dtype=np.uint32)
    idx = rng.choice(flat.size, size=hits, replace=False)
    flat[idx] = near[rng.integers(0, near.size, size=hits)]
    return out


def bf16_bits(values: np.ndarray) -> np.ndarray:
    """uint16 BF16 patterns of finite float32 values, nearest even (input
    preparation: the activation the quantizer receives is BF16)."""
    b = np.ascontiguousarray(values, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_activation(seed: int, m: int, k: int, dist: str = "outliers") -> np.ndarray:
    """uint16 BF16 activation [m, k]: N(0, 1) values, with "outliers" 1 % of
    the K channels (round(0.01 k) distinct indices) times 50 in every row,
    the same recipe as the MXFP8 activations before quantization."""
    rng = np.random.default_rng(seed ^ 0xBF16)
    x = _gaussian(rng, (m, k), 1.0)
    if dist == "outliers":
        ch = rng.choice(k, size=max(1, round(0.01 * k)), replace=False)
        x[:, ch] *= np.float32(50.0)
    return bf16_bits(x)
