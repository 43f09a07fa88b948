"""GPU parity at the edges of the arithmetic (needs an MI355X).

* Negative zero through the fused epilogue: a single product of -2^-140 (or
  -2^-135) is an FP32 subnormal that rounds to BF16 -0. The raw output must
  hold 0x8000 there and the published word 0x0000 (publishing_gemm page,
  module docstring: every output is published with negative zero cleared).
* The whole E8M0 range (publishing_gemm page, PublishingMxfp8Linear._compile:
  one Float8E8M0FNU scale per 32 values). Scale bytes 0..2 and 247..254 make
  e4m3 times 2^(s-127) leave the BF16 range. A W row block that leaves it
  at one end only is shifted into it and scaled back after the K loop; any
  other such workgroup takes the exact path: MFMA on the codes, one scale
  block at a time, then ldexp. Single products are exact on both, so the
  device must match the oracle bit for bit. Dense problems with scale bytes
  at both ends (both operands, or shifted W row blocks) must match within
  the tolerance.
* BF16 activations near the BF16 maximum, whose quantized scale byte is 247
  with codes up to 256 (2^128 after scaling).
* A split-K poll that gives up leaves the workspace failed: nothing is
  published until it is armed again, so no stale sum reaches the mailbox.
* The checker catches a rewound epoch: tags are what keep stale pairs out.
"""

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def env():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    from mxfp8_decode_gemm_amd import binding as mx
    from mxfp8_decode_gemm_amd import device as dv

    torch.cuda.set_device(0)
    return mx, dv


def _publish(env, p, split_k, ws=None):
    """One publish + collect of problem p; returns (raw c_out, collected own
    slot, mailbox)."""
    mx, dv = env
    ops = dv.Operands(p)
    mbx = dv.Mailbox(1, p.out_bytes)
    if ws is None and split_k > 1:
        ws = dv.Workspace(p.n, split_k)
    c = torch.empty(p.m * p.n, dtype=torch.int16, device="cuda")
    dv.publish(mbx, ops, split_k, ws, c)
    out = dv.collect(mbx, p.out_bytes)
    torch.cuda.synchronize()
    st = mbx.state_words()
    assert st[mx.STATE_ERROR] == 0 and st[mx.STATE_NEXT] == 1
    if ws is not None:
        assert ws.header()[mx.WS_ERROR] == 0
    return dv.as_u16(c).reshape(p.m, p.n), dv.as_u16(out).reshape(p.m, p.n), mbx


def _check(raw, got, p, bitwise):
    from oracle import codecs, gemm, mailbox, tolerance

    bits, exact, abs_sum = gemm.gemm_publish_bits(p.w, p.ws, p.x, p.xs)
    ex = tolerance.excess(raw, exact, abs_sum)
    assert np.all(ex <= 1.0), f"max excess {ex.max()} at {np.unravel_index(ex.argmax(), ex.shape)}"
    assert np.array_equal(got, codecs.clear_negative_zero(raw))
    assert not mailbox.check_collected(got)
    if bitwise:
        assert np.array_equal(got, bits)
        assert np.array_equal(raw, codecs.bf16_rne_bits(exact))
    return exact


@pytest.mark.parametrize("x16", ["auto", "0"])
@pytest.mark.parametrize("split_k", [1, 4])
@pytest.mark.parametrize("scales", [(57, 57), (1, 118), (118, 1)])
def test_negative_zero_reaches_the_epilogue(env, scales, split_k, x16, monkeypatch):
    """Products of +-2^-140 (scale bytes 57 and 57: the main loop) and
    +-2^-135 (1 and 118: the W row block shifted into range; 118 and 1: the
    exact path) are the only term of their outputs. The raw output holds BF16 -0 (0x8000) for the negative ones
    and +0 for the positive ones; the mailbox holds 0x0000 for both."""
    if x16 == "0":
        monkeypatch.setattr(env[0], "TILE", "fp8")
    from workloads.generate import Problem

    sw, sx = scales
    m, n, k = 8, 64, 512
    w = np.zeros((n, k), np.uint8)
    x = np.zeros((m, k), np.uint8)
    ws = np.full((n, k // 32), 127, np.uint8)
    xs = np.full((m, k // 32), 127, np.uint8)
    sign = {}
    for j, r in enumerate((3, 20, 37, 50, 63)):
        kk = 100 * j + 7 * r % 97
        t = j % m
        w[r, kk] = 0xB8 if j % 2 == 0 else 0x38   # -1.0 or +1.0
        x[t, kk] = 0x38                            # 1.0
        ws[r, kk // 32] = sw
        xs[t, kk // 32] = sx
        sign[(t, r)] = -1 if j % 2 == 0 else 1
    p = Problem("negzero", m, n, k, split_k, w, ws, x, xs, 0)
    _say(f"case negzero scales={scales} split_k={split_k} x16={x16}")
    raw, got, _ = _publish(env, p, split_k)
    exact = _check(raw, got, p, bitwise=True)
    for (t, r), sg in sign.items():
        assert (exact[t, r] < 0) == (sg < 0) and exact[t, r] != 0
        assert raw[t, r] == (0x8000 if sg < 0 else 0x0000), (t, r, hex(raw[t, r]))
        assert got[t, r] == 0
    assert np.count_nonzero(raw == 0x8000) == sum(1 for v in sign.values() if v < 0)


EXTREMES = [0, 1, 2, 3, 246, 247, 254]


def _extreme_singles(seed, mirror, m=8, n=64, k=2048):
    """Row r has one nonzero W code, in its own 32-block r, times one nonzero x
    code of token r % m in the same K column. One side's scale byte cycles
    through EXTREMES, the other compensates (sum 254 +- 3), so every product
    is a normal number with at most 8 significant bits: exact in BF16."""
    from workloads.generate import Problem

    rng = np.random.default_rng(seed)
    w = np.zeros((n, k), np.uint8)
    x = np.zeros((m, k), np.uint8)
    ws = np.full((n, k // 32), 127, np.uint8)
    xs = np.full((m, k // 32), 127, np.uint8)
    pool = np.r_[np.arange(0x01, 0x08), np.arange(0x08, 0x20), np.arange(0x70, 0x7F)]
    for r in range(n):
        b = r % (k // 32)
        kk = 32 * b + int(rng.integers(32))
        t = r % m
        s_ext = EXTREMES[r % len(EXTREMES)]
        s_cmp = int(np.clip(254 - s_ext + rng.integers(-3, 4), 0, 254))
        w[r, kk] = int(rng.choice(pool)) | (0x80 if rng.integers(2) else 0)
        x[t, kk] = int(rng.choice(pool)) | (0x80 if rng.integers(2) else 0)
        if mirror:
            ws[r, b], xs[t, b] = s_cmp, s_ext
        else:
            ws[r, b], xs[t, b] = s_ext, s_cmp
    return Problem(f"extreme_singles_{'x' if mirror else 'w'}", m, n, k, 1, w, ws, x, xs, seed)


@pytest.mark.parametrize("x16", ["auto", "0"])
@pytest.mark.parametrize("split_k", [1, 4])
@pytest.mark.parametrize("mirror", [False, True])
def test_extreme_scales_single_products(env, mirror, split_k, x16, monkeypatch):
    """Scale bytes 0, 1, 2, 3, 246, 247 and 254 on W (or on x), each paired
    with a compensating partner: bit-exact against the oracle."""
    if x16 == "0":
        monkeypatch.setattr(env[0], "TILE", "fp8")
    p = _extreme_singles(900 + 2 * split_k + mirror, mirror)
    p.split_k = split_k
    _say(f"case {p.name} split_k={split_k} x16={x16}")
    raw, got, _ = _publish(env, p, split_k)
    _check(raw, got, p, bitwise=True)
    assert np.count_nonzero(raw) == p.n  # one nonzero result per row


LOW_BLOCK = [0, 1, 2, 3, 50, 120, 200, 240]
HIGH_BLOCK = [247, 250, 254, 246, 200, 120, 60, 14]


def _shifted_singles(seed, m=8, n=128, k=2048):
    """16-row blocks of W alternate between scale bytes reaching below the
    exact range (0, 1, 2 beside in-range bytes up to 240) and above it (247,
    250, 254 beside in-range bytes down to 14). Each block spans at most 240
    binades, so it stays in the main loop with one shift. Row r has one
    nonzero W code in its own 32-block, times one nonzero x code of token
    r % m whose scale byte (kept inside 3..246) puts the product near 2^0:
    a normal number with at most 8 significant bits, so exact."""
    from workloads.generate import Problem

    rng = np.random.default_rng(seed)
    w = np.zeros((n, k), np.uint8)
    x = np.zeros((m, k), np.uint8)
    ws = np.full((n, k // 32), 127, np.uint8)
    xs = np.full((m, k // 32), 127, np.uint8)
    pool = np.r_[np.arange(0x01, 0x08), np.arange(0x08, 0x20), np.arange(0x70, 0x7F)]
    for r in range(n):
        b = r % (k // 32)
        kk = 32 * b + int(rng.integers(32))
        t = r % m
        group = LOW_BLOCK if (r // 16) % 2 == 0 else HIGH_BLOCK
        s_w = group[r % len(group)]
        s_x = int(np.clip(254 - s_w + rng.integers(-3, 4), 3, 246))
        w[r, kk] = int(rng.choice(pool)) | (0x80 if rng.integers(2) else 0)
        x[t, kk] = int(rng.choice(pool)) | (0x80 if rng.integers(2) else 0)
        ws[r, b], xs[t, b] = s_w, s_x
    return Problem("shifted_singles", m, n, k, 1, w, ws, x, xs, seed)


@pytest.mark.parametrize("x16", ["auto", "0"])
@pytest.mark.parametrize("split_k", [1, 4])
def test_shifted_row_blocks_single_products(env, split_k, x16, monkeypatch):
    """W row blocks whose scale bytes leave 3..246 at one end only: bit-exact
    against the oracle (the shift and its undoing lose nothing here)."""
    if x16 == "0":
        monkeypatch.setattr(env[0], "TILE", "fp8")
    p = _shifted_singles(970 + split_k)
    p.split_k = split_k
    _say(f"case {p.name} split_k={split_k} x16={x16}")
    raw, got, _ = _publish(env, p, split_k)
    _check(raw, got, p, bitwise=True)
    assert np.count_nonzero(raw) == p.n


@pytest.mark.parametrize("x16", ["auto", "0"])
@pytest.mark.parametrize("m,n,k,split_k", [(8, 1000, 2048, 1), (8, 1000, 2048, 4),
                                           (1, 512, 4096, 8)])
def test_shifted_row_blocks_dense(env, m, n, k, split_k, x16, monkeypatch):
    """Dense N(0,1) codes. Even 16-row blocks of W take scale bytes 0..5
    everywhere (their results sit around BF16's subnormals); odd ones take
    247..254 in every fourth 32-block column and 100..119 elsewhere. x takes
    scale bytes 3..6 in those columns (so the large products stay near 2^0)
    and 118..122 elsewhere, always inside 3..246. Every W row block leaves
    3..246 at one end only: the shifted main loop, within the tolerance."""
    if x16 == "0":
        monkeypatch.setattr(env[0], "TILE", "fp8")
    from workloads import generate

    p = generate.random_problem(980 + m + split_k, m, n, k, split_k)
    rng = np.random.default_rng(981 + m)
    nb = k // 32
    hi_col = np.arange(nb) % 4 == 0
    ws = np.empty((n, nb), np.int64)
    for rb in range(0, n, 16):
        rows = slice(rb, min(rb + 16, n))
        cnt = rows.stop - rb
        if (rb // 16) % 2 == 0:
            ws[rows] = rng.integers(0, 6, size=(cnt, nb))
        else:
            ws[rows] = np.where(hi_col, 247 + rng.integers(0, 8, size=(cnt, nb)),
                                100 + rng.integers(0, 20, size=(cnt, nb)))
    xs = np.where(hi_col, 3 + rng.integers(0, 4, size=(m, nb)),
                  118 + rng.integers(0, 5, size=(m, nb)))
    p.ws = ws.astype(np.uint8)
    p.xs = xs.astype(np.uint8)
    assert p.ws.min() <= 2 and p.ws.max() >= 247 and 3 <= p.xs.min() and p.xs.max() <= 246
    _say(f"case shifted_dense m={m} n={n} k={k} split_k={split_k} x16={x16}")
    raw, got, _ = _publish(env, p, split_k)
    exact = _check(raw, got, p, bitwise=False)
    assert np.all(np.isfinite(exact))


@pytest.mark.parametrize("x16", ["auto", "0"])
@pytest.mark.parametrize("m,n,k,split_k", [(8, 1000, 2048, 1), (8, 1000, 2048, 4),
                                           (1, 512, 4096, 8), (5, 7168, 2048, 2)])
def test_extreme_scales_dense(env, m, n, k, split_k, x16, monkeypatch):
    """Dense N(0,1) codes with scale bytes at both ends of the E8M0 range on
    both operands (workloads.generate.extreme_scales): within the tolerance."""
    if x16 == "0":
        monkeypatch.setattr(env[0], "TILE", "fp8")
    from workloads import generate

    base = generate.random_problem(950 + m + split_k, m, n, k, split_k)
    p = generate.extreme_scales(base, 951 + m)
    assert p.ws.min() <= 2 and p.ws.max() >= 247 and p.xs.min() <= 2 and p.xs.max() >= 247
    _say(f"case {p.name} split_k={split_k} x16={x16}")
    raw, got, _ = _publish(env, p, split_k)
    _check(raw, got, p, bitwise=False)


@pytest.mark.parametrize("split_k", [1, 4])
def test_bf16_activation_near_the_bf16_maximum(env, split_k):
    """BF16 activations of up to 1.9921875 * 2^127 quantize to scale byte 247
    and codes up to 256 (2^128 after scaling, past BF16): the fused quantizer's
    codes and scales are the oracle's, and the product, through the exact path,
    is within the tolerance."""
    mx, dv = env
    from oracle import gemm, quant, tolerance
    from workloads import generate
    from workloads.generate import Problem

    m, n, k = 4, 512, 2048
    rng = np.random.default_rng(960 + split_k)
    xb = generate.bf16_activation(960, m, k, "normal")
    for t in range(m):  # a few blocks per row hold values near the maximum
        for b in rng.choice(k // 32, size=6, replace=False):
            xb[t, 32 * b:32 * b + 32] = rng.integers(0x7F00, 0x7F80, size=32) | \
                (rng.integers(2, size=32) << 15)
            xb[t, 32 * b + int(rng.integers(32))] = 0x7F7C | (int(rng.integers(2)) << 15)
    # W small enough that every product stays finite (scale bytes 1..8)
    w = rng.integers(0, 0x7F, size=(n, k)).astype(np.uint8) | \
        (rng.integers(2, size=(n, k)) << 7).astype(np.uint8)
    w[(w & 0x7F) == 0x7F] = 0x38
    ws = rng.integers(1, 9, size=(n, k // 32)).astype(np.uint8)
    xq, xsc = quant.quantize_bf16(xb)
    assert xsc.max() == 247
    p = Problem("bf16_near_max", m, n, k, split_k, w, ws, xq, xsc, 960)
    ops = dv.Operands(p)
    mbx = dv.Mailbox(1, p.out_bytes)
    wsp = dv.Workspace(n, split_k) if split_k > 1 else None
    q = torch.empty(m * k, dtype=torch.uint8, device="cuda")
    s = torch.empty(m * k // 32, dtype=torch.uint8, device="cuda")
    c = torch.empty(m * n, dtype=torch.int16, device="cuda")
    _say(f"case bf16_near_max split_k={split_k}")
    mx.mxgemm_publish_bf16(mbx.mb, ops.w, ops.ws, dv.upload(xb), m, n, k, split_k,
                           wsp.buf if wsp else None, wsp.nbytes if wsp else 0, c, q, s)
    got = dv.as_u16(dv.collect(mbx, p.out_bytes)).reshape(m, n)
    torch.cuda.synchronize()
    assert mbx.state_words()[mx.STATE_ERROR] == 0
    assert np.array_equal(q.cpu().numpy().reshape(m, k), xq)
    assert np.array_equal(s.cpu().numpy().reshape(m, k // 32), xsc)
    raw = dv.as_u16(c).reshape(m, n)
    _, exact, abs_sum = gemm.gemm_publish_bits(w, ws, xq, xsc)
    assert np.all(np.isfinite(exact))
    assert tolerance.within(raw, exact, abs_sum)
    from oracle import codecs

    assert np.array_equal(got, codecs.clear_negative_zero(raw))


def test_splitk_timeout_is_fatal_to_the_workspace(env):
    """A split-K poll forced to give up (poll limit 1, set from the host; every
    kernel exits normally) sets MXG_ERR_SPLITK_SPIN. The next call on that
    workspace publishes nothing, so its collect times out and hands back the
    sentinel instead of sums of pairs that may be stale. Arming the workspace
    and the mailbox again restores parity."""
    mx, dv = env
    from oracle import codecs, gemm, tolerance
    from workloads import generate

    p = generate.config_problem(2)
    ops = dv.Operands(p)
    mbx = dv.Mailbox(1, p.out_bytes)
    ws = dv.Workspace(p.n, 4)
    c = torch.empty(p.m * p.n, dtype=torch.int16, device="cuda")
    _say("case forced split-K timeout, N=7168 K=8192 m=8 S=4")
    # With a poll limit of 1 a wait gives up unless its words are already
    # there at the first look, which a call can happen to meet everywhere:
    # calls (each one published and collected) until one gives up.
    mbx.spin_limit = 1
    for _ in range(16):
        dv.publish(mbx, ops, 4, ws, c)
        dv.collect(mbx, p.out_bytes)
        torch.cuda.synchronize()
        if ws.header()[mx.WS_ERROR] & mx.ERR_SPLITK_SPIN:
            break
    assert ws.header()[mx.WS_ERROR] & mx.ERR_SPLITK_SPIN
    # the next call: nothing published, the collect gives up (short limit)
    mbx.spin_limit = 256
    dv.publish(mbx, ops, 4, ws, c)
    out = dv.collect(mbx, p.out_bytes)
    torch.cuda.synchronize()
    words = out.view(torch.int32).cpu().numpy().view(np.uint32)
    assert np.all(words == 0x80000000)
    assert mbx.state_words()[mx.STATE_ERROR] & mx.ERR_COLLECT_SPIN
    # armed again: parity
    mx.mxgemm_workspace_init(ws.buf, ws.nbytes)
    mbx.reinit()
    dv.publish(mbx, ops, 4, ws, c)
    got = dv.as_u16(dv.collect(mbx, p.out_bytes)).reshape(p.m, p.n)
    torch.cuda.synchronize()
    raw = dv.as_u16(c).reshape(p.m, p.n)
    _, exact, abs_sum = gemm.gemm_publish_bits(p.w, p.ws, p.x, p.xs)
    assert tolerance.within(raw, exact, abs_sum)
    assert np.array_equal(got, codecs.clear_negative_zero(raw))
    assert ws.header()[mx.WS_ERROR] == 0 and mbx.state_words()[mx.STATE_ERROR] == 0


def test_rewound_epoch_is_caught(env):
    """Checker mutation on the device: rewinding the workspace's EPOCH from the
    host after a call makes the previous call's pairs carry a live tag, and a
    call on other data then sums some of them. The parity check must see it
    (and nothing hangs: the stale tags satisfy every poll). Five tries, at
    least one caught."""
    mx, dv = env
    from oracle import gemm, tolerance
    from workloads import generate

    a = generate.config_problem(2, dist="outliers")
    b = generate.config_problem(2, dist="normal")
    ops = [dv.Operands(a), dv.Operands(b)]
    exact = [gemm.gemm_publish_bits(p.w, p.ws, p.x, p.xs)[1:] for p in (a, b)]
    mbx = dv.Mailbox(1, a.out_bytes)
    ws = dv.Workspace(a.n, 4)
    c = torch.empty(a.m * a.n, dtype=torch.int16, device="cuda")
    caught = 0
    for i in range(5):
        _say(f"rewind try {i}")
        dv.publish(mbx, ops[i % 2], 4, ws, c)
        dv.collect(mbx, a.out_bytes)
        torch.cuda.synchronize()
        epoch = int(ws.header()[mx.WS_EPOCH])
        ws.buf[mx.WS_EPOCH] = epoch - 1  # the tag of the call just made
        dv.publish(mbx, ops[(i + 1) % 2], 4, ws, c)
        dv.collect(mbx, a.out_bytes)
        torch.cuda.synchronize()
        raw = dv.as_u16(c).reshape(a.m, a.n)
        ex, s = exact[(i + 1) % 2]
        if not tolerance.within(raw, ex, s):
            caught += 1
    assert caught >= 1
    assert ws.header()[mx.WS_ERROR] == 0
