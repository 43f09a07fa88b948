"""GPU parity of the activation quantizer (mxfp8_quantize, and the one inside
mxgemm_publish_bf16) against the CPU oracle (oracle.quant.quantize_bf16):
codes and scales bit-exact. The fused GEMM is checked three ways: the
quantized activation it writes out equals the oracle's, its BF16 output is
bit-identical to mxgemm_publish on the oracle's codes, and its values are
within the tolerance of the oracle's float64 GEMM. The plain GEMM (mxgemm)
followed by mailbox_publish reproduces the fused publish bit for bit."""

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


def _quantize_dev(env, bits):
    mx, dv = env
    rows, k = bits.shape
    x = dv.upload(bits)
    q = torch.empty(rows * k, dtype=torch.uint8, device="cuda")
    s = torch.empty(rows * k // 32, dtype=torch.uint8, device="cuda")
    mx.mxfp8_quantize(x, rows, k, q, s)
    torch.cuda.synchronize()
    return q.cpu().numpy().reshape(rows, k), s.cpu().numpy().reshape(rows, k // 32)


@pytest.mark.parametrize("rows,k,dist", [(8, 8192, "outliers"), (3, 96, "normal"),
                                         (1, 32, "normal"), (8, 1024, "normal")])
def test_quantize_matches_oracle(env, rows, k, dist):
    from oracle import quant
    from workloads import generate

    _say(f"case rows={rows} k={k} dist={dist}")
    bits = generate.bf16_activation(500 + rows + k, rows, k, dist)
    q, s = _quantize_dev(env, bits)
    wq, ws = quant.quantize_bf16(bits)
    assert np.array_equal(s, ws)
    assert np.array_equal(q, wq)


def test_quantize_every_bf16_pattern(env):
    """All 65536 BF16 patterns, twice: in order (each block of 32 holds 32
    neighbouring patterns, so every block maximum class and every normal code
    occurs), and shuffled behind one large value per block (small values
    against a large scale: e4m3 subnormals and zeros of both signs). Blocks
    with an infinity or NaN take the NaN reading."""
    from oracle import quant

    allp = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    rng = np.random.default_rng(9)
    shuffled = rng.permutation(allp).reshape(-1, 32)
    big = rng.integers(0x3C00, 0x4800, size=shuffled.shape[0]).astype(np.uint16)  # 2^-7..2^17
    shuffled[:, 0] = big | (rng.integers(0, 2, size=big.size).astype(np.uint16) << 15)
    bits = np.stack([allp, shuffled.reshape(-1)])
    q, s = _quantize_dev(env, bits)
    wq, ws = quant.quantize_bf16(bits)
    assert np.array_equal(s, ws)
    assert np.array_equal(q, wq)
    assert (s == 0xFF).any() and (q == 0x80).any()  # the special classes occurred


def _fused_case(env, p, xbits, split_k, ranks=1):
    """mxgemm_publish_bf16 on BF16 x: returns (codes, scales, c_out bits,
    collected) from the device."""
    mx, dv = env
    ops = dv.Operands(p)
    mbx = dv.Mailbox(ranks, p.out_bytes)
    ws = dv.Workspace(p.n, split_k) if split_k > 1 else None
    x = dv.upload(xbits)
    q = torch.empty(p.m * p.k, dtype=torch.uint8, device="cuda")
    s = torch.empty(p.m * p.k // 32, dtype=torch.uint8, device="cuda")
    c = torch.empty(p.m * p.n, dtype=torch.int16, device="cuda")
    mx.mxgemm_publish_bf16(mbx.mb, ops.w, ops.ws, x, p.m, p.n, p.k, split_k,
                           ws.buf if ws else None, ws.nbytes if ws else 0, c, q, s)
    got = dv.as_u16(dv.collect(mbx, p.out_bytes)).reshape(p.m, p.n)
    torch.cuda.synchronize()
    st = mbx.state_words()
    assert st[mx.STATE_NEXT] == 1 and st[mx.STATE_ERROR] == 0
    return (q.cpu().numpy().reshape(p.m, p.k), s.cpu().numpy().reshape(p.m, p.k // 32),
            dv.as_u16(c).reshape(p.m, p.n), got, ops, ws)


@pytest.mark.parametrize("m,n,k,split_k,dist", [
    (8, 1000, 1024, 1, "normal"), (1, 512, 2048, 4, "outliers"), (5, 2056, 4096, 4, "outliers"),
    (8, 1024, 8192, 8, "normal"), (3, 7168, 2048, 2, "outliers"), (8, 7168, 8192, 4, "outliers"),
    # a K slice that takes more than one quantizing round, staged as BF16
    (8, 7168, 16384, 4, "outliers"),
])
def test_fused_quantizer_gemm(env, m, n, k, split_k, dist):
    mx, dv = env
    from oracle import gemm, mailbox, quant, tolerance
    from workloads import generate

    _say(f"case m={m} n={n} k={k} split_k={split_k} dist={dist}")
    p = generate.random_problem(700 + m + n + split_k, m, n, k, split_k, dist)
    xbits = generate.bf16_activation(p.seed, m, k, dist)
    q, s, raw, got, ops, ws = _fused_case(env, p, xbits, split_k)
    wq, wsc = quant.quantize_bf16(xbits)
    assert np.array_equal(s, wsc)
    assert np.array_equal(q, wq)
    # Same codes through the MXFP8 path: the same bits.
    c2 = torch.empty(m * n, dtype=torch.int16, device="cuda")
    mbx2 = dv.Mailbox(1, p.out_bytes)
    mx.mxgemm_publish(mbx2.mb, ops.w, ops.ws, dv.upload(wq), dv.upload(wsc), m, n, k, split_k,
                      ws.buf if ws else None, ws.nbytes if ws else 0, c2)
    dv.collect(mbx2, p.out_bytes)
    torch.cuda.synchronize()
    assert np.array_equal(dv.as_u16(c2).reshape(m, n), raw)
    # Values against the float64 oracle on the oracle's codes.
    _, exact, abs_sum = gemm.gemm_publish_bits(p.w, p.ws, wq, wsc)
    assert tolerance.within(raw, exact, abs_sum)
    model = mailbox.MailboxModel(1, p.out_bytes)
    model.publish(0, raw)
    assert np.array_equal(got, model.collect(p.out_bytes).reshape(m, n))


def test_fused_quantizer_special_values(env):
    """Zeros of both signs, all-zero blocks, BF16 subnormals, values that
    round to zero, and a NaN block reach the GEMM's activation stage."""
    from oracle import quant
    from workloads import generate

    m, n, k = 4, 256, 512
    p = generate.random_problem(81, m, n, k, 1, "normal")
    xb = generate.bf16_activation(81, m, k, "normal")
    xb[0, 0:32] = 0
    xb[0, 32:64] = 0x8000
    xb[1, 0:32] = np.arange(1, 33, dtype=np.uint16)          # subnormals only
    xb[1, 64:96] = np.arange(1, 33, dtype=np.uint16) | 0x8000
    xb[1, 64] = 0x4000                                         # 2.0 beside subnormals
    xb[2, 128] = 0x7FC0                                        # NaN block
    xb[3, 300] = 0x7F7F                                        # the largest finite BF16
    q, s, *_ = _fused_case(env, p, xb, 1)
    wq, wsc = quant.quantize_bf16(xb)
    assert np.array_equal(s, wsc)
    assert np.array_equal(q, wq)


@pytest.mark.parametrize("split_k", [1, 4])
def test_unfused_publish_equals_fused(env, split_k):
    """mxgemm (C only) then mailbox_publish of C: the same mailbox bits and
    collect output as mxgemm_publish (publishing_gemm page, module docstring:
    the consumer sees the same bits either way)."""
    mx, dv = env
    from workloads import generate

    p = generate.config_problem(2) if split_k == 4 else generate.random_problem(5, 8, 2048, 1024)
    ops = dv.Operands(p)
    ws = dv.Workspace(p.n, split_k) if split_k > 1 else None
    wsb, wsn = (ws.buf, ws.nbytes) if ws else (None, 0)
    c_plain = torch.empty(p.m * p.n, dtype=torch.int16, device="cuda")
    mx.mxgemm(ops.w, ops.ws, ops.x, ops.xs, p.m, p.n, p.k, split_k, wsb, wsn, c_plain)
    a = dv.Mailbox(1, p.out_bytes)
    mx.mailbox_publish(a.mb, 0, c_plain, p.out_bytes)
    slots_unfused = None
    torch.cuda.synchronize()
    slots_unfused = a.slot_words()
    out_unfused = dv.as_u16(dv.collect(a, p.out_bytes))
    b = dv.Mailbox(1, p.out_bytes)
    c_fused = torch.empty(p.m * p.n, dtype=torch.int16, device="cuda")
    dv.publish(b, ops, split_k, ws, c_fused)
    torch.cuda.synchronize()
    assert np.array_equal(b.slot_words(), slots_unfused)
    assert np.array_equal(dv.as_u16(dv.collect(b, p.out_bytes)), out_unfused)
    assert torch.equal(c_plain, c_fused)
    if ws is not None:
        assert ws.header()[mx.WS_EPOCH] == 3 and ws.header()[mx.WS_ERROR] == 0


def test_fused_quantizer_graph_replays(env):
    """The BF16 path captured in a graph with its collect: every replay gives
    the eager output; the activation changes between replays (its buffer is
    rewritten eagerly) and the output follows it."""
    mx, dv = env
    from workloads import generate

    p = generate.random_problem(91, 8, 2048, 4096, 4, "outliers")
    ops = dv.Operands(p)
    ws = dv.Workspace(p.n, 4)
    mbx = dv.Mailbox(1, p.out_bytes)
    xa = dv.upload(generate.bf16_activation(1, 8, 4096))
    xb = dv.upload(generate.bf16_activation(2, 8, 4096))
    x = xa.clone()
    out = torch.empty(p.m * p.n, dtype=torch.int16, device="cuda")
    stream = torch.cuda.Stream()

    def call():
        mx.mxgemm_publish_bf16(mbx.mb, ops.w, ops.ws, x, 8, p.n, p.k, 4, ws.buf, ws.nbytes,
                               None, None, None, stream)
        mx.mailbox_collect(mbx.mb, out, p.out_bytes, stream)

    with torch.cuda.stream(stream):
        eager = {}
        for name, src in (("a", xa), ("b", xb)):
            x.copy_(src)
            call()
            stream.synchronize()
            eager[name] = out.clone()
        assert not torch.equal(eager["a"], eager["b"])
        mx.mxg_graph_begin(stream)
        call()
        g = mx.mxg_graph_end(stream)
        for rep in range(6):
            name = "ab"[rep % 2]
            x.copy_(xa if name == "a" else xb)
            out.zero_()
            mx.mxg_graph_launch(g, stream)
            stream.synchronize()
            assert torch.equal(out, eager[name]), f"replay {rep}"
        mx.mxg_graph_destroy(g)
    assert mbx.state_words()[mx.STATE_NEXT] == 8 % 3
