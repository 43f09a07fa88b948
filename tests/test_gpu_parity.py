"""GPU parity of the HIP path against the CPU oracle (needs an MI355X).

Every case runs mxgemm_publish (+ mailbox_publish for emulated peers) and
mailbox_collect through the C ABI and checks:
  * raw BF16 outputs within the oracle tolerance (tests/../oracle/tolerance);
  * the collected own slot bit-equal to the raw output with negative zero
    cleared, and bit-equal to the oracle's bits wherever the values agree;
  * peer slots bit-equal to the oracle mailbox model's output;
  * no sentinel word and no negative-zero half in the output, the whole
    mailbox back to the sentinel, and the state words as the model says.
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


def _oracle():
    from oracle import codecs, gemm, mailbox, tolerance

    return codecs, gemm, mailbox, tolerance


def run_case(env, p, split_k=1, ranks=1, capacity=None, peers=None, calls=1, with_c=True,
             ws=None):
    """Run `calls` publish+collect rounds of problem p; check everything."""
    mx, dv = env
    codecs, gemm, mailbox, tolerance = _oracle()
    cap = capacity or p.out_bytes
    _say(f"case {p.name} seed={p.seed} m={p.m} n={p.n} k={p.k} split_k={split_k} ranks={ranks}")
    ops = dv.Operands(p)
    mbx = dv.Mailbox(ranks, cap)
    if ws is None and split_k > 1:
        ws = dv.Workspace(p.n, split_k)
    epoch0 = ws.header()[mx.WS_EPOCH] if ws is not None else 0
    c_out = torch.empty(p.m * p.n, dtype=torch.int16, device="cuda") if with_c else None
    model = mailbox.MailboxModel(ranks, cap)
    bits, exact, abs_sum = gemm.gemm_publish_bits(p.w, p.ws, p.x, p.xs)
    peer_dev = [dv.upload(peers[r - 1]) for r in range(1, ranks)] if ranks > 1 else []
    outs = []
    for _ in range(calls):
        dv.publish(mbx, ops, split_k, ws, c_out)
        for r in range(1, ranks):
            mx.mailbox_publish(mbx.mb, r, peer_dev[r - 1], p.out_bytes)
        outs.append(dv.collect(mbx, p.out_bytes))
    torch.cuda.synchronize()
    got = [dv.as_u16(o).reshape(ranks * p.m, p.n) for o in outs]
    own = got[0][: p.m]
    # values
    if with_c:
        raw = dv.as_u16(c_out).reshape(p.m, p.n)
        ex = tolerance.excess(raw, exact, abs_sum)
        assert np.all(ex <= 1.0), f"max excess {ex.max()} at {np.unravel_index(ex.argmax(), ex.shape)}"
        assert np.array_equal(own, codecs.clear_negative_zero(raw))
    else:
        ex = tolerance.excess(own, exact, abs_sum)
        assert np.all(ex <= 1.0)
    same = codecs.bf16_to_f64(own) == codecs.bf16_to_f64(bits)
    assert np.array_equal(own[same], bits[same])
    # model: own slot from the device's values, peers from their payloads
    for _ in range(calls):
        model.publish(0, own)
        for r in range(1, ranks):
            model.publish(r, peers[r - 1])
        expect = model.collect(p.out_bytes).reshape(ranks * p.m, p.n)
    for g in got:
        assert np.array_equal(g, expect)
        assert not mailbox.check_collected(g)
    assert not mailbox.check_idle_slots(mbx.slot_words())
    st = mbx.state_words()
    assert st[mx.STATE_NEXT] == model.next == calls % 3
    assert st[mx.STATE_ERROR] == 0
    if ws is not None:
        hdr = ws.header()
        assert hdr[mx.WS_EPOCH] == epoch0 + calls and hdr[mx.WS_ERROR] == 0
    return own, bits, ex


def test_n256_k512_m1(env):
    from workloads import generate

    run_case(env, generate.config_problem(0), calls=4)


@pytest.mark.parametrize("split_k", [1, 2, 4, 8])
def test_small_all_splits(env, split_k):
    from workloads import generate

    p = generate.random_problem(31 + split_k, 8, 320, 2048, split_k)
    run_case(env, p, split_k=split_k, calls=2)


@pytest.mark.parametrize("m", [1, 2, 3, 5, 7, 8])
def test_rows_and_ragged_n(env, m):
    from workloads import generate

    for n, k, s in [(8, 128, 1), (24, 384, 1), (40, 512, 2), (1000, 1024, 4), (136, 1024, 8)]:
        p = generate.random_problem(1000 * m + n, m, n, k, s)
        run_case(env, p, split_k=s)


# Every kernel variant of the library (rows-per-wave blocks, waves along
# rows, waves along K, load depth), forced through mxgemm_tile (binding.TILE). The
# fifth field is the first staging round's size, the sixth whether x is also
# kept as BF16 in LDS (without it: BF16 when it fits, the default).
TILES = ["1,1,4,4", "1,1,8,4", "1,1,16,4", "1,4,1,8", "1,4,1,3", "1,7,1,8", "1,7,1,4",
         "1,7,1,3", "1,7,1,5", "1,2,2,8", "1,2,2,5", "1,4,2,8", "2,1,4,4", "1,8,1,8", "2,2,2,4",
         "1,4,1,3,2", "1,1,16,4,2",  # one staging round of twice the size
         # x left in FP8 in LDS, converted by every wave
         "1,1,4,4,1,0", "1,1,16,4,1,0", "1,4,1,3,1,0", "1,7,1,3,1,0", "1,2,2,8,1,0",
         "1,4,1,3,2,0",
         # x staged as BF16 forced (refused where it does not fit), also at
         # splits the chooser keeps in FP8
         "1,7,1,3,1,1", "1,4,1,3,1,1", "1,7,1,5,1,0", "1,2,2,5,1,0"]


@pytest.mark.parametrize("tile", TILES)
def test_every_tile_variant(env, tile, monkeypatch):
    """Each variant on a ragged N at every split it is built for, with 1, 5
    and 8 tokens and K slices down to one 128-wide block (waves along K left
    without work), and m = 8 at K = 8192, whose activation slice takes several
    staging rounds; then with scale bytes at both E8M0 ends, which every
    workgroup meets and so takes the exact path (x staged as FP8 again where
    the variant staged it as BF16). The 16-wave variant has no split-K form
    (its control wave would pass 1024 threads)."""
    mx, _ = env
    from workloads import generate

    monkeypatch.setattr(mx, "TILE", tile)
    ran = 0
    for m, k, extreme in [(1, 2048, False), (5, 1024, False), (8, 2048, False),
                          (8, 8192, False), (3, 2048, True), (8, 8192, True)]:
        for s in [1, 2, 4, 8]:
            p = generate.random_problem(7000 + 10 * m + s + k, m, 1000, k, s)
            if extreme:  # scale bytes at both E8M0 ends: the exact path
                p = generate.extreme_scales(p, 7001 + m + s)
            try:
                run_case(env, p, split_k=s, calls=2)
                ran += 1
            except mx.MxgUnsupported:
                _say(f"tile {tile} unsupported at m={m} k={k} split_k={s}")
    assert ran >= (6 if tile.startswith("1,1,16,4") else 12)


@pytest.mark.parametrize("x16,split", [("auto", 1), ("0", 1), ("auto", 4), ("0", 4)])
def test_single_nonzero_sweep(env, x16, split, monkeypatch):
    """One nonzero W element and one nonzero x element at swept positions: the
    result is one exact product, so any slip of the MFMA lane, K-piece or
    scale mapping shows up bit for bit. With x kept as BF16 in LDS (the
    default where it fits) and in FP8 (tile spec "fp8"), with and without split-K."""
    mx, dv = env
    if x16 == "0":
        monkeypatch.setattr(mx, "TILE", "fp8")
    codecs, gemm, _, _ = _oracle()
    from workloads.generate import Problem

    n, k, m = 64, 512, 8
    rng = np.random.default_rng(7)
    positions = [(r, kk, t) for r in (0, 5, 17, 34, 63) for kk in (0, 15, 16, 31, 32, 63, 64, 100,
                                                                   127, 128, 200, 511)
                 for t in (0, 3, 7)]
    mbx = dv.Mailbox(1, 2 * m * n)
    wsp = dv.Workspace(n, split) if split > 1 else None
    c_out = torch.empty(m * n, dtype=torch.int16, device="cuda")
    for (r, kk, t) in positions:
        w = np.zeros((n, k), np.uint8)
        x = np.zeros((m, k), np.uint8)
        ws = np.full((n, k // 32), 127, np.uint8)
        xs = np.full((m, k // 32), 127, np.uint8)
        w[r, kk] = rng.choice([0x38, 0xB9, 0x44, 0x51])
        x[t, kk] = rng.choice([0x38, 0x3C, 0xC2])
        ws[r, kk // 32] = rng.integers(118, 136)
        xs[t, kk // 32] = rng.integers(118, 136)
        # background scales of other blocks must not leak in
        ws[r, (kk // 32 + 1) % (k // 32)] = 140
        xs[t, (kk // 32 + 2) % (k // 32)] = 100
        p = Problem("single", m, n, k, split, w, ws, x, xs, 0)
        dv.publish(mbx, dv.Operands(p), split, wsp, c_out)
        out = dv.collect(mbx, p.out_bytes)
        torch.cuda.synchronize()
        got = dv.as_u16(out).reshape(m, n)
        bits, _, _ = gemm.gemm_publish_bits(w, ws, x, xs)
        assert np.array_equal(got, bits), f"position {(r, kk, t)}"


def test_closed_forms(env):
    """Identity-like W returns x; all-ones x returns W's row sums."""
    mx, dv = env
    codecs, gemm, _, tolerance = _oracle()
    from workloads import generate
    from workloads.generate import Problem

    base = generate.random_problem(8, 4, 256, 256)
    w = np.zeros((256, 256), np.uint8)
    w[np.arange(256), np.arange(256)] = 0x38
    ws = np.full((256, 8), 127, np.uint8)
    p = Problem("identity", 4, 256, 256, 1, w, ws, base.x, base.xs, 0)
    own, bits, _ = run_case(env, p)
    xd = codecs.decode_e4m3(base.x) * np.repeat(codecs.decode_e8m0(base.xs), 32, axis=1)
    assert np.array_equal(codecs.bf16_to_f64(own), codecs.bf16_to_f64(codecs.bf16_rne_bits(xd)))
    x1 = np.full((1, 256), 0x38, np.uint8)
    xs1 = np.full((1, 8), 127, np.uint8)
    p2 = Problem("ones", 1, 256, 256, 1, base.w, base.ws, x1, xs1, 0)
    run_case(env, p2)


@pytest.mark.parametrize("split_k", [1, 4])
def test_negative_zero_and_zero_rows(env, split_k):
    """The stress recipe: zero rows (of +0 and -0 codes) publish 0x0000, and
    the tiny rows' results, single products below 2^-135 in magnitude, reach
    the epilogue as BF16 zeros of the product's sign: 0x8000 in the raw output
    wherever the product is negative, 0x0000 in the mailbox everywhere."""
    mx, dv = env
    codecs, gemm, _, _ = _oracle()
    from workloads import generate

    p = generate.random_problem(77, 8, 512, 1024, split_k, "stress")
    own, bits, _ = run_case(env, p, split_k=split_k)
    zr = np.r_[p.meta["zero_rows_pos"], p.meta["zero_rows_neg"], p.meta["tiny_rows"]]
    assert np.all(own[:, zr] == 0)
    ops = dv.Operands(p)
    mbx = dv.Mailbox(1, p.out_bytes)
    ws = dv.Workspace(p.n, split_k) if split_k > 1 else None
    c = torch.empty(p.m * p.n, dtype=torch.int16, device="cuda")
    dv.publish(mbx, ops, split_k, ws, c)
    got = dv.as_u16(dv.collect(mbx, p.out_bytes)).reshape(p.m, p.n)
    torch.cuda.synchronize()
    raw = dv.as_u16(c).reshape(p.m, p.n)
    exact, _ = gemm.gemm_f64(p.w, p.ws, p.x, p.xs)
    tiny = p.meta["tiny_rows"]
    neg = exact[:, tiny] < 0
    assert neg.any() and (exact[:, tiny] > 0).any()
    assert np.all(raw[:, tiny][neg] == 0x8000)
    assert np.all(raw[:, tiny][~neg] == 0x0000)
    assert np.all(got[:, tiny] == 0) and np.all(got == codecs.clear_negative_zero(raw))


def test_fused_equals_unfused(env):
    """The fused epilogue publishes the same bits as the raw output pushed
    through the unfused publish (the consumer cannot tell them apart)."""
    mx, dv = env
    from workloads import generate

    p = generate.random_problem(91, 8, 1024, 2048, 4, "stress")
    ops = dv.Operands(p)
    ws = dv.Workspace(p.n, 4)
    a = dv.Mailbox(1, p.out_bytes)
    b = dv.Mailbox(1, p.out_bytes)
    c_out = torch.empty(p.m * p.n, dtype=torch.int16, device="cuda")
    dv.publish(a, ops, 4, ws, c_out)
    mx.mailbox_publish(b.mb, 0, c_out, p.out_bytes)
    sa = a.slot_words()
    sb = b.slot_words()
    assert np.array_equal(sa, sb)
    oa = dv.collect(a, p.out_bytes)
    ob = dv.collect(b, p.out_bytes)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob)


def test_n7168_k2048_m4(env):
    from workloads import generate

    run_case(env, generate.config_problem(1))


@pytest.mark.parametrize("dist", ["outliers", "normal"])
def test_n7168_k8192_m8_s4(env, dist):
    from workloads import generate

    p = generate.config_problem(2, dist=dist)
    run_case(env, p, split_k=4, capacity=114688, calls=3)


@pytest.mark.parametrize("m", [1, 2, 4, 8])
@pytest.mark.parametrize("split_k", [1, 4, 8])
def test_n4096_k16384_sweep(env, m, split_k):
    from workloads import generate

    p = generate.config_problem(3, m=m, split_k=split_k)
    peers = generate.peer_payloads(p.seed, 4, m, p.n)
    run_case(env, p, split_k=split_k, ranks=4, capacity=65536, peers=peers, calls=4)


def test_stress_alternating(env):
    """Alternating sizes through one mailbox and one workspace: every output
    bit-identical to the first verified output of its size, nothing stale."""
    mx, dv = env
    codecs, gemm, mailbox, tolerance = _oracle()
    from workloads import generate

    probs = [generate.config_problem(4, size=s) for s in (0, 1)]
    ops = [dv.Operands(p) for p in probs]
    peers = [generate.peer_payloads(p.seed, 4, p.m, p.n) for p in probs]
    peer_dev = [[dv.upload(pp[r]) for r in range(3)] for pp in peers]
    mbx = dv.Mailbox(4, 32768)
    ws = dv.Workspace(7168, 4)
    c_out = [torch.empty(p.m * p.n, dtype=torch.int16, device="cuda") for p in probs]
    model = mailbox.MailboxModel(4, 32768)
    expect = [None, None]
    calls = 60
    for i in range(calls):
        s = i % 2
        p = probs[s]
        dv.publish(mbx, ops[s], 4, ws, c_out[s])
        for r in range(1, 4):
            mx.mailbox_publish(mbx.mb, r, peer_dev[s][r - 1], p.out_bytes)
        out = dv.as_u16(dv.collect(mbx, p.out_bytes)).reshape(4 * p.m, p.n)
        if expect[s] is None:
            raw = dv.as_u16(c_out[s]).reshape(p.m, p.n)
            _, exact, abs_sum = gemm.gemm_publish_bits(p.w, p.ws, p.x, p.xs)
            assert tolerance.within(raw, exact, abs_sum)
            model.publish(0, raw)
            for r in range(1, 4):
                model.publish(r, peers[s][r - 1])
            expect[s] = model.collect(p.out_bytes).reshape(4 * p.m, p.n)
        assert np.array_equal(out, expect[s]), f"call {i}"
        assert not mailbox.check_collected(out)
        assert not mailbox.check_idle_slots(mbx.slot_words())
    st = mbx.state_words()
    assert st[mx.STATE_NEXT] == calls % 3 and st[mx.STATE_ERROR] == 0
    assert ws.header()[mx.WS_EPOCH] == 1 + calls


def test_graph_replays_match_eager(env):
    mx, dv = env
    from workloads import generate

    p = generate.random_problem(55, 8, 2048, 4096, 4)
    ops = dv.Operands(p)
    mbx = dv.Mailbox(1, p.out_bytes)
    ws = dv.Workspace(p.n, 4)
    c_out = torch.empty(p.m * p.n, dtype=torch.int16, device="cuda")
    out = torch.empty(p.m * p.n, dtype=torch.int16, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        dv.publish(mbx, ops, 4, ws, c_out)
        dv.collect(mbx, p.out_bytes, out)
        stream.synchronize()
        eager = out.clone()
        mx.mxg_graph_begin(stream)
        for _ in range(3):
            dv.publish(mbx, ops, 4, ws, c_out)
            dv.collect(mbx, p.out_bytes, out)
        g = mx.mxg_graph_end(stream)
        for rep in range(4):
            out.zero_()
            mx.mxg_graph_launch(g, stream)
            stream.synchronize()
            assert torch.equal(out, eager), f"replay {rep}"
            # eager work between replays
            dv.publish(mbx, ops, 4, ws, c_out)
            dv.collect(mbx, p.out_bytes, out)
            stream.synchronize()
            assert torch.equal(out, eager)
        mx.mxg_graph_destroy(g)
    calls = 1 + 4 * 3 + 4
    st = mbx.state_words()
    assert st[mx.STATE_NEXT] == calls % 3
    assert ws.header()[mx.WS_EPOCH] == 1 + calls


def test_collect_spin_limit_sets_error(env):
    """A rank that never publishes: with a tiny poll limit the collect gives
    up, flags the error and still resets the slots (forced from the host; the
    kernel exits normally)."""
    mx, dv = env
    from oracle import mailbox

    mbx = dv.Mailbox(2, 256)
    src = torch.ones(64, dtype=torch.int16, device="cuda")
    mx.mailbox_publish(mbx.mb, 0, src, 128)
    mbx.spin_limit = 8
    dv.collect(mbx, 128)
    torch.cuda.synchronize()
    st = mbx.state_words()
    assert st[mx.STATE_ERROR] & mx.ERR_COLLECT_SPIN
    assert not mailbox.check_idle_slots(mbx.slot_words())
    mbx.reinit()
    torch.cuda.synchronize()
    assert mbx.state_words()[mx.STATE_ERROR] == 0


def test_stray_word_is_reported_by_the_idle_scan(env):
    """A non-sentinel word written from the host into the next generation's
    slot, past the bytes the next call publishes and collects, is what a
    missed reset would leave (all_gather page, module docstring, step 2: no
    call leaves a word for a later one). The collect of that smaller call
    neither reads nor resets it, and the post-collect scan of the whole
    mailbox reports it; the call's own output stays exact. Arming again
    clears it."""
    mx, dv = env
    _, gemm, mailbox, tolerance = _oracle()
    from workloads import generate

    p = generate.random_problem(4343, 2, 64, 256)  # 256 bytes of output
    ops = dv.Operands(p)
    mbx = dv.Mailbox(1, 1024)
    assert not mailbox.check_idle_slots(mbx.slot_words())
    # generation 0, the one the next publish uses; word 128 lies past 256 bytes
    mbx.slots[128] = 0x12345678
    c = torch.empty(p.m * p.n, dtype=torch.int16, device="cuda")
    dv.publish(mbx, ops, 1, None, c)
    out = dv.as_u16(dv.collect(mbx, p.out_bytes)).reshape(p.m, p.n)
    torch.cuda.synchronize()
    _, exact, abs_sum = gemm.gemm_publish_bits(p.w, p.ws, p.x, p.xs)
    assert tolerance.within(out, exact, abs_sum)
    assert not mailbox.check_collected(out)
    words = mbx.slot_words()
    assert mailbox.check_idle_slots(words)
    assert words[0, 0, 128] == 0x12345678 and np.count_nonzero(words != 0x80000000) == 1
    mbx.reinit()
    torch.cuda.synchronize()
    assert not mailbox.check_idle_slots(mbx.slot_words())


def test_stale_epoch_is_not_taken(env):
    """Pairs left by an earlier call never carry the live tag: after a call of
    one size, a call of another size that reuses the same pair addresses still
    matches the oracle."""
    from workloads import generate

    mx, dv = env
    a = generate.random_problem(61, 8, 1024, 4096, 8)
    b = generate.random_problem(62, 2, 1024, 1024, 8)
    c = generate.random_problem(63, 8, 512, 2048, 4)
    ws = dv.Workspace(1024, 8)
    run_case(env, a, split_k=8, ws=ws, calls=2)
    run_case(env, b, split_k=8, ws=ws, calls=2)
    run_case(env, c, split_k=4, ws=ws, calls=2)
    run_case(env, a, split_k=8, ws=ws)
    assert ws.header()[mx.WS_EPOCH] == 1 + 7


@pytest.mark.parametrize("n,k", [(16, 128), (24, 384), (136, 1024), (1000, 512)])
def test_pack_weight_layout(env, n, k):
    """mxgemm_pack_weight moves bytes only: compare with the layout written
    out element by element (byte work is bit-exact)."""
    mx, dv = env
    rng = np.random.default_rng(n + k)
    w = rng.integers(0, 256, size=(n, k), dtype=np.uint8)
    ws = rng.integers(0, 256, size=(n, k // 32), dtype=np.uint8)
    # 32-wide blocks of zero codes (+0 and -0) under extreme scale bytes: the
    # range words leave them out
    for j in range(0, n * (k // 32), 5):
        r, b = divmod(j, k // 32)
        w[r, 32 * b:32 * b + 32] = 0x80 if j % 2 else 0x00
        ws[r, b] = 0 if j % 3 else 255
    wp, wsp = dv.pack_weight(dv.upload(w), dv.upload(ws), n, k)
    torch.cuda.synchronize()
    wp = wp.cpu().numpy()
    wsp = wsp.cpu().numpy()
    rbn, kbt = -(-n // 16), k // 128
    assert wp.size == rbn * kbt * 2048
    assert wsp.size == rbn * kbt * 64 + -(-rbn * 4 // 16) * 16
    expect = np.zeros(rbn * kbt * 2048, np.uint8)
    sexp = np.full(rbn * kbt * 64, 127, np.uint8)
    for rb in range(rbn):
        for kb in range(kbt):
            t = rb * kbt + kb
            for h in range(2):
                for l in range(64):
                    row = rb * 16 + l % 16
                    if row < n:
                        col = kb * 128 + 64 * h + 16 * (l // 16)
                        o = t * 2048 + h * 1024 + 16 * l
                        expect[o:o + 16] = w[row, col:col + 16]
            for r in range(16):
                row = rb * 16 + r
                if row < n:
                    sexp[(t * 16 + r) * 4:(t * 16 + r) * 4 + 4] = ws[row, kb * 4:kb * 4 + 4]
    assert np.array_equal(wp, expect)
    assert np.array_equal(wsp[: sexp.size], sexp)
    # one range word per row block: smallest and largest scale byte over its
    # (row, 32-wide block) pairs holding a nonzero code (0xFF and 0 if none)
    words = wsp[sexp.size: sexp.size + 4 * rbn].view(np.uint32)
    nz = np.any((w & 0x7F).reshape(n, k // 32, 32) != 0, axis=2)
    for rb in range(rbn):
        sel = ws[rb * 16:rb * 16 + 16][nz[rb * 16:rb * 16 + 16]]
        lo, hi = (int(sel.min()), int(sel.max())) if sel.size else (0xFF, 0)
        assert words[rb] == lo | (hi << 8), rb


def graph_soak(env, probs, split_k, ranks, capacity, per_graph, replays, ws_n=None,
               mode="gather"):
    """Calls cycling over `probs` (GEMM+publish into slot 0, emulated peers in
    slots 1.., collect) through one mailbox and one workspace. The first call
    of each problem is verified eagerly (values against the oracle, mailbox
    bits against the oracle model); then `per_graph` calls are captured in one
    HIP graph and replayed `replays` times, every call's collected words
    compared on the device with the verified output of its problem and
    sentinel words counted. mode "gather" collects rank-major
    (mailbox_collect), "sum" all-reduces the slots (mailbox_collect_sum).
    Only elementwise torch ops with preallocated outputs run inside the graph
    (no allocation, no memset)."""
    mx, dv = env
    codecs, gemm, mailbox, tolerance = _oracle()
    from workloads import generate

    ops = [dv.Operands(p) for p in probs]
    peers = [generate.peer_payloads(p.seed, ranks, p.m, p.n) for p in probs]
    peer_dev = [[dv.upload(pp[r]) for r in range(ranks - 1)] for pp in peers]
    mbx = dv.Mailbox(ranks, capacity)
    ws = dv.Workspace(ws_n or max(p.n for p in probs), split_k) if split_k > 1 else None
    epoch0 = ws.header()[mx.WS_EPOCH] if ws is not None else 0
    c_out = [torch.empty(p.m * p.n, dtype=torch.int16, device="cuda") for p in probs]
    rows = ranks if mode == "gather" else 1
    outs = [torch.empty(rows * p.m * p.n, dtype=torch.int16, device="cuda") for p in probs]
    model = mailbox.MailboxModel(ranks, capacity)
    stream = torch.cuda.Stream()
    P = len(probs)

    def call(s):
        p = probs[s]
        dv.publish(mbx, ops[s], split_k, ws, c_out[s], stream=stream)
        for r in range(1, ranks):
            mx.mailbox_publish(mbx.mb, r, peer_dev[s][r - 1], p.out_bytes, stream)
        if mode == "gather":
            mx.mailbox_collect(mbx.mb, outs[s], p.out_bytes, stream)
        else:
            mx.mailbox_collect_sum(mbx.mb, outs[s], p.out_bytes, stream)

    expect = []
    with torch.cuda.stream(stream):
        for s, p in enumerate(probs):
            call(s)
            stream.synchronize()
            raw = dv.as_u16(c_out[s]).reshape(p.m, p.n)
            _, exact, abs_sum = gemm.gemm_publish_bits(p.w, p.ws, p.x, p.xs)
            assert tolerance.within(raw, exact, abs_sum), p.name
            model.publish(0, raw)
            for r in range(1, ranks):
                model.publish(r, peers[s][r - 1])
            if mode == "gather":
                want = model.collect(p.out_bytes).reshape(rows * p.m, p.n)
            else:
                want = model.collect_sum(p.out_bytes).reshape(p.m, p.n)
            assert np.array_equal(dv.as_u16(outs[s]).reshape(rows * p.m, p.n), want), p.name
            expect.append(torch.from_numpy(want.reshape(-1).view(np.int16).copy()).cuda())

    words = [o.numel() // 2 for o in outs]
    out32 = [o.view(torch.int32) for o in outs]
    exp32 = [e.view(torch.int32) for e in expect]
    mism = [torch.zeros(w, dtype=torch.int32, device="cuda") for w in words]
    sent = [torch.zeros(w, dtype=torch.int32, device="cuda") for w in words]
    m_ne = [torch.empty(w, dtype=torch.bool, device="cuda") for w in words]
    m_se = [torch.empty(w, dtype=torch.bool, device="cuda") for w in words]
    sentinel = -(2**31)  # 0x80000000 as int32

    def call_and_check(s):
        call(s)
        torch.ne(out32[s], exp32[s], out=m_ne[s])
        mism[s].add_(m_ne[s])
        torch.eq(out32[s], sentinel, out=m_se[s])
        sent[s].add_(m_se[s])

    def counts():
        return (sum(int(t.sum()) for t in mism), sum(int(t.sum()) for t in sent))

    with torch.cuda.stream(stream):
        for s in range(P):  # the checks once eagerly (warms every kernel)
            call_and_check(s)
        stream.synchronize()
        mx.mxg_graph_begin(stream)
        for i in range(per_graph):
            call_and_check(i % P)
        g = mx.mxg_graph_end(stream)
        for rep in range(replays):
            mx.mxg_graph_launch(g, stream)
            if replays >= 100 and rep % 100 == 99:
                stream.synchronize()
                _say(f"replays {rep + 1}/{replays}: mismatched words {counts()[0]}, "
                     f"sentinel words {counts()[1]}")
        stream.synchronize()
        mx.mxg_graph_destroy(g)
    calls = 2 * P + per_graph * replays
    assert counts() == (0, 0)
    assert not mailbox.check_idle_slots(mbx.slot_words())
    st = mbx.state_words()
    assert st[mx.STATE_NEXT] == calls % 3 and st[mx.STATE_ERROR] == 0
    if ws is not None:
        hdr = ws.header()
        assert hdr[mx.WS_EPOCH] == epoch0 + calls and hdr[mx.WS_ERROR] == 0
    return calls


@pytest.mark.parametrize("m", [1, 2, 4, 8])
@pytest.mark.parametrize("split_k", [1, 4, 8])
def test_n4096_k16384_graph_1000_calls(env, m, split_k):
    """N=4096, K=16384 at every m and split: 1000 back-to-back calls in one HIP graph, four
    emulated rank slots, the three generations cycling."""
    from workloads import generate

    p = generate.config_problem(3, m=m, split_k=split_k)
    graph_soak(env, [p], split_k, 4, 65536, per_graph=1000, replays=1)


@pytest.mark.parametrize("dist", ["outliers", "normal"])
def test_n7168_k8192_m8_s4_graph_100_calls(env, dist):
    """N=7168, K=8192, m=8, split-K 4: the epoch advances once per call over 100
    graph-captured calls, every output identical to the verified one."""
    from workloads import generate

    p = generate.config_problem(2, dist=dist)
    graph_soak(env, [p], 4, 1, 114688, per_graph=100, replays=1)


def test_stress_million_alternating_calls(env):
    """The stress workload at full count: 10^6 calls alternating N=7168/K=4096/m=1
    and N=2048/K=8192/m=8 at split-K 4 (GEMM+publish into
    slot 0, three emulated peers, collect) through one mailbox and one
    workspace, in HIP graphs of 1000 calls replayed 1000 times: zero
    mismatched and zero sentinel words, the mailbox idle and the state words
    exact at the end."""
    from workloads import generate

    probs = [generate.config_problem(4, size=s) for s in (0, 1)]
    graph_soak(env, probs, 4, 4, 32768, per_graph=1000, replays=1000, ws_n=7168)


def test_publish_timed_matches_publish(env):
    """mxgemm_publish_timed: the same output and mailbox effects as
    mxgemm_publish, and its two events bracket the kernel (a positive duration
    shorter than the host's wall time around the call)."""
    import time

    mx, dv = env
    from workloads import generate

    p = generate.random_problem(4242, 8, 2048, 4096, 4)
    ops = dv.Operands(p)
    ws = dv.Workspace(p.n, 4)
    a, b = dv.Mailbox(1, p.out_bytes), dv.Mailbox(1, p.out_bytes)
    ca = torch.empty(p.m * p.n, dtype=torch.int16, device="cuda")
    cb = torch.empty_like(ca)
    dv.publish(a, ops, 4, ws, ca)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()  # materialize the handles
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    mx.mxgemm_publish_timed(b.mb, ops.w, ops.ws, ops.x, ops.xs, p.m, p.n, p.k, 4, ws.buf,
                            ws.nbytes, cb, None, e0, e1)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    assert torch.equal(ca, cb)
    assert np.array_equal(a.slot_words(), b.slot_words())
    ms = e0.elapsed_time(e1)
    assert 0.0 < ms < wall_ms
    assert b.state_words()[mx.STATE_ACTIVE] == 0 and ws.header()[mx.WS_EPOCH] == 3
    with pytest.raises(mx.MxgValueError):
        mx.mxgemm_publish_timed(b.mb, ops.w, ops.ws, ops.x, ops.xs, p.m, p.n, p.k, 4, ws.buf,
                                ws.nbytes, cb, None, None, e1)


def test_large_n_split_grid_rejected_and_plain_runs(env):
    """Maximum sizes: a split-K grid that cannot be resident all at once (its
    workgroups wait for each other) is refused before anything is enqueued,
    leaving the mailbox untouched; the same shape without split-K runs and
    matches the oracle."""
    mx, dv = env
    codecs, gemm, mailbox, tolerance = _oracle()
    from workloads import generate

    p = generate.random_problem(6553, 2, 65536, 1024, 8)
    _say(f"case m={p.m} n={p.n} k={p.k} split_k=8 (expect refusal), then split_k=1")
    ops = dv.Operands(p)
    mbx = dv.Mailbox(1, p.out_bytes)
    ws = dv.Workspace(p.n, 8)
    torch.cuda.synchronize()
    with pytest.raises(mx.MxgUnsupported):
        dv.publish(mbx, ops, 8, ws)
    torch.cuda.synchronize()
    assert not mailbox.check_idle_slots(mbx.slot_words())
    assert ws.header()[mx.WS_EPOCH] == 1
    c = torch.empty(p.m * p.n, dtype=torch.int16, device="cuda")
    dv.publish(mbx, ops, 1, None, c)
    got = dv.as_u16(dv.collect(mbx, p.out_bytes)).reshape(p.m, p.n)
    torch.cuda.synchronize()
    raw = dv.as_u16(c).reshape(p.m, p.n)
    _, exact, abs_sum = gemm.gemm_publish_bits(p.w, p.ws, p.x, p.xs)
    assert tolerance.within(raw, exact, abs_sum)
    assert np.array_equal(got, codecs.clear_negative_zero(raw))
    assert not mailbox.check_idle_slots(mbx.slot_words())
