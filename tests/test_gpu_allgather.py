"""GPU parity of the fused all-gather (mailbox_all_gather) and the word
publish (mailbox_publish_words) against the CPU oracle's mailbox model
(oracle.mailbox.MailboxModel.publish_words / all_gather): output words and
mailbox bits exact, every slot back to the sentinel, the generation advanced.
The stress follows the all_gather page's module docstring (back-to-back
gathers of alternating sizes in graphs must never read a stale word)."""

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SENTINEL_I32 = -(2**31)


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


def _dev(words_u32: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(words_u32).view(np.int32).copy()).cuda()


def _host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32).copy()


# 16 B (one pack), one pack past a 256-thread block, the m=8 N=7168 GEMM
# output, and 4 MiB (more items than one launch has threads at 4 ranks).
SIZES = [16, 16 * 257, 2 * 8 * 7168, 4 << 20]


@pytest.mark.parametrize("nbytes", SIZES)
@pytest.mark.parametrize("ranks,rank", [(1, 0), (2, 0), (2, 1), (4, 2), (8, 7)])
def test_all_gather_matches_model(env, ranks, rank, nbytes):
    mx, dv = env
    from oracle import mailbox
    from workloads import generate

    words = nbytes // 4
    _say(f"case ranks={ranks} rank={rank} nbytes={nbytes}")
    pay = generate.word_payloads(1000 + 31 * ranks + rank + nbytes, ranks, words)
    mbx = dv.Mailbox(ranks, nbytes, rank=rank)
    for r in range(ranks):
        if r != rank:
            mx.mailbox_publish_words(mbx.mb, r, _dev(pay[r]), nbytes)
    got = _host(dv.all_gather(mbx, _dev(pay[rank]), nbytes)).reshape(ranks, words)
    torch.cuda.synchronize()
    model = mailbox.MailboxModel(ranks, nbytes)
    for r in range(ranks):
        if r != rank:
            model.publish_words(r, pay[r])
    want = model.all_gather(rank, pay[rank])
    assert np.array_equal(got, want)
    assert not np.any(got == 0x80000000)
    assert not mailbox.check_idle_slots(mbx.slot_words())
    st = mbx.state_words()
    assert st[mx.STATE_NEXT] == 1 and st[mx.STATE_ERROR] == 0


def test_publish_words_bits(env):
    """The word publish writes exactly the sanitized words into its slot of
    the current generation and nothing else."""
    mx, dv = env
    from oracle import mailbox
    from workloads import generate

    ranks, nbytes = 4, 16 * 300
    pay = generate.word_payloads(77, ranks, nbytes // 4)
    mbx = dv.Mailbox(ranks, 2 * nbytes)
    model = mailbox.MailboxModel(ranks, 2 * nbytes)
    for r in (3, 1):
        mx.mailbox_publish_words(mbx.mb, r, _dev(pay[r]), nbytes)
        model.publish_words(r, pay[r])
    torch.cuda.synchronize()
    assert np.array_equal(mbx.slot_words(), model.slots)


def test_all_gather_in_place(env):
    """src may be the caller's own row of the output."""
    mx, dv = env
    from oracle import mailbox
    from workloads import generate

    ranks, rank, nbytes = 4, 1, 16 * 1000
    words = nbytes // 4
    pay = generate.word_payloads(5, ranks, words)
    mbx = dv.Mailbox(ranks, nbytes, rank=rank)
    for r in range(ranks):
        if r != rank:
            mx.mailbox_publish_words(mbx.mb, r, _dev(pay[r]), nbytes)
    out = torch.full((ranks * words,), 7, dtype=torch.int32, device="cuda")
    out[rank * words:(rank + 1) * words] = _dev(pay[rank])
    dv.all_gather(mbx, out[rank * words:], nbytes, out=out)
    model = mailbox.MailboxModel(ranks, nbytes)
    for r in range(ranks):
        if r != rank:
            model.publish_words(r, pay[r])
    assert np.array_equal(_host(out).reshape(ranks, words), model.all_gather(rank, pay[rank]))


def test_all_gather_with_peers_on_another_stream(env):
    """Peers publish on a second stream while the gather polls: the gather
    waits for their words (both orders are valid; neither may read a stale
    word)."""
    mx, dv = env
    from oracle import mailbox
    from workloads import generate

    ranks, rank, nbytes = 4, 0, 2 * 8 * 7168
    words = nbytes // 4
    mbx = dv.Mailbox(ranks, nbytes, rank=rank)
    side = torch.cuda.Stream()
    main = torch.cuda.Stream()
    model = mailbox.MailboxModel(ranks, nbytes)
    for it in range(6):
        pay = generate.word_payloads(900 + it, ranks, words)
        src = [_dev(pay[r]) for r in range(ranks)]
        torch.cuda.synchronize()
        out = torch.empty(ranks * words, dtype=torch.int32, device="cuda")
        mx.mailbox_all_gather(mbx.mb, src[rank], out, nbytes, main)
        for r in range(1, ranks):
            mx.mailbox_publish_words(mbx.mb, r, src[r], nbytes, side)
        torch.cuda.synchronize()
        for r in range(1, ranks):
            model.publish_words(r, pay[r])
        assert np.array_equal(_host(out).reshape(ranks, words), model.all_gather(rank, pay[rank]))
    st = mbx.state_words()
    assert st[mx.STATE_NEXT] == 6 % 3 and st[mx.STATE_ERROR] == 0
    assert not mailbox.check_idle_slots(mbx.slot_words())


def test_all_gather_spin_limit_sets_error(env):
    """A peer that never publishes: with a tiny poll limit the gather gives
    up, flags the error and still resets the slots (forced from the host)."""
    mx, dv = env
    from oracle import mailbox

    mbx = dv.Mailbox(2, 256, rank=1)
    src = torch.ones(32, dtype=torch.int32, device="cuda")
    mbx.spin_limit = 8
    dv.all_gather(mbx, src, 128)
    torch.cuda.synchronize()
    assert mbx.state_words()[mx.STATE_ERROR] & mx.ERR_COLLECT_SPIN
    assert not mailbox.check_idle_slots(mbx.slot_words())


def _soak(env, sizes, ranks, rank, per_graph, replays):
    """Gathers cycling over `sizes` through one mailbox of the largest size:
    peers publish words, then the fused gather; each call's output compared
    on the device with the oracle's words for that size and sentinel words
    counted. The first round runs eagerly and is checked on the host."""
    mx, dv = env
    from oracle import mailbox
    from workloads import generate

    cap = max(sizes)
    mbx = dv.Mailbox(ranks, cap, rank=rank)
    model = mailbox.MailboxModel(ranks, cap)
    pays = [generate.word_payloads(4000 + i, ranks, s // 4) for i, s in enumerate(sizes)]
    srcs = [[_dev(p[r]) for r in range(ranks)] for p in pays]
    outs = [torch.empty(ranks * s // 4, dtype=torch.int32, device="cuda") for s in sizes]
    expect = []
    stream = torch.cuda.Stream()
    P = len(sizes)

    def call(i):
        for r in range(ranks):
            if r != rank:
                mx.mailbox_publish_words(mbx.mb, r, srcs[i][r], sizes[i], stream)
        mx.mailbox_all_gather(mbx.mb, srcs[i][rank], outs[i], sizes[i], stream)

    with torch.cuda.stream(stream):
        for i in range(P):
            call(i)
            stream.synchronize()
            for r in range(ranks):
                if r != rank:
                    model.publish_words(r, pays[i][r])
            want = model.all_gather(rank, pays[i][rank])
            assert np.array_equal(_host(outs[i]).reshape(ranks, -1), want), sizes[i]
            expect.append(_dev(want.reshape(-1)))
    mism = [torch.zeros_like(o) for o in outs]
    sent = [torch.zeros_like(o) for o in outs]
    m_ne = [torch.empty(o.shape, dtype=torch.bool, device="cuda") for o in outs]
    m_se = [torch.empty(o.shape, dtype=torch.bool, device="cuda") for o in outs]

    def call_and_check(i):
        call(i)
        torch.ne(outs[i], expect[i], out=m_ne[i])
        mism[i].add_(m_ne[i])
        torch.eq(outs[i], SENTINEL_I32, out=m_se[i])
        sent[i].add_(m_se[i])

    def counts():
        return (sum(int(t.sum()) for t in mism), sum(int(t.sum()) for t in sent))

    with torch.cuda.stream(stream):
        for i in range(P):
            call_and_check(i)
        stream.synchronize()
        mx.mxg_graph_begin(stream)
        for j in range(per_graph):
            call_and_check(j % P)
        g = mx.mxg_graph_end(stream)
        for rep in range(replays):
            mx.mxg_graph_launch(g, stream)
            if replays >= 100 and rep % (replays // 10) == replays // 10 - 1:
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
    return calls


def test_all_gather_graph_replays_match_eager(env):
    """Graph replays with eager gathers between them: a short soak of three
    sizes, replayed several times (every replay checked on the device)."""
    _soak(env, [16 * 257, 2 * 8 * 7168, 16], ranks=2, rank=1, per_graph=30, replays=5)


def test_all_gather_million_alternating_gathers(env):
    """10^6 back-to-back gathers alternating between two sizes (the m=8 and
    m=1 outputs of the N=7168 GEMM) in HIP graphs, four rank slots, the
    caller in slot 2: no mismatched and no sentinel word."""
    calls = _soak(env, [2 * 8 * 7168, 2 * 1 * 7168], ranks=4, rank=2, per_graph=1000,
                  replays=1000)
    _say(f"gathers: {calls}")
