"""GPU parity of the all-reduce collect (mailbox_collect_sum) against the CPU
oracle's all-reduce model (oracle.mailbox.allreduce_bf16): bit-exact, since
both add the ranks' BF16 values in FP32 in ascending rank order and round
once to BF16. Every case also checks the mailbox is back to the sentinel and
the generation advanced."""

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


@pytest.mark.parametrize("ranks", [1, 2, 4, 8])
@pytest.mark.parametrize("split_k", [1, 4])
def test_allreduce_after_gemm(env, ranks, split_k):
    mx, dv = env
    from oracle import codecs, gemm, mailbox, tolerance
    from workloads import generate

    p = generate.random_problem(300 + 10 * ranks + split_k, 8, 1000, 1024, split_k)
    _say(f"case m={p.m} n={p.n} k={p.k} split_k={split_k} ranks={ranks}")
    ops = dv.Operands(p)
    mbx = dv.Mailbox(ranks, p.out_bytes)
    ws = dv.Workspace(p.n, split_k) if split_k > 1 else None
    c_out = torch.empty(p.m * p.n, dtype=torch.int16, device="cuda")
    peers = generate.peer_payloads(p.seed, ranks, p.m, p.n)
    dv.publish(mbx, ops, split_k, ws, c_out)
    for r in range(1, ranks):
        mx.mailbox_publish(mbx.mb, r, dv.upload(peers[r - 1]), p.out_bytes)
    got = dv.as_u16(dv.collect_sum(mbx, p.out_bytes)).reshape(p.m, p.n)
    torch.cuda.synchronize()
    raw = dv.as_u16(c_out).reshape(p.m, p.n)
    _, exact, abs_sum = gemm.gemm_publish_bits(p.w, p.ws, p.x, p.xs)
    assert tolerance.within(raw, exact, abs_sum)
    model = mailbox.MailboxModel(ranks, p.out_bytes)
    model.publish(0, raw)
    for r in range(1, ranks):
        model.publish(r, peers[r - 1])
    want = model.collect_sum(p.out_bytes).reshape(p.m, p.n)
    assert np.array_equal(got, want)
    if ranks == 1:  # one rank: the published (negative-zero-cleared) output
        assert np.array_equal(got, codecs.clear_negative_zero(raw))
    assert not mailbox.check_idle_slots(mbx.slot_words())
    st = mbx.state_words()
    assert st[mx.STATE_NEXT] == 1 and st[mx.STATE_ERROR] == 0


def test_allreduce_cancellation_and_order(env):
    """Payloads built so that FP32 order and cancellation decide the bits:
    rank 1 = -rank 0 (sums to +0 with rank 2 = 0), and 2^24, 1, -2^24 over
    three ranks (the 1 is lost in FP32)."""
    mx, dv = env
    from oracle import codecs, mailbox

    n = 4096
    rng = np.random.default_rng(5)
    a = codecs.bf16_round_value(rng.standard_normal(n))
    pays = [a, -a, np.zeros(n)]
    big = np.zeros(n)
    big[:8] = [2.0**24, 1.0, -(2.0**24), 3.0, 2.0**-8, 1.0, 1.0, 2.0**24]
    pays2 = [big, np.roll(big, 1), np.roll(big, 2)]
    for ps in (pays, pays2):
        bits = [codecs.bf16_bits_from_value(v) for v in ps]
        mbx = dv.Mailbox(3, 2 * n)
        for r, b in enumerate(bits):
            mx.mailbox_publish(mbx.mb, r, dv.upload(b), 2 * n)
        got = dv.as_u16(dv.collect_sum(mbx, 2 * n))
        torch.cuda.synchronize()
        want = mailbox.allreduce_bf16(np.stack([codecs.clear_negative_zero(b) for b in bits]))
        assert np.array_equal(got, want)
        assert not mailbox.check_idle_slots(mbx.slot_words())


def test_allreduce_spin_limit_sets_error(env):
    """A rank that never publishes: with a tiny poll limit the all-reduce
    collect gives up, flags the error and still resets the slots (forced
    from the host; the kernel exits normally)."""
    mx, dv = env
    from oracle import mailbox

    mbx = dv.Mailbox(2, 256)
    mx.mailbox_publish(mbx.mb, 0, torch.ones(64, dtype=torch.int16, device="cuda"), 128)
    mbx.spin_limit = 8
    dv.collect_sum(mbx, 128)
    torch.cuda.synchronize()
    assert mbx.state_words()[mx.STATE_ERROR] & mx.ERR_COLLECT_SPIN
    assert not mailbox.check_idle_slots(mbx.slot_words())


def test_allreduce_alternating_sizes_in_graphs(env):
    """The stress workload's alternating sizes through one mailbox with the all-reduce
    collect, 1000 calls per graph replayed 20 times, every output compared
    on the device with the verified one of its size."""
    from test_gpu_parity import graph_soak
    from workloads import generate

    probs = [generate.config_problem(4, size=s) for s in (0, 1)]
    graph_soak(env, probs, 4, 4, 32768, per_graph=1000, replays=20, ws_n=7168, mode="sum")
