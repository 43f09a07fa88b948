"""mxgemm_publish_noalloc through the C ABI against mxgemm_publish (needs an
MI355X).

The no-allocation entry point runs the same kernels with the split-K pairs in
the library's own per-GPU array instead of a caller's workspace. On the same
inputs it must publish what mxgemm_publish publishes: the raw BF16 output and
every mailbox word bit for bit (the same kernel variant sums in the same
order), the values within the oracle's tolerance, and the state words as the
mailbox model says. Two calls in a row, the second on a smaller problem, so the
second reads the pairs and epoch words the first left in the array.
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


def _compare(env, p, split_k, calls=1):
    """`calls` publish+collect rounds of p through both entry points."""
    mx, dv = env
    from oracle import codecs, gemm, mailbox, tolerance

    _say(f"noalloc case m={p.m} n={p.n} k={p.k} split_k={split_k} seed={p.seed}")
    ops = dv.Operands(p)
    a = dv.Mailbox(1, p.out_bytes)
    b = dv.Mailbox(1, p.out_bytes)
    ws = dv.Workspace(p.n, split_k) if split_k > 1 else None
    ca = torch.empty(p.m * p.n, dtype=torch.int16, device="cuda")
    cb = torch.empty_like(ca)
    _, exact, abs_sum = gemm.gemm_publish_bits(p.w, p.ws, p.x, p.xs)
    for _ in range(calls):
        dv.publish(a, ops, split_k, ws, ca)
        mx.mxgemm_publish_noalloc(b.mb, ops.w, ops.ws, ops.x, ops.xs, p.m, p.n, p.k, split_k,
                                  cb)
        torch.cuda.synchronize()
        assert np.array_equal(a.slot_words(), b.slot_words())
        oa = dv.as_u16(dv.collect(a, p.out_bytes))
        ob = dv.as_u16(dv.collect(b, p.out_bytes))
        torch.cuda.synchronize()
        raw = dv.as_u16(cb).reshape(p.m, p.n)
        assert np.array_equal(dv.as_u16(ca), dv.as_u16(cb))
        assert tolerance.within(raw, exact, abs_sum)
        assert np.array_equal(oa, ob)
        assert np.array_equal(ob.reshape(p.m, p.n), codecs.clear_negative_zero(raw))
        assert not mailbox.check_collected(ob)
        assert not mailbox.check_idle_slots(b.slot_words())
    sa, sb = a.state_words(), b.state_words()
    assert sb[mx.STATE_NEXT] == calls % 3 and sb[mx.STATE_ERROR] == 0
    assert np.array_equal(sa, sb)


def test_noalloc_matches_publish_two_calls(env):
    """N=7168, K=8192, m=8, split-K 4, then a smaller one (N=1000,
    K=2048, m=3, split-K 8) that reuses the pair addresses of the first."""
    from workloads import generate

    _compare(env, generate.config_problem(2), 4, calls=2)
    _compare(env, generate.random_problem(8101, 3, 1000, 2048, 8), 8, calls=2)


def test_noalloc_without_split_and_limits(env):
    """Without split-K no array is used; a shape whose pairs exceed the array
    is refused before anything is enqueued, leaving the mailbox idle."""
    mx, dv = env
    from oracle import mailbox
    from workloads import generate

    _compare(env, generate.random_problem(8102, 5, 512, 1024, 1), 1)
    p = generate.random_problem(8103, 1, 16384, 1024, 8)
    ops = dv.Operands(p)
    mbx = dv.Mailbox(1, p.out_bytes)
    with pytest.raises(mx.MxgValueError) as e:
        mx.mxgemm_publish_noalloc(mbx.mb, ops.w, ops.ws, ops.x, ops.xs, p.m, p.n, p.k, 8)
    assert e.value.code == mx.EWORKSPACE
    torch.cuda.synchronize()
    assert not mailbox.check_idle_slots(mbx.slot_words())
