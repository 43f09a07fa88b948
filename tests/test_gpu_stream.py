"""The read-stream measurement aid (mxg_stream_read): its per-chunk checksums
equal the XOR of each 32 KiB chunk's 32-bit words, computed on the host, for
whole and ragged sizes (so every byte was read, and nothing past the end)."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("nbytes", [16, 32768, 3 * 32768, 1 << 20, (1 << 20) + 48, 58720256])
def test_stream_read_checksums(nbytes):
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    from mxfp8_decode_gemm_amd import binding as mx

    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    chunks = -(-nbytes // mx.STREAM_CHUNK_BYTES)
    sink = torch.full((chunks + 1,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    mx.mxg_stream_read(src, nbytes, sink)
    got = sink.cpu().numpy().view(np.uint32)
    per = mx.STREAM_CHUNK_BYTES // 4
    want = np.array([np.bitwise_xor.reduce(host[i * per:(i + 1) * per]) for i in range(chunks)],
                    dtype=np.uint32)
    assert np.array_equal(got[:chunks], want)
    assert got[chunks] == 0x5A5A5A5A  # one word per chunk, no more


def _expected_cfg(host, nwords16, workgroups, interleave, chunk16):
    """Per-workgroup XOR of the 32-bit words each workgroup reads."""
    if workgroups == 0:
        groups = [(c * chunk16, min((c + 1) * chunk16, nwords16))
                  for c in range(-(-nwords16 // chunk16))]
        return [np.bitwise_xor.reduce(host[4 * lo:4 * hi]) if hi > lo else 0 for lo, hi in groups]
    if not interleave:
        per = -(-nwords16 // workgroups)
        out = []
        for g in range(workgroups):
            lo, hi = g * per, min((g + 1) * per, nwords16)
            out.append(np.bitwise_xor.reduce(host[4 * lo:4 * hi]) if hi > lo else 0)
        return out
    chunks = -(-nwords16 // chunk16)
    out = []
    for g in range(workgroups):
        x = np.uint32(0)
        for c in range(g, chunks, workgroups):
            lo, hi = c * chunk16, min((c + 1) * chunk16, nwords16)
            x ^= np.bitwise_xor.reduce(host[4 * lo:4 * hi])
        out.append(x)
    return out


@pytest.mark.parametrize("nbytes", [48, 3 * 32768 + 16, (1 << 20) + 48])
@pytest.mark.parametrize("workgroups,interleave", [(0, 0), (7, 0), (256, 0), (5, 1), (64, 1)])
def test_stream_read_cfg_checksums(nbytes, workgroups, interleave):
    """mxg_stream_read_cfg: every thread count, unroll and load kind, each way
    of splitting the bytes: each workgroup's checksum equals the host's XOR
    of its range (every byte read once, nothing past the end), and no word
    past the grid's is written."""
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    from mxfp8_decode_gemm_amd import binding as mx

    rng = np.random.default_rng(nbytes + workgroups)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    chunk16 = mx.STREAM_CHUNK_BYTES // 16
    want = np.array(_expected_cfg(host, nbytes // 16, workgroups, interleave, chunk16), np.uint32)
    for threads in (256, 512):
        for unroll in (4, 8, 16):
            for kind in range(5):
                sink = torch.full((want.size + 1,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
                mx.mxg_stream_read_cfg(src, nbytes, sink, workgroups, threads, unroll, kind,
                                       bool(interleave))
                got = sink.cpu().numpy().view(np.uint32)
                assert np.array_equal(got[:want.size], want), (threads, unroll, kind)
                assert got[want.size] == 0x5A5A5A5A
