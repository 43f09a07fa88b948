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
