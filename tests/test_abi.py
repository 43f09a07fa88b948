"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and rejects bad arguments on the host before any HIP call."""

import ctypes
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def mx():
    from mxfp8_decode_gemm_amd import build as b

    if not os.path.exists(b.LIB):
        b.build()
    from mxfp8_decode_gemm_amd import binding

    return binding


def test_exports_every_declared_function(mx):
    names = mx.header_functions()
    assert len(names) == 27
    lib = mx.library()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing


def test_header_constants_match_binding(mx):
    with open(os.path.join(ROOT, "include", "mxgemm.h")) as f:
        h = f.read()
    for name, val in [("MXG_GENERATIONS", 3), ("MXG_PACK_BYTES", 16), ("MXG_MAX_ROWS", 8),
                      ("MXG_STATE_NEXT", 0), ("MXG_STATE_ACTIVE", 1), ("MXG_WS_EPOCH", 0),
                      ("MXG_STATE_WORDS", mx.STATE_WORDS),
                      ("MXG_STATE_PEER_GEN", mx.STATE_PEER_GEN),
                      ("MXG_STATE_PEER_ARR", mx.STATE_PEER_ARR)]:
        assert f"#define {name} {val}" in h
    assert "#define MXG_SENTINEL 0x80000000u" in h
    assert mx.SENTINEL == 0x80000000 and mx.GENERATIONS == 3


def test_sizes(mx):
    assert mx.mxg_mailbox_slots_bytes(4, 65536) == 3 * 4 * 65536
    assert mx.mxg_mailbox_slots_bytes(0, 64) == 0
    assert mx.mxg_mailbox_slots_bytes(9, 64) == 0
    assert mx.mxg_mailbox_slots_bytes(1, 24) == 0
    assert mx.mxgemm_workspace_bytes(8, 7168, 8192, 1) == 0
    assert mx.mxgemm_workspace_bytes(8, 7168, 8192, 4) == 256 + 8192 + 4 * 64 * 7168


def _mb(mx, slots=256, state=512, ranks=1, rank=0, cap=512):
    mb = mx.mxg_mailbox()
    mb.slots, mb.state, mb.ranks, mb.rank, mb.capacity_bytes = slots, state, ranks, rank, cap
    return mb


@pytest.mark.parametrize("kw,code", [
    (dict(m=0), -1), (dict(m=9), -1), (dict(n=12), -1), (dict(k=96), -1),
    (dict(split_k=3), -1), (dict(split_k=8, k=512), -1), (dict(w=0), -1),
    (dict(w=272 + 4), -2), (dict(x_scale=4096 + 8), -2), (dict(c_out=8200), -2),
    (dict(n=512), -3), (dict(split_k=2), -4), (dict(split_k=2, ws=4096, ws_bytes=100), -4),
])
def test_publish_validation(mx, kw, code):
    args = dict(w=4096, w_scale=4096, x=4096, x_scale=4096, m=1, n=256, k=512, split_k=1,
                ws=None, ws_bytes=0, c_out=None)
    args.update(kw)
    mb = _mb(mx)
    rc = mx.library().mxgemm_publish(ctypes.byref(mb), args["w"], args["w_scale"], args["x"],
                                     args["x_scale"], args["m"], args["n"], args["k"],
                                     args["split_k"], args["ws"], args["ws_bytes"],
                                     args["c_out"], None)
    assert rc == code


def test_publish_validation_raises(mx):
    mb = _mb(mx)
    with pytest.raises(mx.MxgValueError):
        mx.mxgemm_publish(mb, 4096, 4096, 4096, 4096, 9, 256, 512, 1, None, 0, None, 0)


@pytest.mark.parametrize("kw,code", [
    (dict(ranks=0), -1), (dict(ranks=9), -1), (dict(rank=1), -1), (dict(cap=24), -1),
    (dict(slots=0), -1), (dict(slots=4100), -2),
])
def test_mailbox_init_validation(mx, kw, code):
    a = dict(slots=4096, state=8192, ranks=1, rank=0, cap=512)
    a.update(kw)
    mb = mx.mxg_mailbox()
    rc = mx.library().mailbox_init(ctypes.byref(mb), a["slots"], a["state"], a["ranks"],
                                   a["rank"], a["cap"], None)
    assert rc == code


@pytest.mark.parametrize("nbytes,code", [(0, -3), (24, -3), (1024, -3), (-16, -3)])
def test_collect_and_publish_capacity(mx, nbytes, code):
    mb = _mb(mx)
    lib = mx.library()
    assert lib.mailbox_collect(ctypes.byref(mb), 4096, nbytes, None) == code
    assert lib.mailbox_collect_sum(ctypes.byref(mb), 4096, nbytes, None) == code
    assert lib.mailbox_publish(ctypes.byref(mb), 0, 4096, nbytes, None) == code
    assert lib.mailbox_publish(ctypes.byref(mb), 1, 4096, 16, None) == -1
    assert lib.mailbox_collect(ctypes.byref(mb), 4100, 16, None) == -2
    assert lib.mailbox_collect_sum(ctypes.byref(mb), 4100, 16, None) == -2
    assert lib.mailbox_collect_sum(ctypes.byref(mb), None, 16, None) == -1
    assert lib.mailbox_publish_words(ctypes.byref(mb), 0, 4096, nbytes, None) == code
    assert lib.mailbox_publish_words(ctypes.byref(mb), 1, 4096, 16, None) == -1
    assert lib.mailbox_all_gather(ctypes.byref(mb), 8192, 4096, nbytes, None) == code
    assert lib.mailbox_all_gather(ctypes.byref(mb), 8200, 4096, 16, None) == -2
    assert lib.mailbox_all_gather(ctypes.byref(mb), None, 4096, 16, None) == -1


def test_all_gather_overlap(mx):
    """src may be exactly the caller's own output row, nothing else in out."""
    lib = mx.library()
    mb = _mb(mx, ranks=2, rank=1)
    # out = [4096, 4096 + 2*64); own row at 4096 + 64
    assert lib.mailbox_all_gather(ctypes.byref(mb), 4096, 4096, 64, None) == -1
    assert lib.mailbox_all_gather(ctypes.byref(mb), 4096 + 48, 4096, 64, None) == -1
    assert lib.mailbox_all_gather(ctypes.byref(mb), 4096 - 48, 4096, 64, None) == -1


def test_pack_sizes_and_validation(mx):
    assert mx.mxgemm_packed_weight_bytes(7168, 8192) == 7168 * 8192
    assert mx.mxgemm_packed_weight_bytes(24, 128) == 32 * 128
    # scale tiles, then one range word per 16-row block rounded up to 16 bytes
    assert mx.mxgemm_packed_scale_bytes(24, 128) == 32 * 4 + 16
    assert mx.mxgemm_packed_scale_bytes(7168, 8192) == 7168 * 256 + 448 * 4
    assert mx.mxgemm_packed_scale_bytes(80, 128) == 80 * 4 + 32
    assert mx.mxgemm_packed_weight_bytes(8, 96) == 0
    lib = mx.library()
    assert lib.mxgemm_pack_weight(4096, 4096, 12, 128, 4096, 4096, None) == -1
    assert lib.mxgemm_pack_weight(4096, 4096, 16, 100, 4096, 4096, None) == -1
    assert lib.mxgemm_pack_weight(None, 4096, 16, 128, 4096, 4096, None) == -1
    assert lib.mxgemm_pack_weight(4100, 4096, 16, 128, 4096, 4096, None) == -2


def test_misc(mx):
    lib = mx.library()
    assert mx.strerror(0) == "ok" and "aligned" in mx.strerror(-2)
    # the descriptor as the header declares it: the poll limit travels in it
    assert ctypes.sizeof(mx.mxg_mailbox) == 40
    assert mx.mxg_mailbox.spin_limit.offset == 32 and mx.mxg_mailbox.reserved.offset == 36
    assert not hasattr(lib, "mxg_set_spin_limit")  # no process-wide knob
    assert lib.mxg_graph_begin(None) == -1
    assert lib.mxg_graph_launch(None, None) == -1
    assert lib.mxg_graph_destroy(None) == -1
    assert lib.mxgemm_workspace_init(None, 1024, None) == -1
    assert lib.mxgemm_workspace_init(4096, 1024, None) == -1  # below header + epoch words
    assert lib.mxgemm_workspace_init(4100, 8448, None) == -2


def test_noalloc_validation(mx):
    """mxgemm_publish_noalloc: mxgemm_publish's rules, plus a refusal of split-K
    shapes whose pairs do not fit the library's array (split_k * ceil(n/8)*8 >
    65536), all decided on the host before any HIP call."""
    lib = mx.library()
    mb = _mb(mx, cap=1 << 20)

    def call(**kw):
        a = dict(w=4096, ws=4096, x=4096, xs=4096, m=1, n=256, k=1024, s=1, c=None)
        a.update(kw)
        return lib.mxgemm_publish_noalloc(ctypes.byref(mb), a["w"], a["ws"], a["x"], a["xs"],
                                          a["m"], a["n"], a["k"], a["s"], a["c"], None)

    assert lib.mxgemm_publish_noalloc(None, 4096, 4096, 4096, 4096, 1, 256, 1024, 1, None,
                                      None) == -1
    assert call(m=9) == -1
    assert call(n=12) == -1
    assert call(s=3) == -1
    assert call(s=8, k=512) == -1
    assert call(w=None) == -1
    assert call(x=4100) == -2
    assert call(c=8200) == -2
    assert call(n=1 << 20) == -3           # 2 m n above the slot
    assert call(n=16384, s=8) == -4        # 8 * 16384 pairs columns > 65536
    assert call(n=65536 + 8, s=2) == -4
    assert mx.NOALLOC_PAIR_BYTES == 4 << 20
    with open(os.path.join(ROOT, "include", "mxgemm.h")) as f:
        assert "#define MXG_NOALLOC_PAIR_BYTES (4u << 20)" in f.read()


def test_bf16_publish_validation(mx):
    """mxgemm_publish_bf16: BF16 x required, the two quantized outputs given
    together or not at all, the usual size, alignment and capacity rules."""
    lib = mx.library()
    mb = _mb(mx)

    def call(**kw):
        a = dict(w=4096, ws=4096, x=4096, m=1, n=256, k=512, s=1, wsp=None, wsn=0, c=None,
                 q=None, qs=None)
        a.update(kw)
        return lib.mxgemm_publish_bf16(ctypes.byref(mb), a["w"], a["ws"], a["x"], a["m"],
                                       a["n"], a["k"], a["s"], a["wsp"], a["wsn"], a["c"],
                                       a["q"], a["qs"], None)

    assert call(x=None) == -1
    assert call(m=9) == -1
    assert call(k=96) == -1
    assert call(q=8192) == -1          # codes without scales
    assert call(qs=8192) == -1         # scales without codes
    assert call(x=4096 + 8) == -2
    assert call(q=8192 + 8, qs=9000) == -2
    assert call(n=512) == -3           # 2*m*n above the 512-byte slot
    assert call(s=4) == -4
    assert lib.mxgemm_publish_bf16(None, 4096, 4096, 4096, 1, 256, 512, 1, None, 0, None, None,
                                   None, None) == -1


def test_plain_gemm_validation(mx):
    lib = mx.library()

    def call(**kw):
        a = dict(w=4096, ws=4096, x=4096, xs=4096, m=1, n=256, k=512, s=1, wsp=None, wsn=0,
                 c=8192)
        a.update(kw)
        return lib.mxgemm(a["w"], a["ws"], a["x"], a["xs"], a["m"], a["n"], a["k"], a["s"],
                          a["wsp"], a["wsn"], a["c"], None)

    assert call(c=None) == -1          # the output is the only result
    assert call(x=None) == -1
    assert call(m=0) == -1
    assert call(c=8200) == -2
    assert call(s=2) == -4


def test_quantize_validation(mx):
    lib = mx.library()
    assert lib.mxfp8_quantize(None, 1, 32, 4096, 8192, None) == -1
    assert lib.mxfp8_quantize(4096, 0, 32, 4096, 8192, None) == -1
    assert lib.mxfp8_quantize(4096, 1, 48, 4096, 8192, None) == -1
    assert lib.mxfp8_quantize(4096, 1, 32, None, 8192, None) == -1
    assert lib.mxfp8_quantize(4100, 1, 32, 4096, 8192, None) == -2
    assert lib.mxfp8_quantize(4096, 1, 32, 4104, 8192, None) == -2


def test_stream_read_validation(mx):
    lib = mx.library()
    assert lib.mxg_stream_read(None, 64, 8192, None) == -1
    assert lib.mxg_stream_read(4096, 0, 8192, None) == -1
    assert lib.mxg_stream_read(4096, 24, 8192, None) == -1
    assert lib.mxg_stream_read(4096, 64, None, None) == -1
    assert lib.mxg_stream_read(4104, 64, 8192, None) == -2
    assert lib.mxg_stream_read(4096, 64, 8194, None) == -2
    with open(os.path.join(ROOT, "include", "mxgemm.h")) as f:
        assert f"#define MXG_STREAM_CHUNK_BYTES {mx.STREAM_CHUNK_BYTES}" in f.read()


def test_probe_mfma_validation(mx):
    lib = mx.library()
    assert lib.mxg_probe_mfma(None, 16, 4096, 16, 128, 0, 8192, None) == -1
    assert lib.mxg_probe_mfma(4096, 16, 4096, 16, 0, 0, 8192, None) == -1
    assert lib.mxg_probe_mfma(4096, 16, 4096, 16, 96, 0, 8192, None) == -1
    assert lib.mxg_probe_mfma(4096, 16, 4096, 16, 128, 2, 8192, None) == -1
    assert lib.mxg_probe_mfma(4096, 16, 4096, 16, 128, 1, None, None) == -1
    assert lib.mxg_probe_mfma(4100, 16, 4096, 16, 128, 1, 8192, None) == -2
    assert lib.mxg_probe_mfma(4096, 16, 4096, 16, 128, 1, 8196, None) == -2


def test_tile_validation(mx):
    """mxgemm_tile: a tile spec is required, the plain form needs c_out, BF16
    x only with a mailbox and never beside MXFP8 x; then mxgemm_publish's
    validation (here: m out of range) before any HIP call."""
    lib = mx.library()
    args = [4096, 4096, 4096, 4096, None, 8, 256, 512, 1, None, 0, 8192, None, None, None]
    assert lib.mxgemm_tile(None, None, *args) == -1
    assert lib.mxgemm_tile(b"fp8", None, *args[:11], None, None, None, None) == -1
    plain_bf16 = args[:2] + [None, None, 4096] + args[5:]
    assert lib.mxgemm_tile(b"fp8", None, *plain_bf16) == -1
    assert lib.mxgemm_tile(b"1,7,1,5", None, *(args[:5] + [0] + args[6:])) == -1


def test_stream_read_cfg_validation(mx):
    lib = mx.library()
    ok = [4096, 65536, 8192, 0, 256, 8, 0, 0, None]
    def call(**kw):
        a = list(ok)
        for i, name in enumerate(["src", "bytes", "sink", "wg", "threads", "unroll", "kind",
                                  "inter", "stream"]):
            if name in kw:
                a[i] = kw[name]
        return lib.mxg_stream_read_cfg(*a)
    assert call(src=None) == -1
    assert call(bytes=24) == -1
    assert call(threads=128) == -1
    assert call(unroll=2) == -1
    assert call(kind=5) == -1
    assert call(inter=1, wg=0) == -1
    assert call(wg=-1) == -1
    assert call(kind=2, bytes=0x80000000) == -1
    assert call(src=4104) == -2
    assert call(sink=8194) == -2
