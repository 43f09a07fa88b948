"""ctypes binding of libmxgemm.so: the C ABI of include/mxgemm.h, same names.

Argument marshalling only: every step of the hot path runs in the HIP
library. Device buffers may be passed as torch tensors (their data_ptr is
used) or as integer device addresses; streams as torch streams, raw
hipStream_t integers or None (torch's current stream). Importing this module
loads the library and raises if it has not been built: there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
# MXG_LIBRARY names another build of the same library to load (the host
# sanitizer build of the ABI tests); the default is the in-tree build.
LIB_PATH = os.environ.get("MXG_LIBRARY") or os.path.join(_PKG, "lib", "libmxgemm.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "mxgemm.h")

OK = 0
EINVAL = -1
EALIGN = -2
ECAPACITY = -3
EWORKSPACE = -4
EUNSUPPORTED = -5
EHIP = -6

GENERATIONS = 3
PACK_BYTES = 16
SENTINEL = 0x80000000
MAX_RANKS = 8
MAX_ROWS = 8
STATE_WORDS = 32
STATE_NEXT, STATE_ACTIVE, STATE_COLLECT_ARR, STATE_ERROR = 0, 1, 2, 3
STATE_PEER_GEN, STATE_PEER_ARR = 8, 16
WS_HEADER_BYTES = 256
WS_FLAG_BYTES = 8192
WS_MAX_GROUPS = 2048
NOALLOC_PAIR_BYTES = 4 << 20
WS_EPOCH, WS_ERROR = 0, 2
ERR_COLLECT_SPIN = 0x1
ERR_SPLITK_SPIN = 0x2


class MxgError(Exception):
    """A non-zero return code of the library."""

    def __init__(self, code: int, what: str) -> None:
        super().__init__(f"{what}: {strerror(code)} ({code})")
        self.code = code


class MxgValueError(MxgError, ValueError):
    """The arguments were rejected on the host; nothing was enqueued."""


class MxgUnsupported(MxgValueError):
    """Valid arguments that no kernel variant takes: the caller falls back."""


class MxgHipError(MxgError, RuntimeError):
    """A HIP call failed."""


class mxg_mailbox(ctypes.Structure):
    _fields_ = [
        ("slots", ctypes.c_void_p),
        ("state", ctypes.c_void_p),
        ("ranks", ctypes.c_int32),
        ("rank", ctypes.c_int32),
        ("capacity_bytes", ctypes.c_int64),
        ("spin_limit", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
    ]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m mxfp8_decode_gemm_amd.build` "
            "(there is no fallback implementation)"
        )
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz, u32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                             ctypes.c_size_t, ctypes.c_uint32)
    mbp = ctypes.POINTER(mxg_mailbox)
    sig = {
        "mxg_mailbox_slots_bytes": (sz, [i32, i64]),
        "mailbox_init": (ctypes.c_int, [mbp, vp, vp, i32, i32, i64, vp]),
        "mxgemm_workspace_bytes": (sz, [i32, i32, i32, i32]),
        "mxgemm_workspace_init": (ctypes.c_int, [vp, sz, vp]),
        "mxgemm_packed_weight_bytes": (sz, [i32, i32]),
        "mxgemm_packed_scale_bytes": (sz, [i32, i32]),
        "mxgemm_pack_weight": (ctypes.c_int, [vp, vp, i32, i32, vp, vp, vp]),
        "mxgemm_publish": (ctypes.c_int, [mbp, vp, vp, vp, vp, i32, i32, i32, i32, vp, sz,
                                          vp, vp]),
        "mxgemm_publish_timed": (ctypes.c_int, [mbp, vp, vp, vp, vp, i32, i32, i32, i32, vp,
                                                sz, vp, vp, vp, vp]),
        "mxgemm_publish_noalloc": (ctypes.c_int, [mbp, vp, vp, vp, vp, i32, i32, i32, i32, vp,
                                                  vp]),
        "mailbox_publish": (ctypes.c_int, [mbp, i32, vp, i64, vp]),
        "mailbox_collect": (ctypes.c_int, [mbp, vp, i64, vp]),
        "mailbox_collect_sum": (ctypes.c_int, [mbp, vp, i64, vp]),
        "mailbox_publish_words": (ctypes.c_int, [mbp, i32, vp, i64, vp]),
        "mxgemm_publish_bf16": (ctypes.c_int, [mbp, vp, vp, vp, i32, i32, i32, i32, vp, sz, vp,
                                               vp, vp, vp]),
        "mxgemm": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, i32, i32, vp, sz, vp, vp]),
        "mxgemm_tile": (ctypes.c_int, [ctypes.c_char_p, mbp, vp, vp, vp, vp, vp, i32, i32, i32,
                                       i32, vp, sz, vp, vp, vp, vp]),
        "mxfp8_quantize": (ctypes.c_int, [vp, i32, i32, vp, vp, vp]),
        "mailbox_all_gather": (ctypes.c_int, [mbp, vp, vp, i64, vp]),
        "mxg_stream_read": (ctypes.c_int, [vp, sz, vp, vp]),
        "mxg_probe_mfma": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, vp, vp]),
        "mxg_stream_read_cfg": (ctypes.c_int, [vp, sz, vp, i32, i32, i32, i32, i32, vp]),
        "mxg_graph_begin": (ctypes.c_int, [vp]),
        "mxg_graph_end": (ctypes.c_int, [vp, ctypes.POINTER(vp)]),
        "mxg_graph_launch": (ctypes.c_int, [vp, vp]),
        "mxg_graph_destroy": (ctypes.c_int, [vp]),
        "mxg_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def header_functions() -> list[str]:
    """Names of the functions include/mxgemm.h declares."""
    with open(HEADER_PATH) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text,
                       flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def library() -> ctypes.CDLL:
    return _lib


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------


def _ptr(obj) -> int | None:
    if obj is None:
        return None
    if isinstance(obj, int):
        return obj
    dp = getattr(obj, "data_ptr", None)
    if dp is None:
        raise TypeError(f"expected a device tensor or address, got {type(obj).__name__}")
    return int(dp())


def _stream(stream) -> int | None:
    if stream is None:
        import torch

        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _event(ev) -> int | None:
    if ev is None or isinstance(ev, int):
        return ev
    return int(ev.cuda_event)


def _check(code: int, what: str) -> None:
    if code == OK:
        return
    if code == EUNSUPPORTED:
        raise MxgUnsupported(code, what)
    if code == EHIP:
        raise MxgHipError(code, what)
    raise MxgValueError(code, what)


def strerror(code: int) -> str:
    return _lib.mxg_strerror(code).decode()


# ---------------------------------------------------------------------------
# the C ABI, same names
# ---------------------------------------------------------------------------


def mxg_mailbox_slots_bytes(ranks: int, capacity_bytes: int) -> int:
    return int(_lib.mxg_mailbox_slots_bytes(ranks, capacity_bytes))


def mailbox_init(slots, state, ranks: int, rank: int, capacity_bytes: int,
                 stream=None) -> mxg_mailbox:
    mb = mxg_mailbox()
    _check(_lib.mailbox_init(ctypes.byref(mb), _ptr(slots), _ptr(state), ranks, rank,
                             capacity_bytes, _stream(stream)), "mailbox_init")
    return mb


def mxgemm_workspace_bytes(m: int, n: int, k: int, split_k: int) -> int:
    return int(_lib.mxgemm_workspace_bytes(m, n, k, split_k))


def mxgemm_workspace_init(workspace, workspace_bytes: int, stream=None) -> None:
    _check(_lib.mxgemm_workspace_init(_ptr(workspace), workspace_bytes, _stream(stream)),
           "mxgemm_workspace_init")


def mxgemm_packed_weight_bytes(n: int, k: int) -> int:
    return int(_lib.mxgemm_packed_weight_bytes(n, k))


def mxgemm_packed_scale_bytes(n: int, k: int) -> int:
    return int(_lib.mxgemm_packed_scale_bytes(n, k))


def mxgemm_pack_weight(w, w_scale, n: int, k: int, w_packed, ws_packed, stream=None) -> None:
    _check(_lib.mxgemm_pack_weight(_ptr(w), _ptr(w_scale), n, k, _ptr(w_packed),
                                   _ptr(ws_packed), _stream(stream)), "mxgemm_pack_weight")


# Kernel variant for the GEMM calls below (tests and measurement): None for
# the library's default choice, else a tile spec of mxgemm_tile ("fp8" or
# "rb,wn,wk,depth[,xr[,x16]]"); when set, mxgemm_publish, mxgemm_publish_bf16
# and mxgemm go through mxgemm_tile with it. Python-side only: the library
# itself keeps no such setting.
TILE = None


def _tile_call(mb, w, w_scale, x, x_scale, x_bf16, m, n, k, split_k, workspace,
               workspace_bytes, c_out, x_q_out, x_scale_out, stream, what):
    _check(_lib.mxgemm_tile(TILE.encode(), ctypes.byref(mb) if mb is not None else None,
                            _ptr(w), _ptr(w_scale), _ptr(x), _ptr(x_scale), _ptr(x_bf16), m, n,
                            k, split_k, _ptr(workspace), workspace_bytes, _ptr(c_out),
                            _ptr(x_q_out), _ptr(x_scale_out), _stream(stream)), what)


def mxgemm_tile(tile: str, mb, w, w_scale, x, x_scale, x_bf16, m: int, n: int, k: int,
                split_k: int, workspace, workspace_bytes: int, c_out=None, x_q_out=None,
                x_scale_out=None, stream=None) -> None:
    _check(_lib.mxgemm_tile(tile.encode(), ctypes.byref(mb) if mb is not None else None,
                            _ptr(w), _ptr(w_scale), _ptr(x), _ptr(x_scale), _ptr(x_bf16), m, n,
                            k, split_k, _ptr(workspace), workspace_bytes, _ptr(c_out),
                            _ptr(x_q_out), _ptr(x_scale_out), _stream(stream)), "mxgemm_tile")


def mxgemm_publish(mb: mxg_mailbox, w, w_scale, x, x_scale, m: int, n: int, k: int,
                   split_k: int = 1, workspace=None, workspace_bytes: int = 0,
                   c_out=None, stream=None) -> None:
    if TILE is not None:
        return _tile_call(mb, w, w_scale, x, x_scale, None, m, n, k, split_k, workspace,
                          workspace_bytes, c_out, None, None, stream, "mxgemm_publish")
    _check(_lib.mxgemm_publish(ctypes.byref(mb), _ptr(w), _ptr(w_scale), _ptr(x),
                               _ptr(x_scale), m, n, k, split_k, _ptr(workspace),
                               workspace_bytes, _ptr(c_out), _stream(stream)),
           "mxgemm_publish")


def mxgemm_publish_timed(mb: mxg_mailbox, w, w_scale, x, x_scale, m: int, n: int, k: int,
                         split_k: int, workspace, workspace_bytes: int, c_out, stream,
                         ev_start, ev_stop) -> None:
    """mxgemm_publish with HIP events recorded around the kernel itself;
    events are torch.cuda.Event objects (their cuda_event handle is passed)
    or raw hipEvent_t integers."""
    _check(_lib.mxgemm_publish_timed(ctypes.byref(mb), _ptr(w), _ptr(w_scale), _ptr(x),
                                     _ptr(x_scale), m, n, k, split_k, _ptr(workspace),
                                     workspace_bytes, _ptr(c_out), _stream(stream),
                                     _event(ev_start), _event(ev_stop)),
           "mxgemm_publish_timed")


def mxgemm_publish_noalloc(mb: mxg_mailbox, w, w_scale, x, x_scale, m: int, n: int, k: int,
                           split_k: int = 1, c_out=None, stream=None) -> None:
    _check(_lib.mxgemm_publish_noalloc(ctypes.byref(mb), _ptr(w), _ptr(w_scale), _ptr(x),
                                       _ptr(x_scale), m, n, k, split_k, _ptr(c_out),
                                       _stream(stream)),
           "mxgemm_publish_noalloc")


def mailbox_publish(mb: mxg_mailbox, rank: int, src, nbytes: int, stream=None) -> None:
    _check(_lib.mailbox_publish(ctypes.byref(mb), rank, _ptr(src), nbytes, _stream(stream)),
           "mailbox_publish")


def mailbox_collect(mb: mxg_mailbox, out, nbytes: int, stream=None) -> None:
    _check(_lib.mailbox_collect(ctypes.byref(mb), _ptr(out), nbytes, _stream(stream)),
           "mailbox_collect")


def mailbox_collect_sum(mb: mxg_mailbox, out, nbytes: int, stream=None) -> None:
    _check(_lib.mailbox_collect_sum(ctypes.byref(mb), _ptr(out), nbytes, _stream(stream)),
           "mailbox_collect_sum")


def mxgemm_publish_bf16(mb: mxg_mailbox, w, w_scale, x, m: int, n: int, k: int, split_k: int,
                        workspace, workspace_bytes: int, c_out=None, x_q_out=None,
                        x_scale_out=None, stream=None) -> None:
    if TILE is not None:
        return _tile_call(mb, w, w_scale, None, None, x, m, n, k, split_k, workspace,
                          workspace_bytes, c_out, x_q_out, x_scale_out, stream,
                          "mxgemm_publish_bf16")
    _check(_lib.mxgemm_publish_bf16(ctypes.byref(mb), _ptr(w), _ptr(w_scale), _ptr(x), m, n, k,
                                    split_k, _ptr(workspace), workspace_bytes, _ptr(c_out),
                                    _ptr(x_q_out), _ptr(x_scale_out), _stream(stream)),
           "mxgemm_publish_bf16")


def mxgemm(w, w_scale, x, x_scale, m: int, n: int, k: int, split_k: int, workspace,
           workspace_bytes: int, c_out, stream=None) -> None:
    if TILE is not None:
        return _tile_call(None, w, w_scale, x, x_scale, None, m, n, k, split_k, workspace,
                          workspace_bytes, c_out, None, None, stream, "mxgemm")
    _check(_lib.mxgemm(_ptr(w), _ptr(w_scale), _ptr(x), _ptr(x_scale), m, n, k, split_k,
                       _ptr(workspace), workspace_bytes, _ptr(c_out), _stream(stream)),
           "mxgemm")


def mxfp8_quantize(x, rows: int, k: int, x_q, x_scale, stream=None) -> None:
    _check(_lib.mxfp8_quantize(_ptr(x), rows, k, _ptr(x_q), _ptr(x_scale), _stream(stream)),
           "mxfp8_quantize")


def mailbox_publish_words(mb: mxg_mailbox, rank: int, src, nbytes: int, stream=None) -> None:
    _check(_lib.mailbox_publish_words(ctypes.byref(mb), rank, _ptr(src), nbytes,
                                      _stream(stream)), "mailbox_publish_words")


def mailbox_all_gather(mb: mxg_mailbox, src, out, nbytes: int, stream=None) -> None:
    _check(_lib.mailbox_all_gather(ctypes.byref(mb), _ptr(src), _ptr(out), nbytes,
                                   _stream(stream)), "mailbox_all_gather")


STREAM_CHUNK_BYTES = 32768


def mxg_probe_mfma(a, a_scale, b, b_scale, k: int, scaled: bool, c, stream=None) -> None:
    _check(_lib.mxg_probe_mfma(_ptr(a), _ptr(a_scale), _ptr(b), _ptr(b_scale), k,
                               1 if scaled else 0, _ptr(c), _stream(stream)), "mxg_probe_mfma")


def mxg_stream_read_cfg(src, nbytes: int, sink, workgroups: int, threads: int, unroll: int,
                        load_kind: int, interleave: bool, stream=None) -> None:
    _check(_lib.mxg_stream_read_cfg(_ptr(src), nbytes, _ptr(sink), workgroups, threads, unroll,
                                    load_kind, 1 if interleave else 0, _stream(stream)),
           "mxg_stream_read_cfg")


def mxg_stream_read(src, nbytes: int, sink, stream=None) -> None:
    _check(_lib.mxg_stream_read(_ptr(src), nbytes, _ptr(sink), _stream(stream)),
           "mxg_stream_read")


def mxg_graph_begin(stream=None) -> None:
    _check(_lib.mxg_graph_begin(_stream(stream)), "mxg_graph_begin")


def mxg_graph_end(stream=None) -> int:
    exec_ = ctypes.c_void_p()
    _check(_lib.mxg_graph_end(_stream(stream), ctypes.byref(exec_)), "mxg_graph_end")
    return int(exec_.value)


def mxg_graph_launch(exec_: int, stream=None) -> None:
    _check(_lib.mxg_graph_launch(exec_, _stream(stream)), "mxg_graph_launch")


def mxg_graph_destroy(exec_: int) -> None:
    _check(_lib.mxg_graph_destroy(exec_), "mxg_graph_destroy")


def mxg_strerror(code: int) -> str:
    return strerror(code)
