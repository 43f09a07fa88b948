"""Device-memory plumbing around the C ABI (torch allocates, the library computes).

``Mailbox`` owns the slot and state buffers of one mailbox; ``Workspace`` owns
a split-K workspace; ``upload`` places MXFP8 operands in HBM. Nothing here
computes any part of the GEMM or the mailbox protocol: every call goes
through ``binding``.
"""

from __future__ import annotations

import numpy as np
import torch

from . import binding as mx


def _dev(device) -> torch.device:
    d = torch.device(device if device is not None else "cuda")
    if d.type != "cuda":
        raise ValueError("the MXFP8 publishing GEMM runs on a HIP device")
    return d


def upload(a: np.ndarray, device=None) -> torch.Tensor:
    """A contiguous device copy of a numpy array (uint8/uint16/...)."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(_dev(device))


class Mailbox:
    """A three-generation mailbox of ``ranks`` slots of ``capacity_bytes``."""

    def __init__(self, ranks: int, capacity_bytes: int, rank: int = 0, device=None,
                 stream=None) -> None:
        dev = _dev(device)
        nbytes = mx.mxg_mailbox_slots_bytes(ranks, capacity_bytes)
        if nbytes == 0:
            raise ValueError("invalid mailbox geometry")
        self.slots = torch.empty(nbytes // 4, dtype=torch.int32, device=dev)
        self.state = torch.empty(mx.STATE_WORDS, dtype=torch.int32, device=dev)
        self.ranks, self.rank, self.capacity_bytes = ranks, rank, capacity_bytes
        self.mb = mx.mailbox_init(self.slots, self.state, ranks, rank, capacity_bytes, stream)

    def reinit(self, stream=None) -> None:
        self.mb = mx.mailbox_init(self.slots, self.state, self.ranks, self.rank,
                                  self.capacity_bytes, stream)

    @property
    def spin_limit(self) -> int:
        """Polls before a device wait of a call on this mailbox gives up (0:
        the library's default); carried in the descriptor, read at launch."""
        return int(self.mb.spin_limit)

    @spin_limit.setter
    def spin_limit(self, polls: int) -> None:
        self.mb.spin_limit = polls

    def state_words(self) -> np.ndarray:
        return self.state.cpu().numpy().view(np.uint32).copy()

    def slot_words(self) -> np.ndarray:
        """uint32 [3, ranks, capacity/4] copy of the whole mailbox."""
        w = self.slots.cpu().numpy().view(np.uint32)
        return w.reshape(mx.GENERATIONS, self.ranks, self.capacity_bytes // 4).copy()


class Workspace:
    """A split-K workspace large enough for ``n`` output columns at ``split_k``."""

    def __init__(self, n: int, split_k: int, device=None, stream=None) -> None:
        self.nbytes = max(mx.mxgemm_workspace_bytes(8, n, 128 * split_k, split_k),
                          mx.WS_HEADER_BYTES + mx.WS_FLAG_BYTES)
        self.buf = torch.empty(self.nbytes // 4, dtype=torch.int32, device=_dev(device))
        mx.mxgemm_workspace_init(self.buf, self.nbytes, stream)

    def header(self) -> np.ndarray:
        return self.buf[: mx.WS_HEADER_BYTES // 4].cpu().numpy().view(np.uint32).copy()


def pack_weight(w: torch.Tensor, ws: torch.Tensor, n: int, k: int, stream=None):
    """Device copies of W and its scales in the GEMM's packed tile layout."""
    wp = torch.empty(mx.mxgemm_packed_weight_bytes(n, k), dtype=torch.uint8, device=w.device)
    wsp = torch.empty(mx.mxgemm_packed_scale_bytes(n, k), dtype=torch.uint8, device=w.device)
    mx.mxgemm_pack_weight(w, ws, n, k, wp, wsp, stream)
    return wp, wsp


class Operands:
    """A problem's MXFP8 operands in HBM; W and its scales packed once."""

    def __init__(self, problem, device=None) -> None:
        self.m, self.n, self.k = problem.m, problem.n, problem.k
        w = upload(problem.w, device)
        ws = upload(problem.ws, device)
        self.w, self.ws = pack_weight(w, ws, self.n, self.k)
        self.x = upload(problem.x, device)
        self.xs = upload(problem.xs, device)


def publish(mailbox: Mailbox, ops: Operands, split_k: int = 1, workspace: Workspace = None,
            c_out: torch.Tensor = None, stream=None) -> None:
    """One mxgemm_publish call on device operands."""
    mx.mxgemm_publish(mailbox.mb, ops.w, ops.ws, ops.x, ops.xs, ops.m, ops.n, ops.k, split_k,
                      workspace.buf if workspace is not None else None,
                      workspace.nbytes if workspace is not None else 0, c_out, stream)


def collect(mailbox: Mailbox, nbytes: int, out: torch.Tensor = None, stream=None) -> torch.Tensor:
    """One mailbox_collect; returns the [ranks * nbytes] byte output as uint16."""
    if out is None:
        out = torch.empty(mailbox.ranks * nbytes // 2, dtype=torch.int16,
                          device=mailbox.slots.device)
    mx.mailbox_collect(mailbox.mb, out, nbytes, stream)
    return out


def collect_sum(mailbox: Mailbox, nbytes: int, out: torch.Tensor = None,
                stream=None) -> torch.Tensor:
    """One mailbox_collect_sum; returns the [nbytes] byte all-reduce as uint16."""
    if out is None:
        out = torch.empty(nbytes // 2, dtype=torch.int16, device=mailbox.slots.device)
    mx.mailbox_collect_sum(mailbox.mb, out, nbytes, stream)
    return out


def all_gather(mailbox: Mailbox, src: torch.Tensor, nbytes: int, out: torch.Tensor = None,
               stream=None) -> torch.Tensor:
    """One mailbox_all_gather of slot mailbox.rank; returns the [ranks * nbytes]
    byte output as int32 words."""
    if out is None:
        out = torch.empty(mailbox.ranks * nbytes // 4, dtype=torch.int32,
                          device=mailbox.slots.device)
    mx.mailbox_all_gather(mailbox.mb, src, out, nbytes, stream)
    return out


def as_u16(t: torch.Tensor) -> np.ndarray:
    """uint16 host copy of a 16-bit device tensor."""
    return t.cpu().numpy().view(np.uint16).copy()
