"""The three-generation Lamport mailbox, word by word.

Test infrastructure only (see the package docstring).

What it models (all_gather page, module docstring, steps 1-3, and
``_AllGatherKernel.kernel``; publishing_gemm page, module docstring):

* Layout: mailbox[generation][rank][...] with 3 generations and one slot of
  ``capacity_bytes`` per rank, handled in 16-byte packs; every idle word holds
  the sentinel 0x80000000.
* Publish: a call writes its payload into its own slot of the current
  generation. The GEMM's payload is its [m, N] BF16 output, row-major, with
  negative zero cleared; eight consecutive columns of one token make one
  16-byte pack, the even column in the low half of each 32-bit word. The
  publisher records the generation it wrote (the "active" stage word of the
  publishing_gemm page).
* Collect: every slot of the generation, the caller's own included, is read
  once no word of it is the sentinel (here: the model raises ``WouldSpin``
  where the device would keep polling), copied out rank-major ([R*m, N], the
  layout of a dim-0 gather) and reset to the sentinel. The collect advances
  the generation to (g + 1) mod 3.
* Generation word = number of completed collects mod 3.

The slot uses the prefix [0, 2 m N) of each rank's ``capacity_bytes``, so calls
of different sizes share one mailbox (the all_gather page's byte-capacity
layout; the publishing_gemm page's fixed hidden-size stride is the other
reading, not used).

Word payloads (all_gather page, module docstring, step 1, and
``LamportAllGather.__call__``): the all-gather moves arbitrary 32-bit words,
and a word equal to the sentinel is published as 0 (FP32 negative zero becomes
positive zero); every other word is published unchanged. ``publish_words``
models that publish, ``all_gather`` the fused call (publish the caller's own
slot, then collect every slot).

All-reduce consumer (publishing_gemm page, module docstring: the GEMM's
published output is summed across ranks by the boundary all-reduce). The pages
do not print its internals, so it is taken from the plain meaning of an
all-reduce in FP32: ``collect_sum`` returns, for every BF16 position, the FP32
sum of the rank slots' values taken in ascending rank order, rounded once to
BF16 (nearest even); the mailbox is reset and advanced exactly as by
``collect``.

``EpochModel`` models the split-K hand-off tag: it starts at 1, and every GEMM
call that exchanges partials advances it by one, skipping 0 on wrap-around
(sync page, ``Mailbox`` docstring: each launch tags its hand-offs with its
epoch so a pair from an earlier step never carries a live tag).
"""

from __future__ import annotations

import numpy as np

from .codecs import SENTINEL_U32, bf16_rne_bits, bf16_to_f64, clear_negative_zero

GENERATIONS = 3  # all_gather page, module docstring: three generations
PACK_BYTES = 16  # all_gather page: one thread a 16-byte pack
MAX_RANKS = 8


class WouldSpin(RuntimeError):
    """A collect found a sentinel word: on the device it would keep polling."""


def accepts(nbytes: int, capacity_bytes: int) -> bool:
    """A payload fits when it is 1..capacity bytes and a multiple of 16
    (all_gather page, ``LamportAllGather.accepts``)."""
    return 0 < nbytes <= capacity_bytes and nbytes % PACK_BYTES == 0


def halves_to_words(halves: np.ndarray) -> np.ndarray:
    """uint32 words of a flat uint16 array: word j = h[2j] | h[2j+1] << 16."""
    h = np.asarray(halves, dtype=np.uint16).reshape(-1)
    if h.size % 2:
        raise ValueError("an odd number of BF16 halves does not fill words")
    lo = h[0::2].astype(np.uint32)
    hi = h[1::2].astype(np.uint32)
    return (lo | (hi << np.uint32(16))).astype(np.uint32)


def words_to_halves(words: np.ndarray) -> np.ndarray:
    """Inverse of ``halves_to_words``."""
    w = np.asarray(words, dtype=np.uint32).reshape(-1)
    out = np.empty(w.size * 2, dtype=np.uint16)
    out[0::2] = (w & np.uint32(0xFFFF)).astype(np.uint16)
    out[1::2] = (w >> np.uint32(16)).astype(np.uint16)
    return out


class MailboxModel:
    """Host model of one mailbox with ``ranks`` emulated rank slots.

    One generation counter serves every slot. Each rank keeps its own counter
    and advances it once per call (all_gather page, module docstring, step
    3); when every peer publishes once per collect, all the counters agree
    with this one between calls."""

    def __init__(self, ranks: int, capacity_bytes: int) -> None:
        if not 1 <= ranks <= MAX_RANKS:
            raise ValueError("1..8 rank slots")
        if capacity_bytes <= 0 or capacity_bytes % PACK_BYTES:
            raise ValueError("the capacity must be a positive multiple of 16 bytes")
        self.ranks = ranks
        self.capacity_bytes = capacity_bytes
        self.slots = np.full(
            (GENERATIONS, ranks, capacity_bytes // 4), SENTINEL_U32, dtype=np.uint32
        )
        self.next = 0  # generation the next publish writes
        self.active = 0  # generation the last publish wrote
        self.collects = 0

    # -- publish -----------------------------------------------------------
    def publish(self, rank: int, bf16_bits: np.ndarray) -> None:
        """Publish a [m, N] uint16 BF16 payload into slot ``rank`` of the
        current generation, negative zero cleared."""
        if not 0 <= rank < self.ranks:
            raise ValueError("rank outside the mailbox")
        bits = np.asarray(bf16_bits, dtype=np.uint16)
        nbytes = bits.size * 2
        if not accepts(nbytes, self.capacity_bytes):
            raise ValueError(f"payload of {nbytes} bytes does not fit")
        g = self.next
        self.slots[g, rank, : nbytes // 4] = halves_to_words(clear_negative_zero(bits))
        self.active = g

    def publish_words(self, rank: int, words: np.ndarray) -> None:
        """Publish a payload of uint32 words into slot ``rank`` of the current
        generation, each word equal to the sentinel replaced by 0."""
        if not 0 <= rank < self.ranks:
            raise ValueError("rank outside the mailbox")
        w = np.asarray(words, dtype=np.uint32).reshape(-1)
        nbytes = w.size * 4
        if not accepts(nbytes, self.capacity_bytes):
            raise ValueError(f"payload of {nbytes} bytes does not fit")
        g = self.next
        self.slots[g, rank, : w.size] = sanitize_words(w)
        self.active = g

    def all_gather(self, rank: int, words: np.ndarray) -> np.ndarray:
        """The fused all-gather of one rank: publish its words, then collect
        every slot. Returns uint32 words rank-major, [ranks, words]."""
        w = np.asarray(words, dtype=np.uint32).reshape(-1)
        self.publish_words(rank, w)
        out = self.collect(w.size * 4)
        return halves_to_words(out.reshape(-1)).reshape(self.ranks, w.size)

    # -- collect -----------------------------------------------------------
    def collect(self, nbytes: int) -> np.ndarray:
        """Collect ``nbytes`` from every rank slot of the current generation.

        Returns the uint16 halves laid out rank-major, [ranks, nbytes / 2]
        (reshape to [ranks * m, N] for an [m, N] payload)."""
        if not accepts(nbytes, self.capacity_bytes):
            raise ValueError(f"payload of {nbytes} bytes does not fit")
        g = self.next
        words = self.slots[g, :, : nbytes // 4]
        stale = np.argwhere(words == SENTINEL_U32)
        if stale.size:
            r, j = stale[0]
            raise WouldSpin(f"rank {r} word {j} of generation {g} is the sentinel")
        out = np.stack([words_to_halves(words[r]) for r in range(self.ranks)])
        self.slots[g, :, : nbytes // 4] = SENTINEL_U32
        self.next = (g + 1) % GENERATIONS
        self.collects += 1
        return out

    def collect_sum(self, nbytes: int) -> np.ndarray:
        """Collect ``nbytes`` from every rank slot of the current generation
        and return their all-reduce: [nbytes / 2] uint16 BF16 bits (see
        ``allreduce_bf16``). Resets and advances like ``collect``."""
        return allreduce_bf16(self.collect(nbytes))

    # -- invariants --------------------------------------------------------
    def idle(self) -> bool:
        """Every word of every generation is the sentinel."""
        return bool(np.all(self.slots == SENTINEL_U32))


def sanitize_words(words: np.ndarray) -> np.ndarray:
    """uint32 words with every word equal to the sentinel replaced by 0."""
    w = np.asarray(words, dtype=np.uint32)
    return np.where(w == SENTINEL_U32, np.uint32(0), w).astype(np.uint32)


def allreduce_bf16(halves: np.ndarray) -> np.ndarray:
    """All-reduce of R BF16 payloads, [R, H] uint16 -> [H] uint16: each
    position's values are added in FP32 in ascending rank order (each addition
    rounded to FP32, nearest even), and the FP32 total is rounded once to BF16
    (nearest even)."""
    h = np.asarray(halves, dtype=np.uint16)
    if h.ndim != 2 or h.shape[0] < 1:
        raise ValueError("expected [ranks, halves]")
    vals = bf16_to_f64(h).astype(np.float32)  # BF16 -> FP32 is exact
    acc = vals[0].copy()
    for r in range(1, h.shape[0]):
        acc = np.add(acc, vals[r], dtype=np.float32)
    return bf16_rne_bits(acc.astype(np.float64))


def check_collected(out_halves: np.ndarray) -> list[str]:
    """Problems in a collect output: a sentinel word or a negative-zero half.

    Neither can occur: publishes clear negative zero, which also rules out the
    word 0x80000000 (all_gather page, module docstring, step 1)."""
    problems = []
    h = np.asarray(out_halves, dtype=np.uint16)
    words = halves_to_words(h.reshape(-1))
    n_sent = int(np.count_nonzero(words == SENTINEL_U32))
    n_negz = int(np.count_nonzero(h == 0x8000))
    if n_sent:
        problems.append(f"{n_sent} sentinel words in the collect output")
    if n_negz:
        problems.append(f"{n_negz} negative-zero halves in the collect output")
    return problems


def check_idle_slots(slot_words: np.ndarray) -> list[str]:
    """Problems in a whole mailbox after a collect: any non-sentinel word left
    behind (all_gather page, module docstring, step 2: no call leaves a word
    for a later one)."""
    w = np.asarray(slot_words, dtype=np.uint32)
    left = int(np.count_nonzero(w != SENTINEL_U32))
    return [f"{left} words left behind in the mailbox"] if left else []


class EpochModel:
    """The split-K hand-off tag: 1 after initialisation, +1 per GEMM call that
    exchanges partials, never 0."""

    def __init__(self) -> None:
        self.epoch = 1

    def advance(self) -> None:
        self.epoch = (self.epoch + 1) & 0xFFFFFFFF
        if self.epoch == 0:
            self.epoch = 1
