"""Pins for the oracle's Lamport mailbox model and its checker (CPU only).

Includes the page constants under tests/golden/, the packing closed form, the
hand-worked pack words, the alternating-size invariant and a mutation test: the
own-slot copy that lands after the reset (the failure the all_gather page's
module docstring describes for another gather) must be caught by the checker.
"""

import json
import os

import numpy as np
import pytest

from oracle import codecs, gemm, mailbox
from workloads import generate

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_page_constants():
    with open(os.path.join(GOLDEN, "page_constants.json")) as f:
        g = json.load(f)
    assert codecs.SENTINEL_U32 == g["sentinel_u32"]["value"]
    assert np.int32(g["sentinel_fill_int32"]["value"]).view(np.uint32) == codecs.SENTINEL_U32
    assert np.float32(-0.0).view(np.uint32) == codecs.SENTINEL_U32
    assert mailbox.GENERATIONS == g["generations"]["value"]
    assert mailbox.PACK_BYTES == g["pack_bytes"]["value"]
    assert gemm.MAX_ROWS == g["max_activation_rows"]["value"]
    assert gemm.BLOCK == g["scale_block"]["value"]
    assert mailbox.PACK_BYTES // 2 == g["columns_per_pack"]["value"]


def test_pack_words_closed_form():
    rng = np.random.default_rng(0)
    halves = rng.integers(0, 65536, size=(3, 64)).astype(np.uint16)
    words = mailbox.halves_to_words(halves)
    # Little-endian bytes of the [m, N] BF16 array are the mailbox bytes.
    assert words.tobytes() == halves.astype("<u2").tobytes()
    assert np.array_equal(mailbox.words_to_halves(words), halves.reshape(-1))


def test_hand_worked_pack_words():
    with open(os.path.join(GOLDEN, "hand_worked_pack.json")) as f:
        g = json.load(f)
    bits = np.array([[int(v, 16) for v in row] for row in g["published_bf16"]],
                    dtype=np.uint16)
    words = mailbox.halves_to_words(bits).reshape(g["m"], -1)
    expect = np.array([[int(v, 16) for v in row] for row in g["published_words"]],
                      dtype=np.uint32)
    assert np.array_equal(words, expect)


def test_publish_collect_roundtrip_rank_major():
    mb = mailbox.MailboxModel(ranks=4, capacity_bytes=256)
    rng = np.random.default_rng(1)
    payloads = [rng.integers(0, 65536, size=(2, 16)).astype(np.uint16) for _ in range(4)]
    payloads[2][0, 3] = 0x8000
    for r in range(4):
        mb.publish(r, payloads[r])
    assert mb.active == 0
    out = mb.collect(64).reshape(8, 16)
    for r in range(4):
        assert np.array_equal(out[2 * r : 2 * r + 2], codecs.clear_negative_zero(payloads[r]))
    assert mb.idle() and mb.next == 1
    assert not mailbox.check_collected(out)


def test_generation_cycles_mod_three():
    mb = mailbox.MailboxModel(ranks=1, capacity_bytes=64)
    for call in range(7):
        assert mb.next == call % 3
        mb.publish(0, np.ones((1, 8), dtype=np.uint16))
        mb.collect(16)
    assert mb.next == 7 % 3


def test_missing_publish_would_spin():
    mb = mailbox.MailboxModel(ranks=2, capacity_bytes=64)
    mb.publish(0, np.ones((1, 8), dtype=np.uint16))
    with pytest.raises(mailbox.WouldSpin):
        mb.collect(16)


def test_sentinel_word_never_published():
    mb = mailbox.MailboxModel(ranks=1, capacity_bytes=64)
    bits = np.array([[0x0000, 0x8000, 0x8000, 0x8000, 0, 0, 1, 2]], dtype=np.uint16)
    mb.publish(0, bits)
    assert not np.any(mb.slots[0, 0, :4] == codecs.SENTINEL_U32)
    out = mb.collect(16)
    assert not mailbox.check_collected(out)


def test_capacity_rules():
    assert mailbox.accepts(16, 16) and not mailbox.accepts(0, 16)
    assert not mailbox.accepts(24, 64) and not mailbox.accepts(80, 64)
    with pytest.raises(ValueError):
        mailbox.MailboxModel(ranks=1, capacity_bytes=24)
    mb = mailbox.MailboxModel(ranks=1, capacity_bytes=32)
    with pytest.raises(ValueError):
        mb.publish(0, np.zeros((3, 8), dtype=np.uint16))


def test_alternating_sizes_leave_nothing_behind():
    mb = mailbox.MailboxModel(ranks=4, capacity_bytes=512)
    rng = np.random.default_rng(2)
    for call in range(12):
        m, n = ((1, 128), (8, 32))[call % 2]
        for r in range(4):
            mb.publish(r, rng.integers(0, 65536, size=(m, n)).astype(np.uint16))
        out = mb.collect(2 * m * n)
        assert not mailbox.check_collected(out)
        assert not mailbox.check_idle_slots(mb.slots)


class _OwnCopyLandsLate(mailbox.MailboxModel):
    """Planted mistake: the caller takes its own slot from registers, and its
    own store lands only after the collect has reset the slot."""

    def publish(self, rank, bf16_bits):
        self._late = (rank, self.next, np.asarray(bf16_bits, dtype=np.uint16))
        bits = codecs.clear_negative_zero(self._late[2])
        self._own = mailbox.halves_to_words(bits)

    def collect(self, nbytes):
        g = self.next
        out = np.stack([mailbox.words_to_halves(self._own)])
        self.slots[g, :, : nbytes // 4] = codecs.SENTINEL_U32
        rank, gen, bits = self._late
        self.slots[gen, rank, : bits.size // 2] = mailbox.halves_to_words(
            codecs.clear_negative_zero(bits))
        self.next = (g + 1) % mailbox.GENERATIONS
        return out


def test_checker_catches_late_own_copy():
    mb = _OwnCopyLandsLate(ranks=1, capacity_bytes=256)
    mb.publish(0, np.full((1, 64), 0x3F80, dtype=np.uint16))
    mb.collect(128)
    assert mailbox.check_idle_slots(mb.slots)  # a word was left behind
    # Three calls later the generation comes round; a smaller call of another
    # size then finds the stale word where it expects the sentinel.
    good = mailbox.MailboxModel(ranks=1, capacity_bytes=256)
    good.slots = mb.slots.copy()
    good.next = 0
    assert not good.idle()


def test_epoch_model_skips_zero():
    e = mailbox.EpochModel()
    assert e.epoch == 1
    e.epoch = 0xFFFFFFFF
    e.advance()
    assert e.epoch == 1


def test_model_matches_oracle_gemm_bits():
    p = generate.random_problem(21, 2, 64, 128, dist="stress")
    bits, _, _ = gemm.gemm_publish_bits(p.w, p.ws, p.x, p.xs)
    mb = mailbox.MailboxModel(ranks=1, capacity_bytes=p.out_bytes)
    mb.publish(0, bits)
    out = mb.collect(p.out_bytes).reshape(p.m, p.n)
    assert np.array_equal(out, bits)
    assert mb.idle()
