"""Pins of the word all-gather in the oracle (MailboxModel.publish_words,
all_gather, sanitize_words) against what the all_gather page fixes and plain
invariants."""

import json
import os

import numpy as np
import pytest

from oracle import mailbox

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")


def test_sentinel_word_arrives_as_zero_and_nothing_else_changes():
    """all_gather page, LamportAllGather.__call__ docstring: words equal to
    0x80000000 arrive as 0 (FP32 negative zero becomes positive zero). Words
    that merely contain the pattern in one half, or differ by one bit, are
    payload and arrive unchanged."""
    with open(GOLDEN) as f:
        sentinel = int(json.load(f)["sentinel_u32"]["hex"], 16)
    words = np.array([sentinel, sentinel + 1, sentinel - 1, 0x00008000, 0x80008000,
                      0xFFFFFFFF, 0, 0x3F800000], dtype=np.uint32)
    mb = mailbox.MailboxModel(1, 32)
    got = mb.all_gather(0, words)
    assert list(got[0]) == [0, sentinel + 1, sentinel - 1, 0x00008000, 0x80008000,
                            0xFFFFFFFF, 0, 0x3F800000]
    assert mb.idle() and mb.next == 1


def test_rank_major_order_and_reset():
    """all_gather page, module docstring, step 2: each rank's pack goes to the
    output rank-major (a dim-0 gather), and every slot read is reset."""
    rng = np.random.default_rng(3)
    ranks, n = 4, 64
    payloads = rng.integers(0, 2**32, size=(ranks, n), dtype=np.uint64).astype(np.uint32)
    mb = mailbox.MailboxModel(ranks, 4 * n)
    for r in range(1, ranks):
        mb.publish_words(r, payloads[r])
    got = mb.all_gather(0, payloads[0])
    assert np.array_equal(got, mailbox.sanitize_words(payloads))
    assert mb.idle()


def test_missing_peer_would_spin():
    mb = mailbox.MailboxModel(2, 64)
    with pytest.raises(mailbox.WouldSpin):
        mb.all_gather(0, np.arange(16, dtype=np.uint32))


def test_generations_cycle_and_sizes_alternate():
    """Alternating sizes through one mailbox never leave a word behind
    (all_gather page, module docstring, step 2: whatever the sizes)."""
    mb = mailbox.MailboxModel(2, 256)
    for i in range(9):
        n = 64 if i % 2 else 8
        w = np.full(n, 0x80000000 if i % 3 == 0 else i, dtype=np.uint32)
        mb.publish_words(1, w + 1)
        got = mb.all_gather(0, w)
        assert np.array_equal(got[0], mailbox.sanitize_words(w))
        assert np.array_equal(got[1], mailbox.sanitize_words(w + 1))
        assert mb.idle() and mb.next == (i + 1) % 3
