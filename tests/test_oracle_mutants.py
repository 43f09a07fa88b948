"""Planted mistakes in the oracle (CPU only): each one must fail a pin.

Every mutant below is a copy of one oracle function, table or constant with a
single plausible mistake in it: a wrong bias, a dropped sign or term, a wrong
block index, a transposed result, another rounding rule, a missed reset or
generation step. The test swaps the mutant in, runs the pins of the oracle
(every test function of the ``test_oracle_*`` modules, each parametrized case
included) and requires that at least one of them fails. The mutants live here
only, never in ``oracle/``; without them every pin passes (the rest of the
suite). A mutant that no pin catches would mark a hole in the pins.
"""

from __future__ import annotations

import importlib
import itertools
import math

import numpy as np
import pytest

from oracle import codecs, gemm, mailbox, quant, tolerance

PIN_MODULES = (
    "test_oracle_codecs",
    "test_oracle_gemm",
    "test_oracle_tolerance",
    "test_oracle_quant",
    "test_oracle_quant_bf16",
    "test_oracle_mailbox",
    "test_oracle_allgather",
    "test_oracle_allreduce",
)


def _cases(fn):
    """Keyword-argument dicts of a test function, one per parametrized case."""
    marks = [mk for mk in getattr(fn, "pytestmark", []) if mk.name == "parametrize"]
    per_mark = []
    for mk in marks:
        names = mk.args[0]
        names = [s.strip() for s in names.split(",")] if isinstance(names, str) else list(names)
        rows = []
        for v in mk.args[1]:
            if hasattr(v, "values") and hasattr(v, "marks"):  # pytest.param
                v = v.values
            if len(names) == 1 and not (isinstance(v, tuple) and len(v) == 1):
                v = (v,)
            rows.append(dict(zip(names, v)))
        per_mark.append(rows)
    for combo in itertools.product(*per_mark):
        kw = {}
        for part in combo:
            kw.update(part)
        yield kw


def _pins():
    """(name, callable) for every pin case, in module order."""
    out = []
    for modname in PIN_MODULES:
        mod = importlib.import_module(modname)
        for name in sorted(dir(mod)):
            fn = getattr(mod, name)
            if not (name.startswith("test_") and callable(fn)):
                continue
            for kw in _cases(fn):
                label = f"{modname}::{name}" + (f"[{kw}]" if kw else "")
                out.append((label, (lambda f=fn, k=kw: f(**k))))
    return out


def _first_failing_pin():
    for label, call in _pins():
        try:
            call()
        except (Exception, pytest.fail.Exception):
            return label
    return None


# ---------------------------------------------------------------------------
# Mutant builders. Each takes a MonkeyPatch and swaps one mistake in, in every
# place the oracle binds the name (tables and imports built from it included).
# ---------------------------------------------------------------------------

def _e4m3_value(bias=7, signed=True, subnormals=True, nan_whole_top=False):
    def value(code):
        sign = -1.0 if (code >> 7) and signed else 1.0
        exponent = (code >> 3) & 0xF
        mantissa = code & 0x7
        if exponent == 0xF and (mantissa == 0x7 or nan_whole_top):
            return math.nan
        if exponent == 0 and subnormals:
            return sign * mantissa * 2.0 ** (-bias - 2)
        return sign * (1.0 + mantissa / 8.0) * 2.0 ** (exponent - bias)
    return value


def _swap_e4m3(value):
    def apply(mp):
        mp.setattr(codecs, "e4m3_value", value)
        mp.setattr(quant, "e4m3_value", value)
        mp.setattr(codecs, "E4M3_TABLE", np.array([value(c) for c in range(256)]))
        code_of = {}
        for c in range(256):
            v = value(c)
            if not math.isnan(v):
                code_of[(v, math.copysign(1.0, v))] = c
        mp.setattr(quant, "_CODE_OF", code_of)
    return apply


def _swap_e8m0(value):
    def apply(mp):
        mp.setattr(codecs, "e8m0_value", value)
        mp.setattr(codecs, "E8M0_TABLE", np.array([value(c) for c in range(256)]))
    return apply


def _swap(obj, name, make):
    """Replace obj.name by make(original)."""
    def apply(mp):
        mp.setattr(obj, name, make(getattr(obj, name)))
    return apply


def _swap_everywhere(name, make):
    """Replace a codecs function and every module's imported copy of it."""
    def apply(mp):
        new = make(getattr(codecs, name))
        for mod in (codecs, gemm, mailbox, quant, tolerance):
            if hasattr(mod, name):
                mp.setattr(mod, name, new)
    return apply


def _round_steps(step_rule):
    """bf16_round_value with another rule for the number of BF16 steps."""
    def make(_orig):
        def round_value(v):
            v = np.asarray(v, dtype=np.float64)
            q = codecs.bf16_quantum(v)
            r = step_rule(v / q) * q
            r = np.where(np.abs(v) >= codecs.BF16_OVERFLOW, np.copysign(np.inf, v), r)
            return np.copysign(r, v)
        return round_value
    return make


def _dequantize_with(factor_rule, scaled=True):
    def make(_orig):
        def dequantize(codes, scales):
            codes = np.asarray(codes, dtype=np.uint8)
            scales = np.asarray(scales, dtype=np.uint8)
            values = codecs.decode_e4m3(codes)
            return values * factor_rule(codecs.decode_e8m0(scales)) if scaled else values
        return dequantize
    return make


def _gemm_with(contract):
    def make(_orig):
        def gemm_f64(w, ws, x, xs):
            gemm.check_shapes(w, ws, x, xs)
            return contract(gemm.dequantize(w, ws), gemm.dequantize(x, xs))
        return gemm_f64
    return make


def _collect_with(next_gen=lambda g: (g + 1) % 3, reset=True, order=lambda r: r,
                  generation=lambda mb: mb.next):
    def make(_orig):
        def collect(self, nbytes):
            if not mailbox.accepts(nbytes, self.capacity_bytes):
                raise ValueError("payload does not fit")
            g = generation(self)
            words = self.slots[g, :, : nbytes // 4]
            if np.any(words == mailbox.SENTINEL_U32):
                raise mailbox.WouldSpin("sentinel")
            out = np.stack([mailbox.words_to_halves(words[r]) for r in order(range(self.ranks))])
            if reset:
                self.slots[g, :, : nbytes // 4] = mailbox.SENTINEL_U32
            self.next = next_gen(g)
            self.collects += 1
            return out
        return collect
    return make


def _publish_unsanitized(_orig):
    def publish(self, rank, bf16_bits):
        bits = np.asarray(bf16_bits, dtype=np.uint16)
        g = self.next
        self.slots[g, rank, : bits.size // 2] = mailbox.halves_to_words(bits)
        self.active = g
    return publish


def _swap_packing(mp):
    """The odd column in the low half of each word (and the matching unpack)."""
    def to_words(halves):
        h = np.asarray(halves, dtype=np.uint16).reshape(-1)
        return (h[1::2].astype(np.uint32) | (h[0::2].astype(np.uint32) << np.uint32(16)))

    def to_halves(words):
        w = np.asarray(words, dtype=np.uint32).reshape(-1)
        out = np.empty(w.size * 2, dtype=np.uint16)
        out[1::2] = (w & np.uint32(0xFFFF)).astype(np.uint16)
        out[0::2] = (w >> np.uint32(16)).astype(np.uint16)
        return out

    mp.setattr(mailbox, "halves_to_words", to_words)
    mp.setattr(mailbox, "words_to_halves", to_halves)


def _allreduce_with(order=lambda r: r, fp64=False):
    def make(_orig):
        def allreduce(halves):
            h = np.asarray(halves, dtype=np.uint16)
            vals = codecs.bf16_to_f64(h)
            if fp64:
                return codecs.bf16_rne_bits(vals.sum(axis=0))
            ranks = list(order(range(h.shape[0])))
            acc = vals[ranks[0]].astype(np.float32)
            for r in ranks[1:]:
                acc = np.add(acc, vals[r].astype(np.float32), dtype=np.float32)
            return codecs.bf16_rne_bits(acc.astype(np.float64))
        return allreduce
    return make


def _epoch_keeps_zero(_orig):
    def advance(self):
        self.epoch = (self.epoch + 1) & 0xFFFFFFFF
    return advance


def _exponent_with(rule):
    def make(_orig):
        def block_exponent(amax):
            if amax == 0.0:
                return -127
            return rule(amax)
        return block_exponent
    return make


def _e4m3_round_ties_away(orig):
    def e4m3_round(y):
        a = abs(y)
        quantum = 2.0**-9 if a < 2.0**-6 else math.ldexp(1.0, math.frexp(a)[1] - 4)
        n = math.floor(a / quantum + 0.5)
        r = math.copysign(n * quantum, y)
        return quant._CODE_OF[(r, math.copysign(1.0, r))]
    return e4m3_round


def _quantize_bf16_nonfinite(scale_byte, keep_sign):
    def make(orig):
        def quantize_bf16(bits):
            bits = np.asarray(bits, dtype=np.uint16)
            codes, scales = orig(bits)
            bad = scales == quant.E8M0_NAN
            scales = np.where(bad, np.uint8(scale_byte), scales).astype(np.uint8)
            if not keep_sign:
                rows = np.repeat(bad, quant.BLOCK, axis=1)
                codes = np.where(rows, np.uint8(quant.E4M3_NAN), codes).astype(np.uint8)
            return codes, scales
        return quantize_bf16
    return make


MUTANTS = {
    # e4m3fn / E8M0 decoding
    "e4m3 exponent bias 8": _swap_e4m3(_e4m3_value(bias=8)),
    "e4m3 sign bit ignored": _swap_e4m3(_e4m3_value(signed=False)),
    "e4m3 exponent field 0 decoded as normal": _swap_e4m3(_e4m3_value(subnormals=False)),
    "e4m3 whole top binade NaN (IEEE-style e4m3)": _swap_e4m3(_e4m3_value(nan_whole_top=True)),
    "E8M0 bias 128": _swap_e8m0(lambda c: math.nan if c == 255 else math.ldexp(1.0, c - 128)),
    "E8M0 255 read as 2^128": _swap_e8m0(lambda c: math.ldexp(1.0, c - 127)),
    # BF16 rounding and the negative-zero clear
    "BF16 truncation": _swap(codecs, "bf16_round_value", _round_steps(np.trunc)),
    "BF16 ties away from zero": _swap(
        codecs, "bf16_round_value",
        _round_steps(lambda s: np.copysign(np.floor(np.abs(s) + 0.5), s))),
    "BF16 rounded through FP32 first": _swap(
        codecs, "bf16_round_value",
        lambda orig: lambda v: orig(np.asarray(v, dtype=np.float64).astype(np.float32)
                                    .astype(np.float64))),
    "BF16 subnormals flushed to zero": _swap(
        codecs, "bf16_round_value",
        lambda orig: lambda v: np.where(np.abs(np.asarray(v, dtype=np.float64)) < 2.0**-126,
                                        np.copysign(0.0, v), orig(v))),
    "BF16 sign of a rounded-away zero dropped": _swap(
        codecs, "bf16_round_value", lambda orig: lambda v: orig(v) + 0.0),
    "BF16 eight mantissa bits": _swap(codecs, "BF16_MANT_BITS", lambda _o: 8),
    "BF16 smallest normal exponent -125": _swap(codecs, "BF16_MIN_EXP", lambda _o: -125),
    "negative zero not cleared": _swap_everywhere(
        "clear_negative_zero", lambda _o: lambda b: np.asarray(b, dtype=np.uint16)),
    "sign cleared on every subnormal": _swap_everywhere(
        "clear_negative_zero",
        lambda _o: lambda b: np.where((np.asarray(b) & 0x7F80) == 0, np.asarray(b) & 0x7FFF,
                                      b).astype(np.uint16)),
    # the GEMM
    "scale index k mod blocks (tile, not repeat)": _swap(
        gemm, "dequantize", _dequantize_with(lambda f: np.tile(f, (1, 32)))),
    "scale block boundary off by one": _swap(
        gemm, "dequantize",
        _dequantize_with(lambda f: np.roll(np.repeat(f, 32, axis=1), 1, axis=1))),
    "scales dropped": _swap(gemm, "dequantize", _dequantize_with(None, scaled=False)),
    "last K block dropped": _swap(gemm, "gemm_f64", _gemm_with(
        lambda wd, xd: (xd[:, :-32] @ wd[:, :-32].T, np.abs(xd[:, :-32]) @ np.abs(wd[:, :-32]).T))),
    "result transposed ([N, m])": _swap(gemm, "gemm_f64", _gemm_with(
        lambda wd, xd: ((xd @ wd.T).T, (np.abs(xd) @ np.abs(wd).T).T))),
    "FP32 accumulation": _swap(gemm, "gemm_f64", _gemm_with(
        lambda wd, xd: ((xd.astype(np.float32) @ wd.T.astype(np.float32)).astype(np.float64),
                        np.abs(xd) @ np.abs(wd).T))),
    "magnitude sum taken as |C|": _swap(gemm, "gemm_f64", _gemm_with(
        lambda wd, xd: (xd @ wd.T, np.abs(xd @ wd.T)))),
    "published bits rounded through FP32": _swap(
        gemm, "published_bits",
        lambda _o: lambda c: codecs.clear_negative_zero(codecs.bf16_rne_bits(
            np.asarray(c, dtype=np.float64).astype(np.float32).astype(np.float64)))),
    "zero cleared before rounding, not after": _swap(
        gemm, "published_bits",
        lambda _o: lambda c: codecs.bf16_rne_bits(np.where(np.asarray(c) == 0, 0.0, c))),
    # the mailbox
    "collect leaves the slot": _swap(mailbox.MailboxModel, "collect", _collect_with(reset=False)),
    "generations mod 2": _swap(mailbox.MailboxModel, "collect",
                               _collect_with(next_gen=lambda g: (g + 1) % 2)),
    "collect never advances": _swap(mailbox.MailboxModel, "collect",
                                    _collect_with(next_gen=lambda g: g)),
    "collect output rank order reversed": _swap(
        mailbox.MailboxModel, "collect", _collect_with(order=lambda rs: list(rs)[::-1])),
    "publish without the negative-zero clear": _swap(
        mailbox.MailboxModel, "publish", _publish_unsanitized),
    "odd column in the low half of a word": _swap_packing,
    "sentinel words not replaced": _swap(
        mailbox, "sanitize_words", lambda _o: lambda w: np.asarray(w, dtype=np.uint32)),
    "all-reduce summed in float64": _swap(mailbox, "allreduce_bf16", _allreduce_with(fp64=True)),
    "all-reduce in descending rank order": _swap(
        mailbox, "allreduce_bf16", _allreduce_with(order=lambda rs: list(rs)[::-1])),
    "epoch wraps to 0": _swap(mailbox.EpochModel, "advance", _epoch_keeps_zero),
    # the quantizer
    "block exponent floor(log2(amax/448))": _swap(quant, "block_exponent", _exponent_with(
        lambda a: max(-127, min(127, math.floor(math.log2(a / 448.0)))))),
    "block exponent from the next power of two of amax": _swap(
        quant, "block_exponent", _exponent_with(
            lambda a: max(-127, min(127, math.ceil(math.log2(a)) - 8)))),
    "e4m3 ties away from zero": _swap(quant, "e4m3_round", _e4m3_round_ties_away),
    "non-finite block scale 0 instead of 0xFF": _swap(
        quant, "quantize_bf16", _quantize_bf16_nonfinite(0x00, keep_sign=True)),
    "NaN codes lose the element's sign": _swap(
        quant, "quantize_bf16", _quantize_bf16_nonfinite(quant.E8M0_NAN, keep_sign=False)),
    # the acceptance bound
    "bound without the ulp term": _swap(
        tolerance, "bound",
        lambda _o: lambda exact, abs_sum: tolerance.REL_ABS_SUM * np.asarray(abs_sum,
                                                                              dtype=np.float64)),
    "bound of half an ulp": _swap(
        tolerance, "bound",
        lambda o: lambda exact, abs_sum: o(exact, abs_sum) - 0.5 * codecs.bf16_quantum(exact)),
    "bound with 1e-5 of the magnitude sum": _swap(tolerance, "REL_ABS_SUM", lambda _o: 1e-5),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name):
    with pytest.MonkeyPatch.context() as mp:
        MUTANTS[name](mp)
        caught_by = _first_failing_pin()
    assert caught_by is not None, f"no pin catches the mutant: {name}"


def test_every_pin_passes_without_a_mutant():
    """The check above means something only if the pins pass on the oracle."""
    assert _first_failing_pin() is None
