"""Pins of the oracle's 16-bit conversions against library routines (CPU only).

Widening is checked on all 65,536 patterns. Narrowing (round to nearest, ties
to even) is checked against numpy's binary16 conversion and torch's bfloat16
conversion on every fp32 sign/exponent/high-fraction pattern (all 2^16 upper
halves) combined with the low halves that decide rounding (round bit, sticky
bits, and the bits in between), plus 2^24 random patterns. Setting
ZS_EXHAUSTIVE_CASTS=1 widens the sweep to all 2^32 patterns (about ten
minutes). NaNs are compared by class: payload bits are not part of the
contract.
"""
import os

import numpy as np
import pytest

import oracle

CHUNK = 1 << 24
EXHAUSTIVE = os.environ.get("ZS_EXHAUSTIVE_CASTS") == "1"

# Low 16 bits of the fp32 pattern: every combination of bits 12..15 (the
# binary16 round bit and the three fraction bits above it) with sticky
# patterns below, plus the bfloat16 tie/sticky patterns around bit 15.
_LOW = sorted({(hi << 12) | lo for hi in range(16) for lo in (0x000, 0x001, 0x7FF, 0x800, 0xFFF)}
              | {0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000})


def _is_nan16(bits, dtype):
    bits = bits.astype(np.uint32)
    if dtype == "bf16":
        return ((bits & 0x7F80) == 0x7F80) & ((bits & 0x007F) != 0)
    return ((bits & 0x7C00) == 0x7C00) & ((bits & 0x03FF) != 0)


def test_fp16_widening_exhaustive():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.half_to_float(bits, "fp16")
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_widening_exhaustive():
    torch = pytest.importorskip("torch")
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.half_to_float(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _patterns():
    if EXHAUSTIVE:
        for start in range(0, 1 << 32, CHUNK):
            yield np.arange(start, start + CHUNK, dtype=np.uint64).astype(np.uint32)
        return
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    yield (hi[:, None] | np.array(_LOW, np.uint32)[None, :]).ravel()
    yield np.random.default_rng(0).integers(0, 1 << 32, CHUNK, dtype=np.uint64).astype(np.uint32)


def _narrow_check(dtype, ref_fn):
    for u in _patterns():
        start = int(u[0])
        x = u.view(np.float32)
        ours = oracle.float_to_half(x, dtype)
        ref = ref_fn(x)
        xnan = np.isnan(x)
        assert np.array_equal(_is_nan16(ours, dtype), xnan), hex(start)
        ok = ours[~xnan] == ref[~xnan]
        if not ok.all():
            bad = np.flatnonzero(~ok)[0]
            raise AssertionError(f"{dtype}: x bits {u[~xnan][bad]:#010x} -> ours "
                                 f"{ours[~xnan][bad]:#06x} ref {ref[~xnan][bad]:#06x}")


def test_fp16_narrowing():
    with np.errstate(over="ignore"):
        _narrow_check("fp16", lambda x: x.astype(np.float16).view(np.uint16))


def test_bf16_narrowing():
    torch = pytest.importorskip("torch")
    _narrow_check("bf16", lambda x: torch.from_numpy(x).to(torch.bfloat16).view(torch.int16)
                  .numpy().view(np.uint16))


def test_narrowing_special_values():
    cases = [
        # (value, bf16 bits, fp16 bits)
        (0.0, 0x0000, 0x0000), (-0.0, 0x8000, 0x8000),
        (1.0, 0x3F80, 0x3C00), (65504.0, 0x4780, 0x7BFF),
        (65519.996, 0x4780, 0x7BFF),   # below the fp16 rounding midpoint 65520
        (65520.0, 0x4780, 0x7C00),     # tie between 65504 and 2^16 -> even = inf
        (2.0 ** -24, 0x3380, 0x0001),
        (2.0 ** -25, 0x3300, 0x0000),  # tie -> even (0)
        (1.5 * 2.0 ** -25, 0x3340, 0x0001),
        (float("inf"), 0x7F80, 0x7C00), (float("-inf"), 0xFF80, 0xFC00),
    ]
    for v, b, h in cases:
        x = np.array([v], np.float32)
        assert oracle.float_to_half(x, "bf16")[0] == b, v
        assert oracle.float_to_half(x, "fp16")[0] == h, v
