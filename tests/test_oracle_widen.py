"""Pins for the oracle's exact widening of stored values to float64 (no GPU).

Every oracle result starts with ``oracle.attention.widen``: bfloat16 data is
carried as uint16 bit patterns, float32 data as float32.  The torch SDPA and
closed-form pins of the attention go through the same function, so it needs
a check of its own that does not:

* the bfloat16 format's own definition, decoded field by field in plain
  Python (1 sign bit, 8 exponent bits with bias 127, 7 fraction bits;
  exponent 0 subnormal, exponent 255 infinity or NaN) for all 65,536 bit
  patterns;
* torch's own bfloat16 -> float64 conversion over the same patterns;
* values decoded by hand;
* float32 bit patterns (normal, subnormal, infinite, NaN) against the
  struct module's decoding of IEEE binary32;
* planted mistakes (bits read as float16, a shift of 15 or 8 bits, the sign
  bit dropped, a truncated fraction) that the definition check must catch.
"""
import math
import struct

import numpy as np
import pytest
import torch

import oracle.attention as oa

ALL_BF16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def bf16_by_definition(bits: int) -> float:
    """Value of a bfloat16 bit pattern from the format's fields."""
    sign = -1.0 if bits >> 15 else 1.0
    exp = (bits >> 7) & 0xFF
    frac = bits & 0x7F
    if exp == 0xFF:
        return sign * math.inf if frac == 0 else math.nan
    if exp == 0:  # zero and subnormals: frac * 2^(1 - 127 - 7)
        return sign * math.ldexp(frac, -133)
    return sign * math.ldexp(128 + frac, exp - 127 - 7)


def definition_mismatches(widen_fn) -> list:
    """Bit patterns whose widened value differs from the definition (NaN
    must stay NaN; zeros must keep their sign)."""
    got = np.asarray(widen_fn(ALL_BF16))
    bad = []
    if got.shape != ALL_BF16.shape or got.dtype != np.float64:
        return ["shape or dtype"]
    for b in range(1 << 16):
        want, have = bf16_by_definition(b), float(got[b])
        if math.isnan(want):
            if not math.isnan(have):
                bad.append(b)
        elif have != want or math.copysign(1.0, have) != math.copysign(1.0, want):
            bad.append(b)
    return bad


def test_every_bf16_pattern_matches_the_format_definition():
    assert definition_mismatches(oa.widen) == []


def test_every_bf16_pattern_matches_torch():
    ref = torch.from_numpy(ALL_BF16.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = oa.widen(ALL_BF16)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    # bitwise on the float64 values: equal magnitudes and signs of zero
    assert np.array_equal(got[~nan].view(np.int64), ref[~nan].view(np.int64))


@pytest.mark.parametrize("bits,value", [
    (0x3F80, 1.0),
    (0xC000, -2.0),
    (0x0001, 2.0 ** -133),           # smallest subnormal
    (0x0080, 2.0 ** -126),           # smallest normal
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),  # largest finite
    (0xFF80, -math.inf),
    (0x7F80, math.inf),
    (0x3EAB, 0.333984375),           # 1/3 rounded to 8 significant bits
    (0x4049, 3.140625),              # pi rounded to 8 significant bits
])
def test_hand_decoded_values(bits, value):
    assert float(oa.widen(np.array([bits], dtype=np.uint16))[0]) == value


def test_negative_zero_and_nan_payloads():
    got = oa.widen(np.array([0x8000, 0x7FC0, 0xFFC1, 0x7F81], dtype=np.uint16))
    assert got[0] == 0.0 and math.copysign(1.0, got[0]) == -1.0
    assert np.isnan(got[1:]).all()


def test_float32_patterns_widen_exactly():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 1 << 32, size=20000, dtype=np.uint64).astype(np.uint32)
    special = np.array([0, 1, 0x007FFFFF, 0x00800000, 0x7F7FFFFF, 0x7F800000, 0xFF800000, 0x7FC00000,
                        0x80000000, 0x3F800000, 0xBF800000], dtype=np.uint32)
    bits = np.concatenate([bits, special])
    got = oa.widen(bits.view(np.float32))
    for b, g in zip(bits.tolist(), got.tolist()):
        want = struct.unpack("<f", struct.pack("<I", b))[0]
        if math.isnan(want):
            assert math.isnan(g), hex(b)
        else:
            assert g == want and math.copysign(1.0, g) == math.copysign(1.0, want), hex(b)


def test_widen_rejects_other_types():
    with pytest.raises(TypeError):
        oa.widen(np.zeros(3, dtype=np.int16))


# --- planted mistakes: each must be caught by the definition check ---------

def _as_fp16(x):
    return np.asarray(x).view(np.float16).astype(np.float64)


def _shift(n):
    return lambda x: (np.asarray(x).astype(np.uint32) << np.uint32(n)).view(np.float32).astype(np.float64)


def _no_sign(x):
    return oa.widen(np.asarray(x) & np.uint16(0x7FFF))


def _short_fraction(x):
    return oa.widen(np.asarray(x) & np.uint16(0xFFFE))


@pytest.mark.parametrize("mutant", [_as_fp16, _shift(15), _shift(8), _no_sign, _short_fraction],
                         ids=["read-as-fp16", "shift-15", "shift-8", "sign-dropped", "fraction-truncated"])
def test_planted_widening_mistakes_are_caught(mutant):
    assert len(definition_mismatches(mutant)) > 0
