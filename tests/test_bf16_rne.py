"""Pins of the oracle's bf16 round-to-nearest-even.

- against exact rational rounding (Python fractions) on random float64 values;
- against torch's fp32 -> bf16 conversion, a library routine, over every fp32 bit pattern;
- explicit ties, subnormals and overflow.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

MAX_BF16 = (2 - 2 ** -7) * 2.0 ** 127


def bf16_grid_neighbours(x: float):
    """The two bf16 values around x, by enumeration of the bf16 grid near x."""
    if x == 0:
        return 0.0, 0.0
    e = math.floor(math.log2(abs(x)))
    q = 2.0 ** (max(e, -126) - 7)          # spacing of bf16 values in this binade
    lo = math.floor(Fraction(x) / Fraction(q)) * q
    return lo, lo + q


def exact_rne(x: float) -> float:
    lo, hi = bf16_grid_neighbours(x)
    dlo, dhi = Fraction(x) - Fraction(lo), Fraction(hi) - Fraction(x)
    if dlo < dhi:
        r = lo
    elif dhi < dlo:
        r = hi
    else:   # tie: the one whose last kept mantissa bit is 0
        q = hi - lo
        r = lo if (Fraction(lo) / Fraction(q)) % 2 == 0 else hi
    if abs(r) > MAX_BF16:
        return math.copysign(math.inf, x)
    return r


def test_random_float64_against_exact_rational(orc):
    rng = np.random.default_rng(11)
    xs = np.concatenate([
        rng.standard_normal(3000) * 0.1,
        rng.standard_normal(1000) * 1e30,
        rng.standard_normal(1000) * 1e-38,      # around the bf16 subnormal range
        rng.standard_normal(500) * 1e-40,
    ])
    for x in xs:
        assert orc.round_bf16(float(x)) == exact_rne(float(x)), x


def test_ties_subnormals_overflow(orc):
    one = 1.0
    assert orc.round_bf16(one + 2 ** -8) == 1.0                    # tie -> even (down)
    assert orc.round_bf16(one + 3 * 2 ** -8) == one + 2 ** -6       # tie -> even (up)
    assert orc.round_bf16(one + 2 ** -8 + 2 ** -40) == one + 2 ** -7  # just above the tie
    assert orc.round_bf16(-(one + 2 ** -8)) == -1.0
    assert orc.round_bf16(2.0 ** -133) == 2.0 ** -133               # smallest subnormal
    assert orc.round_bf16(2.0 ** -134) == 0.0                       # tie to even (zero)
    assert orc.round_bf16(1.5 * 2.0 ** -134) == 2.0 ** -133
    assert orc.round_bf16(3 * 2.0 ** -134) == 2 * 2.0 ** -133       # tie -> even
    assert orc.round_bf16(MAX_BF16) == MAX_BF16
    assert orc.round_bf16(MAX_BF16 + 2.0 ** 119) == math.inf        # tie between max and 2^128 -> inf
    assert orc.round_bf16(MAX_BF16 + 2.0 ** 118) == MAX_BF16
    assert orc.round_bf16(-1e39) == -math.inf
    assert math.isnan(orc.round_bf16(math.nan))
    assert orc.round_bf16(math.inf) == math.inf
    assert math.copysign(1.0, orc.round_bf16(-0.0)) == -1.0


@pytest.mark.slow
def test_all_fp32_patterns_against_torch(orc):
    """Every one of the 2^32 fp32 bit patterns: the oracle's RNE equals torch's fp32 -> bf16."""
    chunk = 1 << 26
    mism = 0
    for start in range(0, 1 << 32, chunk):
        bits = np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32)
        ours = orc.round_bf16_f32bits(bits)
        ref = torch.from_numpy(bits.view(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        nan = ((bits & 0x7F800000) == 0x7F800000) & ((bits & 0x007FFFFF) != 0)
        ours_nan = ((ours & 0x7F80) == 0x7F80) & ((ours & 0x007F) != 0)
        ref_nan = ((ref & 0x7F80) == 0x7F80) & ((ref & 0x007F) != 0)
        assert np.array_equal(ours_nan, nan) and np.array_equal(ref_nan, nan)
        mism += int(np.count_nonzero((ours != ref) & ~nan))
    assert mism == 0
