"""Pins for the oracle's fp16 rounding (IEEE 754 binary16, nearest-even).

The oracle rounds from the binary64 bit fields.  It is pinned against numpy's
float32->float16 and float64->float16 conversions (both round to nearest,
ties to even), exhaustively over every float32 bit pattern, plus hand-derived
special cases (ties, overflow threshold, subnormal boundary).
"""
import concurrent.futures as cf

import numpy as np
import pytest

import oracle as O

pytestmark = pytest.mark.filterwarnings("ignore:overflow encountered in cast")


def _block(start, n):
    bits = np.arange(start, start + n, dtype=np.uint64).astype(np.uint32)
    ours = O.f16_from_f32bits(bits)
    ref = bits.view(np.float32).astype(np.float16).view(np.uint16)
    nan_ours = (ours & 0x7C00) == 0x7C00
    nan_ours &= (ours & 0x03FF) != 0
    nan_ref = np.isnan(bits.view(np.float32))
    # NaNs are compared as a class (payloads are not part of the definition)
    bad = (ours != ref) & ~(nan_ours & nan_ref)
    bad |= nan_ours != nan_ref
    return int(np.count_nonzero(bad))


@pytest.mark.slow
def test_f32_to_f16_exhaustive():
    """Every one of the 2^32 float32 patterns rounds as numpy rounds it."""
    n = 1 << 25
    with cf.ThreadPoolExecutor(8) as ex:
        bad = sum(ex.map(lambda k: _block(k * n, n), range((1 << 32) // n)))
    assert bad == 0


def test_f32_to_f16_relevant_range():
    """All float32 in the binades that can reach fp16 (|x| in [2^-26, 2^17))."""
    lo = np.uint32(101 << 23)   # exponent field 101 = 2^-26
    hi = np.uint32(144 << 23)   # exponent field 144 = 2^17
    n = int(hi - lo)
    step = 1 << 24
    bad = 0
    for sign in (0, 1 << 31):
        for s in range(0, n, step):
            bad += _block(int(lo) + sign + s, min(step, n - s))
    assert bad == 0


def test_f64_to_f16_random_and_ties():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(200000) * 1000,
        rng.standard_normal(200000) * 1e-6,
        np.ldexp(rng.random(200000), rng.integers(-30, 20, 200000)),
    ])
    # exact ties between neighbouring fp16 values, in normal and subnormal range
    h = np.arange(0, 0x7BFF, dtype=np.uint16)
    a = h.view(np.float16).astype(np.float64)
    b = (h + 1).view(np.float16).astype(np.float64)
    x = np.concatenate([x, -x, (a + b) / 2, -(a + b) / 2])
    ours = O.f16_from_f64(x)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f16_special_values():
    cases = [
        (0.0, 0x0000), (-0.0, 0x8000), (1.0, 0x3C00), (-2.0, 0xC000),
        (65504.0, 0x7BFF),                  # largest finite
        (65519.99, 0x7BFF),                 # below the halfway point to 2^16
        (65520.0, 0x7C00),                  # halfway rounds to even -> infinity
        (float("inf"), 0x7C00), (float("-inf"), 0xFC00),
        (2.0 ** -24, 0x0001),               # smallest subnormal
        (2.0 ** -25, 0x0000),               # tie between 0 and 2^-24 -> even (0)
        (3 * 2.0 ** -25, 0x0002),           # tie between 1 and 2 quanta -> even (2)
        (2.0 ** -14, 0x0400),               # smallest normal
        (1023.5 * 2.0 ** -24, 0x0400),      # tie carrying subnormal into normal
        (1.0 + 2.0 ** -11, 0x3C00),         # tie -> even mantissa 0
        (1.0 + 3 * 2.0 ** -11, 0x3C02),     # tie -> even mantissa 2
        (2047.5, 0x6800),                   # tie at 2047/2048 -> 2048
    ]
    for x, bits in cases:
        assert int(O.f16_from_f64(x)[0]) == bits, (x, hex(bits))
    nan = O.f16_from_f64(float("nan"))[0]
    assert (nan & 0x7C00) == 0x7C00 and (nan & 0x3FF) != 0


def test_f16_decode_all_patterns():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = O.f64_from_f16(h)
    ref = h.view(np.float16).astype(np.float64)
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()
    # decode then encode is the identity on every non-NaN pattern
    back = O.f16_from_f64(ours)
    finite = ~np.isnan(ref)
    assert np.array_equal(back[finite], h[finite])
