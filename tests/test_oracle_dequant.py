"""Pins for the oracle's INT4/INT8 packing and dequantization.

Dequantization is out[e] = fp16((q[e] - zp[g]) * scale[g]) with g = e // group
("GPU Compression Pipeline - TDD Roadmap", Phase 1.1 INT4 Dequantization and
Phase 1.2 INT8 Dequantization).  Pins:

* the roadmap's printed INT4 example (low nibble first, scale 0.5 -> 0.0..3.5);
* the roadmap's INT8 example, its fp16 results derived from exact rationals;
* the whole (q, zp, scale) domain against numpy's float64 -> float16 rounding
  of the exact product (the product has at most 19 significant bits, so the
  float64 and float32 products are exact and round identically);
* closed forms that reveal each element's group index and the zero point's
  direction;
* brute force for pack/unpack.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

pytestmark = pytest.mark.filterwarnings("ignore:overflow encountered in cast")

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    d = {}
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, v = line.split(":", 1)
        d[k.strip()] = v.split()
    return d


def test_int4_roadmap_example():
    g = _read_golden("int4_roadmap_example.txt")
    packed = np.array([int(x, 16) for x in g["packed"]], np.uint8)
    scale = np.array([0.5], np.float16).view(np.uint16)
    zp = np.array([int(g["zero_point"][0])], np.int8)
    out = O.dequant_int4(packed, scale, zp, group=8)
    expected = np.array([float(x) for x in g["expected"]], np.float16).view(np.uint16)
    assert np.array_equal(out, expected)
    # the same with the zero point omitted (NULL -> 0)
    assert np.array_equal(O.dequant_int4(packed, scale, None, group=8), expected)


def _rne_f16_of_fraction(x: Fraction) -> int:
    """Exact round-to-nearest-even of a rational to fp16 (finite normal/subnormal
    range), written with integer arithmetic only."""
    if x == 0:
        return 0
    sign = 0x8000 if x < 0 else 0
    x = abs(x)
    e = 15
    while x >= Fraction(2) ** (e + 1) and e < 16:
        e += 1
    while x < Fraction(2) ** e and e > -14:
        e -= 1
    q = Fraction(2) ** (e - 10) if x >= Fraction(2) ** -14 else Fraction(2) ** -24
    n = x / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * q
    # re-encode from the rounded value
    if v < Fraction(2) ** -14:
        return sign | int(v / Fraction(2) ** -24)
    e = 15
    while v >= Fraction(2) ** (e + 1):
        e += 1
    while v < Fraction(2) ** e:
        e -= 1
    frac = int((v / Fraction(2) ** e - 1) * 1024)
    return sign | ((e + 15) << 10) | frac


def test_int8_roadmap_example():
    g = _read_golden("int8_roadmap_example.txt")
    values = np.array([int(x) for x in g["values"]], np.int8)
    s_bits = np.array([float(g["scale"][0])], np.float16).view(np.uint16)
    assert int(s_bits[0]) == int(g["scale_fp16_bits"][0], 16)
    s_exact = Fraction(1311, 2 ** 17)           # the fp16 value of 0.01
    assert float(s_exact) == float(np.uint16(s_bits[0]).view(np.float16))
    derived = [_rne_f16_of_fraction(int(v) * s_exact) for v in values]
    assert derived == [int(b, 16) for b in g["expected_bits"]]
    out = O.dequant_int8(values, s_bits, None, group=8)
    assert [int(x) for x in out] == derived
    # round-half-away-from-zero would give 0x3BAF for the tie at 96
    assert int(out[5]) == 0x3BAE


def _finite_f16_bits():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return h[(h & 0x7C00) != 0x7C00]


def test_int4_full_domain():
    """Every code 0..15 x every zero point -128..127 x every finite fp16 scale."""
    scales = _finite_f16_bits()                         # 63488 patterns
    s64 = scales.view(np.float16).astype(np.float64)
    s32 = scales.view(np.float16).astype(np.float32)
    codes = np.tile(np.arange(16, dtype=np.uint8), scales.size)
    packed = O.pack_int4(codes)
    q = np.arange(16, dtype=np.float64)
    for z in range(-128, 128):
        zp = np.full(scales.size, z, np.int8)
        out = O.dequant_int4(packed, scales, zp, group=16).reshape(scales.size, 16)
        ref64 = ((q[None, :] - z) * s64[:, None]).astype(np.float16).view(np.uint16)
        ref32 = ((q[None, :].astype(np.float32) - np.float32(z)) * s32[:, None]).astype(np.float16).view(np.uint16)
        assert np.array_equal(out, ref64), z
        assert np.array_equal(ref32, ref64), z


def test_int8_full_domain_zp0_and_zp_sweep():
    scales = _finite_f16_bits()
    s64 = scales.view(np.float16).astype(np.float64)
    qv = np.arange(-128, 128, dtype=np.int64).astype(np.int8)
    q = np.tile(qv, scales.size)
    out = O.dequant_int8(q, scales, None, group=256).reshape(scales.size, 256)
    ref = (qv.astype(np.float64)[None, :] * s64[:, None]).astype(np.float16).view(np.uint16)
    assert np.array_equal(out, ref)
    sub = scales[::97]
    s64 = sub.view(np.float16).astype(np.float64)
    q = np.tile(qv, sub.size)
    for z in range(-128, 128, 5):
        zp = np.full(sub.size, z, np.int8)
        out = O.dequant_int8(q, sub, zp, group=256).reshape(sub.size, 256)
        ref = ((qv.astype(np.float64)[None, :] - z) * s64[:, None]).astype(np.float16).view(np.uint16)
        assert np.array_equal(out, ref), z


@pytest.mark.parametrize("group", [8, 128, 256, 1000, 4096])
def test_group_addressing_closed_form(group):
    """Scales s_g = 2^-(g mod 8) * (1 + (g mod 1024)/1024) are exact in fp16.
    Pass 1 sets q - zp = 1, so out[e] == s_{e // group} reveals g mod 1024;
    pass 2 sets q - zp = 1 + (g // 1024 mod 15), revealing the high part."""
    n_groups = 2100
    n = n_groups * group
    g = np.arange(n_groups)
    s = np.ldexp(1.0 + (g % 1024) / 1024.0, -(g % 8))
    s_bits = s.astype(np.float16).view(np.uint16)
    assert np.array_equal(s_bits.view(np.float16).astype(np.float64), s)   # exact
    ge = np.arange(n) // group
    zp = np.full(n_groups, 3, np.int8)
    codes = np.full(n, 4, np.uint8)                          # q - zp = 1
    out = O.dequant_int4(O.pack_int4(codes), s_bits, zp, group)
    assert np.array_equal(out, s_bits[ge])
    k = 1 + (g // 1024) % 15
    codes = k[ge].astype(np.uint8)                           # zp 0: q - zp = k
    out = O.dequant_int4(O.pack_int4(codes), s_bits, None, group)
    got = out.view(np.float16).astype(np.float64)
    want = (k * s).astype(np.float16).astype(np.float64)[ge]
    assert np.array_equal(got, want)


def test_zero_point_direction():
    s = np.array([0.75], np.float16).view(np.uint16)
    for z in range(0, 16):
        zp = np.array([z], np.int8)
        codes = np.arange(16, dtype=np.uint8)
        out = O.dequant_int4(O.pack_int4(codes), s, zp, group=16).view(np.float16)
        assert out[z] == 0.0 and not np.signbit(out[z])        # q == zp -> +0
        if z + 1 < 16:
            assert out[z + 1] == np.float16(0.75)               # q - zp = +1
        if z > 0:
            assert out[z - 1] == np.float16(-0.75)              # q - zp = -1
    neg = np.array([-0.5], np.float16).view(np.uint16)
    out = O.dequant_int4(np.array([0x33], np.uint8), neg, np.array([3], np.int8), 2)
    assert np.all(out == 0x8000)                                # 0 * negative -> -0


def test_per_tensor_special_case():
    """group = rows*cols is the roadmap's single-scale fused test (scale 0.1)."""
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, 1024, dtype=np.uint8)
    s = np.array([0.1], np.float16).view(np.uint16)
    out = O.dequant_int4(O.pack_int4(codes), s, None, group=1024)
    ref = (codes.astype(np.float64) * np.float16(0.1).astype(np.float64)).astype(np.float16)
    assert np.array_equal(out, ref.view(np.uint16))


def test_pack_unpack_brute_force():
    b = np.arange(256, dtype=np.uint32).astype(np.uint8)
    codes = O.unpack_int4(b)
    assert np.array_equal(codes[0::2], b & 15) and np.array_equal(codes[1::2], b >> 4)
    assert np.array_equal(O.pack_int4(codes), b)
    pairs = np.array([(lo, hi) for hi in range(16) for lo in range(16)], np.uint8).ravel()
    assert np.array_equal(O.pack_int4(pairs), b)
