"""Pins of the oracle's codebook dequantization (the pages' value
dictionaries: small integer codes plus a tiny lookup table per group).

* a table filled from the affine rule, lut[g][q] = fp16((q - zp[g]) * s[g]),
  reproduces the oracle's affine dequant (itself pinned to the roadmap's
  worked examples) on every element: group index and nibble order agree;
* a hand-written example with a per-tensor dictionary and with groups;
* an identity-like table exposes each code: lut[g][q] = 16 g + q.
"""
import numpy as np

import oracle as O
import synth


def test_affine_table_matches_affine_dequant():
    rng = np.random.default_rng(0)
    for rows, cols, group in ((64, 256, 128), (32, 300, 100), (8, 1024, 1024), (4, 64, 16)):
        n = rows * cols
        codes = rng.integers(0, 16, n, dtype=np.uint8)
        scales = synth.fp16_bits(rng.uniform(-0.05, 0.05, n // group))
        zp = rng.integers(-8, 16, n // group).astype(np.int8)
        ng = n // group
        q = np.arange(16, dtype=np.int64)
        vals = (q[None, :] - zp.astype(np.int64)[:, None]) * O.f64_from_f16(scales)[:, None]
        lut = O.f16_from_f64(vals.ravel()).reshape(ng, 16)
        packed = O.pack_int4(codes)
        assert np.array_equal(O.dequant_int4_lut(packed, lut, group), O.dequant_int4(packed, scales, zp, group))


def test_by_hand():
    packed = np.array([0x21, 0xF0], np.uint8)          # codes 1, 2, 0, 15
    lut = np.arange(16, dtype=np.uint16) * 3 + 100     # one dictionary for the tensor
    assert O.dequant_int4_lut(packed, lut, 4).tolist() == [103, 106, 100, 145]
    lut2 = np.stack([lut, lut + 1000])                 # two groups of two
    assert O.dequant_int4_lut(packed, lut2, 2).tolist() == [103, 106, 1100, 1145]


def test_index_table_exposes_codes():
    rng = np.random.default_rng(1)
    n, group = 4096, 64
    codes = rng.integers(0, 16, n, dtype=np.uint8)
    lut = (16 * np.arange(n // group)[:, None] + np.arange(16)[None, :]).astype(np.uint16)
    out = O.dequant_int4_lut(O.pack_int4(codes), lut, group)
    e = np.arange(n)
    assert np.array_equal(out, (16 * (e // group) + codes).astype(np.uint16))
