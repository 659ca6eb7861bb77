"""Pins of the oracle's zero-run coding of fp16 activations (the pages'
zero-run encoding for ReLU outputs: runs of zeros stored instead of full
arrays; here a per-1024-element bitmap of nonzero elements followed by the
nonzero values in order).

* the layout, from hand-written expected words: element 32 w + k is bit k of
  word w; val_off counts nonzeros before each block;
* closed forms: all zeros gives no values and zero bitmaps; no zeros gives
  vals equal to the input; -0.0 is kept (bits compared, not values);
* round trips on ReLU-shaped data, every length near a block boundary;
* a block whose counts do not match fails alone and is not written.
"""
import numpy as np

import oracle as O


def test_layout_by_hand():
    x = np.zeros(2100, np.uint16)
    x[0] = 0x3C00        # 1.0
    x[33] = 0x8000       # -0.0 is not zero bits
    x[1023] = 0x4000
    x[1024] = 0x0001     # smallest subnormal
    x[2099] = 0xFBFF
    bitmap, val_off, vals = O.zr_encode(x)
    assert bitmap.size == 3 * 32
    want = np.zeros(96, np.uint32)
    want[0] = 1
    want[1] = 1 << 1
    want[31] = 1 << 31
    want[32] = 1
    want[2099 // 32] = 1 << (2099 % 32)
    assert np.array_equal(bitmap, want)
    assert val_off.tolist() == [0, 3, 4, 5]
    assert vals.tolist() == [0x3C00, 0x8000, 0x4000, 0x0001, 0xFBFF]


def test_closed_forms():
    z = np.zeros(5000, np.uint16)
    b, o, v = O.zr_encode(z)
    assert v.size == 0 and not b.any() and not o.any()
    rng = np.random.default_rng(0)
    f = rng.integers(1, 65536, 5000).astype(np.uint16)
    b, o, v = O.zr_encode(f)
    assert np.array_equal(v, f) and o.tolist() == [0, 1024, 2048, 3072, 4096, 5000]
    assert np.all(b[:4 * 32] == 0xFFFFFFFF)
    assert np.array_equal(O.zr_decode(b, o, v, 5000)[0], f)


def test_round_trips():
    rng = np.random.default_rng(1)
    for n in (0, 1, 31, 32, 33, 1023, 1024, 1025, 2047, 2048, 3000, 100000):
        a = np.maximum(0, rng.standard_normal(n) - 1.3).astype(np.float16).view(np.uint16)
        b, o, v = O.zr_encode(a)
        out, st = O.zr_decode(b, o, v, n)
        assert np.all(st == 0) and np.array_equal(out, a), n
        assert v.size == np.count_nonzero(a)


def test_inconsistent_block_fails_alone():
    rng = np.random.default_rng(2)
    a = np.maximum(0, rng.standard_normal(4096) - 1.0).astype(np.float16).view(np.uint16)
    b, o, v = O.zr_encode(a)
    b = b.copy()
    b[32 * 2] ^= 1 << 5                       # block 2 gains or loses a bit
    out = np.full(4096, 0x7777, np.uint16)
    out, st = O.zr_decode(b, o, v, 4096, out)
    assert st.tolist() == [0, 0, 5, 0]
    assert np.all(out[2048:3072] == 0x7777)
    assert np.array_equal(out[:2048], a[:2048]) and np.array_equal(out[3072:], a[3072:])
    bits = O.zr_encode(np.ones(1000, np.uint16))[0].copy()
    bits[31] |= 1 << 31                       # a bit past n
    _, st = O.zr_decode(bits, np.array([0, 1001], np.uint64), np.ones(1001, np.uint16), 1000)
    assert st.tolist() == [5]
