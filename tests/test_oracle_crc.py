"""Pins of the oracle's CRC-32 (the per-chunk checksum of the roadmap's
container validation, "GPU Compression Pipeline - TDD Roadmap", Phase 6.1).

The oracle computes it bit by bit from the polynomial.  It is pinned to
* the CRC catalogue's published check value for this CRC (ISO-HDLC /
  IEEE 802.3): the nine ASCII bytes "123456789" give 0xCBF43926;
* Python's zlib.crc32, an independent implementation of the same CRC, on
  buffers of every length up to 300 and larger random ones;
* the empty message (0), and the detection of every single-byte change.
"""
import zlib

import numpy as np

import oracle as O


def test_published_check_value():
    assert O.crc32(b"123456789") == 0xCBF43926
    assert O.crc32(b"") == 0


def test_matches_zlib_on_many_lengths():
    rng = np.random.default_rng(0)
    for n in list(range(0, 300)) + [4095, 4096, 65536 + 7, 200001]:
        x = rng.integers(0, 256, n, dtype=np.uint8)
        assert O.crc32(x) == zlib.crc32(x.tobytes()), n
    for fill in (0, 0xFF, 0xAB):
        x = np.full(10000, fill, np.uint8)
        assert O.crc32(x) == zlib.crc32(x.tobytes())


def test_every_single_byte_change_is_detected():
    rng = np.random.default_rng(1)
    x = rng.integers(0, 256, 257, dtype=np.uint8)
    c = O.crc32(x)
    for i in range(x.size):
        y = x.copy()
        y[i] ^= np.uint8(rng.integers(1, 256))
        assert O.crc32(y) != c, i


def test_chunk_table():
    rng = np.random.default_rng(2)
    comp = rng.integers(0, 256, 50000, dtype=np.uint8)
    comp_off = np.array([0, 0, 1, 17, 4096, 4097, 30000, 50000], np.uint64)
    got = O.crc32_chunks(comp, comp_off)
    for i in range(comp_off.size - 1):
        a, b = int(comp_off[i]), int(comp_off[i + 1])
        assert got[i] == zlib.crc32(comp[a:b].tobytes()), i
