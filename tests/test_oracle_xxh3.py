"""Pins of the oracle's XXH3-64 (seed 0, default secret), the block checksum
the roadmap's container format names (page "GPU Compression Pipeline - TDD
Roadmap", Phase 6.1): against the xxhash package's own implementation,
which shares nothing with the oracle, on every input length through all of
the definition's length classes and block boundaries, and on large inputs;
and the property the container check relies on (a changed byte changes the
hash)."""
import numpy as np
import pytest

import oracle as O

xxhash = pytest.importorskip("xxhash")


def test_every_length_to_2200_and_block_boundaries():
    rng = np.random.default_rng(31)
    lengths = list(range(0, 2201)) + [1024 * k + d for k in range(2, 9) for d in (-65, -64, -63, -1, 0, 1)]
    for n in lengths:
        d = rng.integers(0, 256, n, dtype=np.uint8).tobytes()
        assert O.xxh3_64(d) == xxhash.xxh3_64_intdigest(d), n


def test_structured_and_large_inputs():
    rng = np.random.default_rng(32)
    cases = [bytes(65536), b"\xab" * 65536, bytes(range(256)) * 300,
             rng.integers(0, 4, 300_001, dtype=np.uint8).tobytes(),
             rng.integers(0, 256, 1 << 20, dtype=np.uint8).tobytes()]
    for d in cases:
        assert O.xxh3_64(d) == xxhash.xxh3_64_intdigest(d), len(d)


def test_chunks_hash_their_own_bytes():
    rng = np.random.default_rng(33)
    sizes = rng.integers(0, 5000, 300)
    comp = rng.integers(0, 256, int(sizes.sum()), dtype=np.uint8)
    comp_off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.uint64)
    h = O.xxh3_chunks(comp, comp_off)
    for i in range(sizes.size):
        assert int(h[i]) == xxhash.xxh3_64_intdigest(comp[int(comp_off[i]):int(comp_off[i + 1])].tobytes())


def test_every_single_byte_change_is_seen():
    rng = np.random.default_rng(34)
    for n in (1, 3, 8, 16, 100, 200, 240, 241, 1024, 1025, 3000):
        d = rng.integers(0, 256, n, dtype=np.uint8)
        base = O.xxh3_64(d)
        for k in range(n):
            e = d.copy()
            e[k] ^= np.uint8(1 + (k % 255))
            assert O.xxh3_64(e) != base, (n, k)
