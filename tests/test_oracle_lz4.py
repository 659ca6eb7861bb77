"""Pins for the oracle's LZ4 block decoder and compressors.

The pages name LZ4 for compressed weight blocks ("GPU Compression Pipeline -
TDD Roadmap", Phase 2.1 and Phase 3.1) but do not define the format; these
tests pin the oracle to the public LZ4 block format with:

* hand-assembled streams at every field boundary (literal lengths 0/14/15/16/
  269/270/271/524/525, match lengths 4/18/19/20/273/274/275, distances
  1/2/3/4/7/8/63/64/65/65535), the expected bytes written out by hand;
* the overlap rule (distance < length repeats with period = distance);
* a random sequence generator that builds streams and expected output side by
  side, without the compressor;
* round trips and brute force for the compressor, and the two exact block
  sizes of the roadmap's 64 KiB 0xAB test input;
* corrupted streams (every truncation, bad distances, overruns, size
  mismatches): status != OK and nothing written past the chunk.
"""
import ctypes as C
import os

import numpy as np
import pytest

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def B(*parts):
    """Concatenate ints and byte strings into a uint8 array."""
    out = bytearray()
    for p in parts:
        if isinstance(p, int):
            out.append(p)
        else:
            out += bytes(p)
    return np.frombuffer(bytes(out), np.uint8)


def dec(stream, n):
    st, out, produced = O.lz4_decode(stream, n)
    return st, bytes(out[:produced])


def lit(n, seed=0):
    """n deterministic literal bytes (i*7+seed mod 251)."""
    return bytes((i * 7 + seed) % 251 for i in range(n))


def ext(v):
    """Extra length bytes for a saturated nibble: v = total - 15."""
    return bytes([255] * (v // 255) + [v % 255])


# --------------------------------------------------------- hand vectors

def test_empty_and_short_literals():
    assert dec(B(0x00), 0) == (O.OK, b"")
    assert dec(B(0x30, b"abc"), 3) == (O.OK, b"abc")
    assert dec(B(0xE0, lit(14)), 14) == (O.OK, lit(14))


@pytest.mark.parametrize("L", [15, 16, 269, 270, 271, 524, 525, 526, 1000])
def test_literal_length_extension(L):
    # token high nibble 15, then L-15 as 255-bytes and a final byte < 255
    stream = B(0xF0, ext(L - 15), lit(L))
    assert dec(stream, L) == (O.OK, lit(L))


def test_literal_ext_bytes_by_hand():
    assert list(ext(0)) == [0]
    assert list(ext(254)) == [254]            # L = 269
    assert list(ext(255)) == [255, 0]         # L = 270
    assert list(ext(256)) == [255, 1]         # L = 271
    assert list(ext(510)) == [255, 255, 0]    # L = 525


@pytest.mark.parametrize("M", [4, 5, 18, 19, 20, 273, 274, 275, 529, 1000])
def test_match_length_extension(M):
    # 8 literals "ABCDEFGH", match distance 8 of length M, then an empty last sequence
    code = M - 4
    tok = (8 << 4) | min(code, 15)
    mext = ext(code - 15) if code >= 15 else b""
    stream = B(tok, b"ABCDEFGH", 8, 0, mext, 0x00)
    expected = b"ABCDEFGH" + (b"ABCDEFGH" * 200)[:M]
    assert dec(stream, 8 + M) == (O.OK, expected)


@pytest.mark.parametrize("dist,M", [(1, 4), (1, 37), (2, 9), (3, 10), (4, 13), (7, 30),
                                    (8, 8), (63, 100), (64, 64), (65, 200), (65, 10)])
def test_overlapping_and_plain_distances(dist, M):
    prefix = lit(70, seed=3)
    code = M - 4
    tok = (15 << 4) | min(code, 15)
    mext = ext(code - 15) if code >= 15 else b""
    stream = B(tok, ext(70 - 15), prefix, dist & 255, dist >> 8, mext, 0x20, b"zz")
    # byte-serial copy written out: the match repeats the last `dist` bytes
    period = prefix[-dist:]
    expected = prefix + (period * (M // dist + 1))[:M] + b"zz"
    assert dec(stream, 70 + M + 2) == (O.OK, expected)


def test_distance_65535():
    prefix = lit(65535, seed=11)
    stream = B(0xF0, ext(65535 - 15), prefix, 0xFF, 0xFF, 0x10, b"q")
    # token 0xF0: the match nibble is 0 -> length 4, copying prefix[0:4]
    expected = prefix + prefix[:4] + b"q"
    assert dec(stream, 65535 + 4 + 1) == (O.OK, expected)


def test_two_sequences_and_last_literals():
    # "abcd" + match(dist 4, len 6) + "xy" + match(dist 3, len 4) + last "!"
    stream = B(0x42, b"abcd", 4, 0, 0x20, b"xy", 3, 0, 0x10, b"!")
    expected = b"abcd" + b"abcdab" + b"xy" + b"bxyb" + b"!"
    assert dec(stream, len(expected)) == (O.OK, expected)


# -------------------------------------------------------- error handling

def _decode_guarded(stream, cap, guard=64):
    """Decode with a guard band after the chunk; return (status, guard intact)."""
    stream = np.ascontiguousarray(stream, np.uint8)
    buf = np.full(cap + guard, 0xA5, np.uint8)
    produced = C.c_uint64(0)
    st = O.lib().ltref_lz4_decode_block(stream.ctypes.data_as(C.c_void_p), stream.size,
                                        buf.ctypes.data_as(C.c_void_p), cap, C.byref(produced))
    return int(st), bool(np.all(buf[cap:] == 0xA5))


def test_every_truncation_fails():
    stream, expected = O.seqgen(123, 3000)
    assert dec(stream, expected.size) == (O.OK, bytes(expected))
    for cut in range(stream.size):
        st, intact = _decode_guarded(stream[:cut], expected.size)
        assert st != O.OK and intact, cut


def test_bad_distances_and_overruns():
    assert dec(B(0x40, b"abcd", 0, 0, 0x00), 8)[0] == O.BAD_OFFSET          # distance 0
    assert dec(B(0x40, b"abcd", 5, 0, 0x00), 8)[0] == O.BAD_OFFSET          # before chunk start
    assert dec(B(0x40, b"abcd", 4, 0, 0x00), 8)[0] == O.OK                  # exactly at start
    assert dec(B(0x40, b"abcd", 4, 0, 0x00), 7)[0] == O.OVERRUN             # one byte too many
    assert dec(B(0x40, b"abcd", 4, 0, 0x00), 9)[0] == O.SIZE_MISMATCH       # one byte short
    assert dec(B(0x30, b"abc"), 2)[0] == O.OVERRUN
    assert dec(B(), 0)[0] == O.TRUNCATED                                     # empty input
    assert dec(B(0x40, b"abcd", 4), 8)[0] == O.TRUNCATED                    # half distance
    assert dec(B(0xF0), 20)[0] == O.TRUNCATED                                # missing ext byte
    assert dec(B(0xF0, 255, 255), 600)[0] == O.TRUNCATED
    for cap in (7, 9, 100):
        st, intact = _decode_guarded(B(0x40, b"abcd", 4, 0, 0x00), cap)
        assert intact


def test_flipped_bytes_never_write_outside():
    """One flipped byte (as the roadmap's corruption test does for its
    container): status may or may not be OK, but the guard band survives."""
    rng = np.random.default_rng(9)
    stream, expected = O.seqgen(77, 5000)
    for _ in range(2000):
        s = stream.copy()
        s[rng.integers(0, s.size)] ^= np.uint8(rng.integers(1, 256))
        st, intact = _decode_guarded(s, expected.size)
        assert intact


# ----------------------------------------------- generator-built streams

def _seqgen_batch(seeds, targets):
    """Streams from the sequence generator, decoded as one chunk table (one
    block per stream) by the oracle's table decoder; returns the statuses,
    the decoded bytes and the expected bytes."""
    streams, expect = [], []
    for s, t in zip(seeds, targets):
        a, b = O.seqgen(int(s), int(t))
        streams.append(a)
        expect.append(b)
    comp_off = np.concatenate([[0], np.cumsum([a.size for a in streams])]).astype(np.uint64)
    dst_off = np.concatenate([[0], np.cumsum([b.size for b in expect])]).astype(np.uint64)
    t = O.Table(np.concatenate(streams), comp_off, dst_off)
    out, st = O.decode_table(t)
    return st, out, np.concatenate(expect)


def test_seqgen_fuzz():
    """100,000 generator-built streams (sequence lists whose encoded bytes and
    expected output are built side by side, independent of the compressor)
    decode to their expected bytes."""
    n = 100_000
    seeds = np.arange(n)
    targets = np.array([0, 1, 50, 700, 5000, 20000])[seeds % 6]
    targets[seeds % 97 == 0] = 70000
    for lo in range(0, n, 20_000):
        st, out, exp = _seqgen_batch(seeds[lo:lo + 20_000], targets[lo:lo + 20_000])
        assert np.all(st == O.OK), np.nonzero(st)[0][:5] + lo
        assert np.array_equal(out, exp)


# ------------------------------------------------------------ compressor

def test_exact_sizes_64k():
    g = {}
    for line in open(os.path.join(GOLD, "lz4_64k_sizes.txt")):
        if line.strip() and not line.startswith("#"):
            k, v = line.split(":")
            g[k.strip()] = int(v)
    x = np.full(65536, 0xAB, np.uint8)
    c = O.lz4_compress(x)
    assert c.size == g["greedy_0xAB_65536"]
    assert list(c[:4]) == [0x1F, 0xAB, 0x01, 0x00]
    assert list(c[4:260]) == [0xFF] * 256 and c[260] == 0xE7
    assert list(c[261:]) == [0x50] + [0xAB] * 5
    s = O.lz4_store(x)
    assert s.size == g["store_65536"]
    assert list(s[:258]) == [0xF0] + [0xFF] * 256 + [0xF1]
    for blk in (c, s):
        st, out, _ = O.lz4_decode(blk, 65536)
        assert st == O.OK and np.array_equal(out, x)


def test_all_literal_block_round_trip():
    x = np.random.default_rng(1).integers(0, 256, 65536, dtype=np.uint8)
    c = O.lz4_compress(x)
    assert c.size == 65794          # incompressible: the compressor emits one literal run
    st, out, _ = O.lz4_decode(c, x.size)
    assert st == O.OK and np.array_equal(out, x)


def test_store_sizes():
    for n in (0, 1, 14, 15, 16, 269, 270, 271, 1000):
        s = O.lz4_store(np.zeros(n, np.uint8))
        want = 1 + n if n < 15 else 1 + (n - 15) // 255 + 1 + n
        assert s.size == want


def _round_trip_all(n, alphabet):
    """Every string of length n over `alphabet`, each compressed as its own
    block by the oracle's table compressor and decoded back by its table
    decoder (one chunk per string)."""
    k = len(alphabet)
    idx = np.arange(k ** n, dtype=np.int64)
    digits = np.empty((idx.size, n), np.uint8)
    a = np.asarray(alphabet, np.uint8)
    for p in range(n):
        digits[:, p] = a[(idx // k ** p) % k]
    src = digits.ravel()
    dst_off = (np.arange(idx.size + 1, dtype=np.uint64) * np.uint64(n))
    t = O.compress_table(src, dst_off)
    out, st = O.decode_table(t)
    assert np.all(st == O.OK)
    assert np.array_equal(out, src)
    return t


def test_compressor_brute_force_small():
    """Every string of <= 14 bytes over {0x00, 0xAB} and every string of <= 3
    bytes over all 256 values round-trips."""
    assert O.lz4_decode(O.lz4_compress(np.zeros(0, np.uint8)), 0)[0] == O.OK
    for n in range(1, 15):
        _round_trip_all(n, [0x00, 0xAB])
    for n in range(1, 4):
        _round_trip_all(n, list(range(256)))


@pytest.mark.slow
def test_compressor_brute_force_20():
    """Every string of length 15 ..= 20 over {0x00, 0xAB} (2,064,384 strings);
    with the fast test, all 2,097,151 strings of length <= 20."""
    for n in range(15, 21):
        _round_trip_all(n, [0x00, 0xAB])


def test_compressor_random_round_trips():
    rng = np.random.default_rng(4)
    for trial in range(300):
        n = int(rng.integers(0, 70000))
        kind = trial % 4
        if kind == 0:
            x = rng.integers(0, 256, n, dtype=np.uint8)
        elif kind == 1:
            x = rng.integers(0, 3, n, dtype=np.uint8)
        elif kind == 2:
            x = (rng.random(n) < 0.1).astype(np.uint8) * rng.integers(0, 256, n, dtype=np.uint8)
        else:
            x = np.repeat(rng.integers(0, 256, n // 50 + 1, dtype=np.uint8), 50)[:n]
        c = O.lz4_compress(x)
        assert c.size <= O.lz4_bound(n)
        st, out, _ = O.lz4_decode(c, n)
        assert st == O.OK and np.array_equal(out, x)
