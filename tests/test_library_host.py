"""Host-side checks of liblt.so that need no GPU.

* the library loads and exports every function include/lt.h declares;
* argument validation returns LT_ERR_INVALID_ARG before any device work;
* the host packer (nibble packing, LZ4 compressor) produces blocks that the
  CPU oracle decodes back to the input, on every workload.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle as O
import synth
from lz4_blocks import matches, max_match_distance, sequence_starts
import weight_dequantization_amd as lt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names += re.findall(r"\b(lt_[a-z0-9_]+)\s*\(", src)
    return sorted(set(names))


def test_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 10
    L = C.CDLL(lt.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert lt.lib().lt_abi_version() == lt.ABI_VERSION == 15
    assert lt.lib().lt_status_str(1) == b"invalid argument"
    assert lt.lib().lt_status_str(lt.LT_ERR_TOO_LARGE) == b"request exceeds the static workspace"


def test_invalid_arguments_rejected_without_gpu():
    L = lt.lib()
    V = C.c_void_p
    fake = V(0x10000)        # never dereferenced: validation fails first
    unaligned = V(0x10008)
    # null pointers
    assert L.lt_dequant_int4(None, fake, None, 4, 4, 4, fake, None) == lt.LT_ERR_INVALID_ARG
    assert L.lt_dequant_int4(fake, None, None, 4, 4, 4, fake, None) == lt.LT_ERR_INVALID_ARG
    # unaligned output, zero sizes, odd element count, bad groups
    assert L.lt_dequant_int4(fake, fake, None, 4, 4, 4, unaligned, None) == lt.LT_ERR_INVALID_ARG
    assert L.lt_dequant_int4(fake, fake, None, 0, 4, 4, fake, None) == lt.LT_ERR_INVALID_ARG
    assert L.lt_dequant_int4(fake, fake, None, 1, 3, 3, fake, None) == lt.LT_ERR_INVALID_ARG
    assert L.lt_dequant_int4(fake, fake, None, 4, 6, 4, fake, None) == lt.LT_ERR_INVALID_ARG
    assert L.lt_dequant_int8(fake, fake, None, 4, 4, 0, fake, None) == lt.LT_ERR_INVALID_ARG
    assert L.lt_dequant_int8(fake, fake, None, 3, 4, 8, fake, None) == lt.LT_ERR_INVALID_ARG
    # chunk tables
    t = lt._Table(0x10000, 0x10000, 0x10000, 4, 65536, 9, 100)           # 16 codes need 8 bytes
    assert L.lt_fused_lz4_int4(C.byref(t), fake, None, 4, 4, 4, fake, None, None) == lt.LT_ERR_INVALID_ARG
    t = lt._Table(0x10000, 0x10000, 0x10000, 1, 0, 8, 100)               # max_chunk_bytes 0
    assert L.lt_fused_lz4_int4(C.byref(t), fake, None, 4, 4, 4, fake, None, None) == lt.LT_ERR_INVALID_ARG
    t = lt._Table(0x10000, 0x10000, 0x10000, 1, (1 << 20) + 1, 8, 100)   # above the limit
    assert L.lt_decode_lz4(C.byref(t), fake, None, None) == lt.LT_ERR_INVALID_ARG
    t = lt._Table(None, 0x10000, 0x10000, 1, 8, 8, 100)
    assert L.lt_decode_lz4(C.byref(t), fake, None, None) == lt.LT_ERR_INVALID_ARG
    t = lt._Table(0x10000, 0x10000, 0x10000, 1, 8, 8, 100)
    assert L.lt_decode_lz4(C.byref(t), unaligned, None, None) == lt.LT_ERR_INVALID_ARG
    assert L.lt_decode_lz4(None, fake, None, None) == lt.LT_ERR_INVALID_ARG
    # int8 table size must equal rows*cols
    t = lt._Table(0x10000, 0x10000, 0x10000, 1, 16, 16, 100)
    assert L.lt_fused_lz4_int8(C.byref(t), fake, None, 4, 8, 8, fake, None, None) == lt.LT_ERR_INVALID_ARG
    # a declared window beyond the format's
    t = lt._Table(0x10000, 0x10000, 0x10000, 1, 8, 8, 100, 65536, 0)
    assert L.lt_decode_lz4(C.byref(t), fake, None, None) == lt.LT_ERR_INVALID_ARG
    # a sequence index needs both arrays
    t = lt._Table(0x10000, 0x10000, 0x10000, 1, 8, 8, 100, 0, 0, 0x10000, None, 4)
    assert L.lt_decode_lz4(C.byref(t), fake, None, None) == lt.LT_ERR_INVALID_ARG
    t = lt._Table(0x10000, 0x10000, 0x10000, 1, 8, 8, 100, 0, 0, None, 0x10000, 4)
    assert L.lt_decode_lz4(C.byref(t), fake, None, None) == lt.LT_ERR_INVALID_ARG
    # empty tables are valid no-ops (no device work)
    t = lt._Table(0, 0, 0, 0, 0, 0, 0)
    assert L.lt_decode_lz4(C.byref(t), fake, None, None) == lt.LT_OK


def test_pack_int4_matches_oracle():
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 16, 100002, dtype=np.uint8)
    assert np.array_equal(lt.pack_int4(codes), O.pack_int4(codes))
    with pytest.raises(lt.LtError):
        lt.pack_int4(codes[:3])


def _oracle_round_trip(data, dst_off):
    comp, comp_off = lt.compress_chunks(data, dst_off)
    t = O.Table(comp, comp_off, dst_off)
    out, st = O.decode_table(t)
    assert np.all(st == O.OK) and np.array_equal(out, data)
    return comp.size


def test_packer_blocks_decode_with_oracle_small():
    rng = np.random.default_rng(1)
    for n in (0, 1, 12, 13, 100, 4095, 70000):
        for kind in range(3):
            if kind == 0:
                x = rng.integers(0, 256, n, dtype=np.uint8)
            elif kind == 1:
                x = np.zeros(n, np.uint8)
            else:
                x = (rng.random(n) < 0.2).astype(np.uint8) * rng.integers(0, 4, n, dtype=np.uint8)
            _oracle_round_trip(x, np.array([0, n], np.uint64))
    x = np.full(65536, 0xAB, np.uint8)
    assert _oracle_round_trip(x, np.array([0, 65536], np.uint64)) < 300


def test_packer_tiny_and_mlp_small():
    for w in (synth.tiny_int4_1024(), synth.mlp_int4_small()):
        packed = lt.pack_int4(w.codes)
        size = _oracle_round_trip(packed, w.dst_off)
        ref = O.compress_table(packed, w.dst_off).comp_bytes
        # the product packer is within a few percent of the oracle's greedy compressor
        assert size <= ref * 1.03, (size, ref)


@pytest.mark.slow
def test_packer_full_workloads():
    for name in ("int8_8192x8192", "mlp_int4_8192x28672", "relu_4096x14336"):
        w = synth.WORKLOADS[name]()
        data = {"int8_8192x8192": lambda: w.q.view(np.uint8), "mlp_int4_8192x28672": lambda: lt.pack_int4(w.codes),
                "relu_4096x14336": lambda: w.data}[name]()
        size = _oracle_round_trip(data, w.dst_off)
        print(name, "compressed", size, "of", data.size)


def test_packer_mixed_chunks():
    w = synth.int4_weight(512, 8192, 128, 77, chunking="mixed")
    packed = lt.pack_int4(w.codes)
    _oracle_round_trip(packed, w.dst_off)


@pytest.mark.parametrize("max_dist", [1, 4096, lt.SMALL_WINDOW, 65535])
def test_packer_honours_declared_window(max_dist):
    """Every match the packer writes reaches at most max_dist bytes back, and
    the blocks still decode (oracle) to the input."""
    rng = np.random.default_rng(max_dist)
    n = 200000
    base = rng.integers(0, 256, 40000, dtype=np.uint8)
    x = np.concatenate([base, base[::-1], base, rng.integers(0, 3, n - 120000, dtype=np.uint8)])
    dst_off = np.array([0, 65536, 131072, n], np.uint64)
    comp, comp_off = lt.compress_chunks(x, dst_off, max_dist=max_dist)
    for c in range(3):
        blk = comp[int(comp_off[c]):int(comp_off[c + 1])]
        assert max_match_distance(blk) <= max_dist
    out, st = O.decode_table(O.Table(comp, comp_off, dst_off))
    assert np.all(st == O.OK) and np.array_equal(out, x)


@pytest.mark.parametrize("max_dist", [1, 4096, 65535])
def test_greedy_packer_round_trips_within_its_window(max_dist):
    """The greedy parse's blocks decode (oracle) to the input and keep every
    match within max_dist, on random, zero, short-alphabet and repeated data
    and on chunks of 0 to 13 bytes."""
    rng = np.random.default_rng(40 + max_dist)
    base = rng.integers(0, 256, 30000, dtype=np.uint8)
    parts = [base, np.zeros(5000, np.uint8), rng.integers(0, 3, 30000, dtype=np.uint8), base,
             rng.integers(0, 256, 13, dtype=np.uint8)]
    x = np.concatenate(parts)
    dst_off = np.array([0, 0, 12, 25, 40000, 70000, x.size], np.uint64)
    comp, comp_off = lt.compress_chunks(x, dst_off, max_dist=max_dist, greedy=True)
    for c in range(dst_off.size - 1):
        blk = comp[int(comp_off[c]):int(comp_off[c + 1])]
        assert all(d <= max_dist for d, _ in matches(blk))
    out, st = O.decode_table(O.Table(comp, comp_off, dst_off))
    assert np.all(st == O.OK) and np.array_equal(out, x)


def test_greedy_packer_takes_the_short_matches_the_default_leaves():
    """Data whose only repeats are 5-byte strings: the greedy parse codes
    them as matches of 4 to 7 bytes, the default parse (8-byte minimum,
    runs aside) leaves them as literals; on the layer's codes the greedy
    parse writes about as many sequences as the oracle's greedy compressor."""
    rng = np.random.default_rng(5)
    x = rng.integers(0, 256, 65536, dtype=np.uint8)
    for k in range(200, 65000, 37):
        x[k:k + 5] = x[k - 150:k - 145]
    dst_off = np.array([0, x.size], np.uint64)
    g = matches(lt.compress_chunks(x, dst_off, greedy=True)[0])
    d = matches(lt.compress_chunks(x, dst_off)[0])
    assert sum(1 for dist, m in g if m < 8 and dist > 1) > 1000
    assert all(m >= 8 or dist == 1 for dist, m in d)
    w = synth.mlp_int4_small(rows=64)
    packed = lt.pack_int4(w.codes)
    gc, go = lt.compress_chunks(packed, w.dst_off, greedy=True)
    oc = O.compress_table(packed, w.dst_off)
    ng = lt.index_chunks(gc, go)[1].size
    no = lt.index_chunks(oc.comp, oc.comp_off)[1].size
    assert 0.9 * no <= ng <= 1.1 * no, (ng, no)


def _index_matches_walk(comp, comp_off):
    seq_off, seq_pos = lt.index_chunks(comp, comp_off)
    assert seq_off[0] == 0 and seq_off.size == comp_off.size
    for i in range(comp_off.size - 1):
        blk = comp[int(comp_off[i]):int(comp_off[i + 1])]
        got = seq_pos[int(seq_off[i]):int(seq_off[i + 1])].tolist()
        assert got == sequence_starts(blk), "chunk %d" % i
    return seq_off, seq_pos


def test_index_chunks_lists_every_sequence():
    """The host index matches a walk of each block, for the packer's blocks,
    the oracle compressor's and generated streams with extreme lengths."""
    w = synth.int4_weight(64, 4096, 128, 5, chunking="mixed")
    packed = lt.pack_int4(w.codes)
    comp, comp_off = lt.compress_chunks(packed, w.dst_off)
    _index_matches_walk(comp, comp_off)
    t = O.compress_table(packed, w.dst_off)
    _index_matches_walk(t.comp, t.comp_off)
    streams = [O.seqgen(sd, n)[0] for sd, n in [(1, 0), (2, 15), (3, 300), (4, 70000), (5, 4096)]]
    comp_off = np.cumsum([0] + [s.size for s in streams]).astype(np.uint64)
    seq_off, _ = _index_matches_walk(np.concatenate(streams), comp_off)
    assert seq_off[1] - seq_off[0] == 1          # an empty block is one token


def test_index_chunks_malformed_and_args():
    L = lt.lib()
    blk = O.seqgen(9, 5000)[0]
    for cut in (1, 2, blk.size // 2, blk.size - 1):
        part = blk[:cut]
        _index_matches_walk(part, np.array([0, cut], np.uint64))
    seq_off = np.zeros(2, np.uint64)
    comp_off = np.array([0, blk.size], np.uint64)
    V = C.c_void_p
    ptr = lambda a: a.ctypes.data_as(V)
    assert L.lt_index_chunks(ptr(blk), ptr(comp_off), 1, None, None, 0, 1) == lt.LT_ERR_INVALID_ARG
    assert L.lt_index_chunks(ptr(blk), ptr(np.array([5, 0], np.uint64)), 1, ptr(seq_off), None, 0, 1) \
        == lt.LT_ERR_INVALID_ARG
    assert L.lt_index_chunks(ptr(blk), ptr(comp_off), 1, ptr(seq_off), None, 0, 1) == lt.LT_OK
    small = np.zeros(1, np.uint32)
    assert L.lt_index_chunks(ptr(blk), ptr(comp_off), 1, ptr(seq_off), ptr(small), 1, 1) \
        == lt.LT_ERR_INVALID_ARG
    assert seq_off[1] > 1                       # sized even when the buffer is short


def test_streamed_arguments_rejected_without_gpu():
    """The streamed entry points check the staging buffer and the host table
    on the host and return LT_ERR_INVALID_ARG before any device work."""
    L = lt.lib()
    V = C.c_void_p
    ptr = lambda a: a.ctypes.data_as(V)
    fake = V(0x10000)
    comp = np.zeros(4096, np.uint8)
    comp_off = np.array([0, 1000, 3000], np.uint64)
    dst_off = np.array([0, 4096, 8192], np.uint64)
    seq_off = np.array([0, 3, 9], np.uint64)
    seq_pos = np.zeros(9, np.uint32)

    def table(coff=comp_off, soff=None, n_seq=0, n=2):
        return lt._Table(ptr(comp), ptr(coff), ptr(dst_off), n, 4096, 8192, comp.size, 0, 0,
                         None if soff is None else ptr(soff), None if soff is None else ptr(seq_pos), n_seq)

    def dec(t, staging=fake, nbytes=1 << 20):
        return L.lt_stream_decode_lz4(C.byref(t), fake, None, staging, nbytes, None, None)

    inv = lt.LT_ERR_INVALID_ARG
    assert dec(table(), staging=None) == inv
    assert dec(table(), staging=V(0x10010)) == inv             # staging not 256-byte aligned
    meta = 2 * 256                                             # two offset arrays of 3 entries
    assert dec(table(), nbytes=meta + 256) == inv              # under two aligned halves
    assert dec(table(), nbytes=meta + 2 * 1792) == inv         # the 2000-byte chunk needs 2048 per half
    assert dec(table(np.array([8, 1000, 3000], np.uint64))) == inv      # must start at 0
    assert dec(table(np.array([0, 3000, 1000], np.uint64))) == inv      # decreasing
    assert dec(table(np.array([0, 1000, 5000], np.uint64))) == inv      # past comp_bytes
    assert dec(table(soff=seq_off, n_seq=8)) == inv            # index past n_seq
    assert dec(table(soff=np.array([0, 5, 4], np.uint64), n_seq=9)) == inv
    # the device-table checks apply too
    t = table()
    t.max_dist = 65536
    assert dec(t) == inv
    assert L.lt_stream_decode_lz4(None, fake, None, fake, 1 << 20, None, None) == inv
    assert L.lt_stream_decode_lz4(C.byref(table()), V(0x10008), None, fake, 1 << 20, None, None) == inv
    # int4: 8192 packed bytes are 16384 codes
    f = lambda rows, cols, g, sc=fake: L.lt_stream_fused_lz4_int4(C.byref(table()), sc, None, rows, cols, g,
                                                                 fake, None, fake, 1 << 20, None, None)
    assert f(4, 4096, 128, sc=None) == inv
    assert f(4, 4096, 100) == inv
    assert f(8, 4096, 128) == inv
    # nothing to do: no device work, OK
    empty = lt._Table(0, 0, 0, 0, 0, 0, 0)
    assert L.lt_stream_decode_lz4(C.byref(empty), fake, None, None, 0, None, None) == lt.LT_OK


def test_staging_bytes_holds_the_largest_window():
    """ChunkTable.staging_bytes sizes each half for the largest run of k
    consecutive chunks, with the library's 256-byte rounding."""
    torch = pytest.importorskip("torch")
    comp = np.zeros(10000, np.uint8)
    comp_off = np.array([0, 100, 5100, 5200, 10000], np.uint64)
    dst_off = np.array([0, 1, 2, 3, 4], np.uint64)
    t = lt.ChunkTable.from_host(comp, comp_off, dst_off, device="cpu")
    up = lambda x: (x + 255) // 256 * 256
    meta = 2 * up(8 * 5)
    assert t.staging_bytes(1) == meta + 2 * up(5000 + 16)
    assert t.staging_bytes(2) == meta + 2 * up(5100 + 16)
    assert t.staging_bytes(99) == meta + 2 * up(10000 + 16)
    t.set_index(np.array([0, 1, 7, 8, 30], np.uint64), np.zeros(30, np.uint32))
    assert t.staging_bytes(1) == meta + up(8 * 5) + up(4 * 30) + 2 * up(5000 + 16)


def test_range_arguments_rejected_without_gpu():
    """Chunk-range calls check the range and its bounds on the host."""
    L = lt.lib()
    V = C.c_void_p
    fake = V(0x10000)
    inv = lt.LT_ERR_INVALID_ARG
    t = lt._Table(0x10000, 0x10000, 0x10000, 4, 65536, 8192, 100)
    dec = lambda first, count, lo, hi, out=fake: L.lt_decode_lz4_range(C.byref(t), first, count, lo, hi, out,
                                                                     None, None)
    assert dec(3, 2, 0, 16) == inv                 # past the last chunk
    assert dec(0, 1, 32, 16) == inv                # bounds reversed
    assert dec(0, 1, 0, 8193) == inv               # past total_bytes
    assert dec(0, 1, 8, 16) == inv                 # first bound not a multiple of 16
    assert dec(0, 1, 0, 16, V(0x10004)) == inv     # unaligned output
    assert dec(2, 0, 0, 0) == lt.LT_OK             # empty range: nothing to do
    assert L.lt_decode_lz4_range(None, 0, 1, 0, 16, fake, None, None) == inv
    f4 = lambda rows, cols, g, sc=fake: L.lt_fused_lz4_int4_range(C.byref(t), sc, None, rows, cols, g, 0, 1, 0,
                                                                 16, fake, None, None)
    assert f4(4, 4096, 128, sc=None) == inv
    assert f4(4, 4096, 100) == inv
    assert f4(8, 4096, 128) == inv                 # 8192 bytes hold 16384 codes
    f8 = lambda rows, cols: L.lt_fused_lz4_int8_range(C.byref(t), fake, None, rows, cols, cols, 0, 1, 0, 16,
                                                     fake, None, None)
    assert f8(4, 4096) == inv                      # int8: one byte per element
    # the streamed calls also require non-decreasing dst_off
    comp = np.zeros(64, np.uint8)
    coff = np.array([0, 10, 20], np.uint64)
    doff = np.array([0, 32, 16], np.uint64)
    ptr = lambda a: a.ctypes.data_as(V)
    h = lt._Table(ptr(comp), ptr(coff), ptr(doff), 2, 4096, 32, 64)
    assert L.lt_stream_decode_lz4(C.byref(h), fake, None, fake, 1 << 20, None, None) == inv


def test_checksum_chunks_matches_oracle():
    """The host packer's per-chunk XXH3-64 equals the oracle's (and the
    xxhash package's), on packer blocks and on arbitrary byte ranges that
    cover every length class of the hash."""
    w = synth.int4_weight(64, 4096, 128, 6, chunking="mixed")
    comp, comp_off = lt.compress_chunks(lt.pack_int4(w.codes), w.dst_off)
    assert np.array_equal(lt.checksum_chunks(comp, comp_off), O.xxh3_chunks(comp, comp_off))
    rng = np.random.default_rng(3)
    buf = rng.integers(0, 256, 200000, dtype=np.uint8)
    lens = [0, 1, 2, 3, 4, 7, 8, 9, 16, 17, 32, 33, 64, 65, 96, 97, 128, 129, 240, 241, 1024, 1025, 1088, 5000]
    lens += list(rng.integers(0, 3000, 60))
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.uint64)
    assert off[-1] <= buf.size
    got = lt.checksum_chunks(buf, off, threads=3)
    assert np.array_equal(got, O.xxh3_chunks(buf, off))
    xxhash = pytest.importorskip("xxhash")
    for i in range(len(lens)):
        assert int(got[i]) == xxhash.xxh3_64_intdigest(buf[int(off[i]):int(off[i + 1])].tobytes())
    L = lt.lib()
    V = C.c_void_p
    ptr = lambda a: a.ctypes.data_as(V)
    h = np.zeros(2, np.uint64)
    assert L.lt_checksum_chunks(ptr(buf), ptr(np.array([5, 1, 9], np.uint64)), 2, ptr(h), 1) == lt.LT_ERR_INVALID_ARG
    assert L.lt_checksum_chunks(ptr(buf), None, 2, ptr(h), 1) == lt.LT_ERR_INVALID_ARG


def test_verify_arguments_rejected_without_gpu():
    L = lt.lib()
    fake = C.c_void_p(0x10000)
    t = lt._Table(0x10000, 0x10000, 0x10000, 4, 65536, 8192, 100)
    assert L.lt_verify_chunks(None, None, fake, fake, None) == lt.LT_ERR_INVALID_ARG
    assert L.lt_verify_chunks(C.byref(t), None, None, None, None) == lt.LT_ERR_INVALID_ARG   # nowhere to report
    assert L.lt_verify_chunks(C.byref(t), fake, fake, None, None) == lt.LT_ERR_INVALID_ARG   # expect needs status
    empty = lt._Table(0, 0, 0, 0, 0, 0, 0)
    assert L.lt_verify_chunks(C.byref(empty), None, fake, None, None) == lt.LT_OK


def test_encode_zero_runs_matches_oracle():
    """The host zero-run encoder writes the oracle's bitmap, offsets and
    values, for ReLU-shaped data at lengths around the block size and for
    the activation workload's stress patterns."""
    rng = np.random.default_rng(5)
    for n in (0, 1, 31, 1023, 1024, 1025, 4097, 100001):
        x = np.maximum(0, rng.standard_normal(n) - 1.3).astype(np.float16).view(np.uint16).copy()
        if n > 40:
            x[7] = 0x8000
            x[33] = 0x0001
        got = lt.encode_zero_runs(x, threads=3)
        ref = O.zr_encode(x)
        for g, r in zip(got, ref):
            assert np.array_equal(g, r), n
    a = synth.activation(64, 4096, 4, stress_frac=0.05)
    x = a.data.view(np.uint16)
    for g, r in zip(lt.encode_zero_runs(x), O.zr_encode(x)):
        assert np.array_equal(g, r)


def test_zero_run_arguments_rejected_without_gpu():
    L = lt.lib()
    fake = C.c_void_p(0x10000)
    z = lt._ZrTensor(0x10000, 0x10000, 0x10000, 4096, 10)
    assert L.lt_decode_zero_runs(None, fake, None, None) == lt.LT_ERR_INVALID_ARG
    assert L.lt_decode_zero_runs(C.byref(z), C.c_void_p(0x10002), None, None) == lt.LT_ERR_INVALID_ARG
    assert L.lt_decode_zero_runs(C.byref(lt._ZrTensor(0x10000, None, 0x10000, 4096, 10)), fake, None, None) \
        == lt.LT_ERR_INVALID_ARG
    assert L.lt_decode_zero_runs(C.byref(lt._ZrTensor(0x10000, 0x10000, None, 4096, 10)), fake, None, None) \
        == lt.LT_ERR_INVALID_ARG
    assert L.lt_decode_zero_runs(C.byref(lt._ZrTensor(None, None, None, 0, 0)), fake, None, None) == lt.LT_OK
    x = np.ones(10, np.uint16)
    bm, vo, vals = np.zeros(32, np.uint32), np.zeros(2, np.uint64), np.zeros(4, np.uint16)
    p = lambda a: a.ctypes.data_as(C.c_void_p)
    assert L.lt_encode_zero_runs(p(x), 10, p(bm), p(vo), p(vals), 4, 1) == lt.LT_ERR_INVALID_ARG   # 10 values
    assert L.lt_encode_zero_runs(p(x), 10, p(bm), p(vo), None, 0, 1) == lt.LT_OK and vo[1] == 10


def test_lut_arguments_rejected_without_gpu():
    L = lt.lib()
    fake = C.c_void_p(0x10000)
    inv = lt.LT_ERR_INVALID_ARG
    assert L.lt_dequant_int4_lut(fake, fake, 4, 64, 8, fake, None) == inv            # groups under 16
    assert L.lt_dequant_int4_lut(fake, fake, 4, 64, 100, fake, None) == inv          # shape rule
    assert L.lt_dequant_int4_lut(C.c_void_p(0x10002), fake, 4, 64, 16, fake, None) == inv   # packed alignment
    assert L.lt_dequant_int4_lut(fake, C.c_void_p(0x10008), 4, 64, 16, fake, None) == inv   # table alignment
    assert L.lt_dequant_int4_lut(fake, fake, 1, 17, 17, fake, None) == inv           # odd element count
    assert L.lt_dequant_int4_lut(None, fake, 4, 64, 16, fake, None) == inv


def test_gemv_arguments_rejected_without_gpu():
    L = lt.lib()
    fake = C.c_void_p(0x10000)
    t = lt._Table(0x10000, 0x10000, 0x10000, 4, 65536, 4 * 4096 // 2, 100)
    g = lambda rows, cols, group, x=fake, y=fake: L.lt_fused_lz4_int4_gemv(C.byref(t), fake, None, rows, cols, group,
                                                                          x, y, None, None)
    assert g(4, 4096, 128, x=None) == lt.LT_ERR_INVALID_ARG
    assert g(4, 4096, 128, y=C.c_void_p(0x10002)) == lt.LT_ERR_INVALID_ARG
    assert g(8, 4096, 128) == lt.LT_ERR_INVALID_ARG            # table holds 4 x 4096 codes
    assert g(4, 4096, 64) == lt.LT_ERR_UNSUPPORTED             # groups under 128
    t2 = lt._Table(0x10000, 0x10000, 0x10000, 4, 65536, 4 * 3328 // 2, 100)
    assert L.lt_fused_lz4_int4_gemv(C.byref(t2), fake, None, 4, 3328, 128, fake, fake, None, None) \
        == lt.LT_ERR_UNSUPPORTED                                # rows not a multiple of 512 codes


def test_static_workspace_rejects_tables_that_do_not_fit():
    """lt_stream_fused_lz4_int4_static checks on the host, before any device
    call, that the table's offsets plus two halves of the largest chunk fit
    its fixed workspace."""
    L = lt.lib()
    comp = np.zeros(16, np.uint8)
    comp_off = np.array([0, 17 << 20], np.uint64)      # one chunk of 17 MiB compressed
    dst_off = np.array([0, 16], np.uint64)
    p = lambda a: a.ctypes.data_as(C.c_void_p)
    t = lt._Table(p(comp).value, p(comp_off).value, p(dst_off).value, 1, 16, 16, 17 << 20)
    fake = C.c_void_p(0x10000)
    assert L.lt_stream_fused_lz4_int4_static(C.byref(t), fake, None, 1, 32, 32, fake, None, None) == \
        lt.LT_ERR_TOO_LARGE
    # the usual argument checks come first
    assert L.lt_stream_fused_lz4_int4_static(C.byref(t), None, None, 1, 32, 32, fake, None, None) == \
        lt.LT_ERR_INVALID_ARG
    assert L.lt_stream_fused_lz4_int4_static(C.byref(t), fake, None, 1, 30, 30, fake, None, None) == \
        lt.LT_ERR_INVALID_ARG


def test_order_chunks_starts_the_largest_first():
    """The launch order is a permutation of the chunks by decreasing decoded
    size, chunks of one size in table order."""
    rng = np.random.default_rng(8)
    n = 500
    sizes = rng.choice([16384, 65536, 262144], n)
    dst_off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.uint64)
    order = lt.order_chunks(dst_off)
    assert sorted(order.tolist()) == list(range(n))
    assert order.tolist() == sorted(range(n), key=lambda i: (-int(sizes[i]), i))
    assert lt.order_chunks(np.zeros(1, np.uint64)).size == 0
    assert lt.order_chunks(np.arange(0, 5 * 65536, 65536, dtype=np.uint64)).tolist() == [0, 1, 2, 3]
    bad = dst_off.copy()
    bad[3] = bad[5]
    with pytest.raises(lt.LtError):
        lt.order_chunks(bad)


def test_order_chunks_by_sequences():
    """On a sequence-dense table the launch order is by decreasing decoded
    size, then by decreasing sequence count, equal counts in table order."""
    rng = np.random.default_rng(9)
    n = 700
    sizes = rng.choice([16384, 65536], n)
    seqs = rng.integers(0, 40, n)
    seqs[::7] = 17                                   # ties keep table order
    dst_off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.uint64)
    seq_off = np.concatenate([[0], np.cumsum(seqs)]).astype(np.uint64)
    order = lt.order_chunks(dst_off, seq_off)
    assert sorted(order.tolist()) == list(range(n))
    assert order.tolist() == sorted(range(n), key=lambda i: (-int(sizes[i]), -int(seqs[i]), i))
    one = np.arange(0, 5 * 65536, 65536, dtype=np.uint64)
    assert lt.order_chunks(one, np.array([0, 3, 3, 10, 11], np.uint64)).tolist() == [2, 0, 3, 1]
    L = lt.lib()
    out = np.zeros(4, np.uint32)
    assert L.lt_order_chunks_by_sequences(one.ctypes.data_as(C.c_void_p), None, 4,
                                          out.ctypes.data_as(C.c_void_p)) == lt.LT_ERR_INVALID_ARG
    bad = np.array([0, 3, 2, 10, 11], np.uint64)        # seq_off not monotone
    with pytest.raises(lt.LtError):
        lt.order_chunks(one, bad)
    with pytest.raises(ValueError):
        lt.order_chunks(one, seq_off[:3])


def test_file_stream_arguments_rejected_without_gpu():
    """The file-streaming calls refuse a bad descriptor, a missing or too
    small pinned buffer and a bad table before any device work."""
    L = lt.lib()
    V = C.c_void_p
    ptr = lambda a: a.ctypes.data_as(V)
    comp = np.zeros(64, np.uint8)
    coff = np.array([0, 32, 64], np.uint64)
    doff = np.array([0, 64, 128], np.uint64)
    h = lt._Table(ptr(comp), ptr(coff), ptr(doff), 2, 4096, 128, 64)
    fake = V(0x10000)
    pin = np.zeros(1 << 16, np.uint8)
    inv = lt.LT_ERR_INVALID_ARG
    assert L.lt_stream_file_decode_lz4(-1, 0, C.byref(h), fake, None, ptr(pin), pin.size, 1, fake, 1 << 20, None,
                                       None) == inv
    assert L.lt_stream_file_decode_lz4(0, 0, C.byref(h), fake, None, None, pin.size, 1, fake, 1 << 20, None,
                                       None) == inv
    assert L.lt_stream_file_decode_lz4(0, 0, C.byref(h), fake, None, ptr(pin), 256, 1, fake, 1 << 20, None,
                                       None) == inv
    assert L.lt_stream_file_decode_lz4(0, 0, None, fake, None, ptr(pin), pin.size, 1, fake, 1 << 20, None,
                                       None) == inv
    assert L.lt_stream_file_fused_lz4_int4(0, 0, C.byref(h), None, None, 16, 16, 16, fake, None, ptr(pin),
                                           pin.size, 1, fake, 1 << 20, None, None) == inv   # no scales
    assert L.lt_status_str(lt.LT_ERR_IO).decode() == "a file read failed or ended early"


def test_gemm_arguments_rejected_without_gpu():
    """The fused GEMM refuses shapes off the tile grid, batches other than 16
    and 32, small groups and a short workspace before any device work."""
    L = lt.lib()
    fake = C.c_void_p(0x10000)
    n = 8
    t = lt._Table(0x10000, 0x10000, 0x10000, n, 1 << 16, 16 * 256 // 2, 100)
    ws = lt.gemm_workspace_bytes(n, 16)
    assert ws == n * 6 * 16 * 16 * 4
    call = lambda rows, cols, group, batch, wsb, tb=t: L.lt_fused_lz4_int4_gemm(
        C.byref(tb), fake, None, rows, cols, group, fake, batch, fake, fake, wsb, None, None)
    assert call(16, 256, 128, 16, ws - 4) == lt.LT_ERR_INVALID_ARG              # workspace too small
    assert call(16, 256, 128, 8, ws) == lt.LT_ERR_UNSUPPORTED                   # batch
    assert call(16, 256, 64, 16, ws) == lt.LT_ERR_UNSUPPORTED                   # group under 128
    t2 = lt._Table(0x10000, 0x10000, 0x10000, n, 1 << 16, 8 * 256 // 2, 100)
    assert call(8, 256, 128, 16, ws, t2) == lt.LT_ERR_UNSUPPORTED               # rows % 16
    t3 = lt._Table(0x10000, 0x10000, 0x10000, n, 1 << 16, 16 * 192 // 2, 100)
    assert call(16, 192, 64, 16, ws, t3) == lt.LT_ERR_UNSUPPORTED               # cols % 128
    assert call(16, 512, 128, 16, ws) == lt.LT_ERR_INVALID_ARG                  # table size != shape
    assert L.lt_fused_lz4_int4_gemm(None, fake, None, 16, 256, 128, fake, 16, fake, fake, ws, None,
                                    None) == lt.LT_ERR_INVALID_ARG


def test_release_build_has_no_debug_counters():
    L = lt.lib()
    n = C.c_uint32(5)
    assert L.lt_debug_violations(C.byref(n), C.byref(n), 0) == lt.LT_ERR_UNSUPPORTED
    assert L.lt_debug_selftest(None, None) == lt.LT_ERR_UNSUPPORTED


def test_build_concat_lays_tables_end_to_end():
    """A table over several tensors is their tables end to end: the same
    compressed chunks, offsets shifted, and the oracle decodes it to the
    tensors' bytes back to back."""
    import oracle as O
    rng = np.random.default_rng(12)
    srcs, dst_offs = [], []
    for n, chunk in ((70000, 16384), (4096, 4096), (200003, 65536)):
        src = rng.integers(0, 4, n, dtype=np.uint8) * 17
        srcs.append(src)
        dst_offs.append(np.append(np.arange(0, n, chunk, dtype=np.uint64), np.uint64(n)))
    table, starts = lt.ChunkTable.build_concat(srcs, dst_offs, device="cpu", order=False)
    assert starts.tolist() == [0, 70000, 74096]
    assert table.n_chunks == sum(d.size - 1 for d in dst_offs)
    assert table.total_bytes == sum(s.size for s in srcs)
    comp = table.comp.numpy()[:table.comp_bytes]
    comp_off = table.comp_off.numpy().view(np.uint64)
    dst_off = table.dst_off.numpy().view(np.uint64)
    k = 0
    for src, d, st in zip(srcs, dst_offs, starts):
        one, one_off = lt.compress_chunks(src, d, max_dist=lt.PACK_WINDOW)
        for j in range(d.size - 1):
            assert dst_off[k + j] == d[j] + st
            a = comp[comp_off[k + j]:comp_off[k + j + 1]]
            assert np.array_equal(a, one[one_off[j]:one_off[j + 1]])
        k += d.size - 1
    t = O.Table(comp, comp_off, dst_off)
    got, st = O.decode_table(t, 4)
    assert not np.any(st)
    assert np.array_equal(got[:table.total_bytes], np.concatenate(srcs))
    with pytest.raises(ValueError):
        lt.ChunkTable.build_concat(srcs, dst_offs[:2], device="cpu")
    with pytest.raises(ValueError):
        lt.ChunkTable.build_concat([srcs[0]], [dst_offs[1]], device="cpu")
