"""GPU parity: every liblt entry point against the CPU oracle, element by element.

Bar: bit-exact for decoded bytes and for fp16 outputs (the dequantized value
is the exact product rounded once, so 0 ULP is well defined).  Inputs are the
seeded synthetic workloads (synth) at full size and at small sizes that span
several 1 KiB tiles, several chunks and a ragged tail; LZ4 streams come from
both the library's host packer (the configuration the benchmark times) and
the oracle's own compressor and sequence generator.  Expected values come from
the oracle applied to the generator's codes, never from the GPU path.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import weight_dequantization_amd as lt
from lz4_blocks import max_match_distance

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield
    torch.cuda.synchronize()


def t_u16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def t_i8(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.int8)).to(DEV)


def t_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to(DEV)


def host_u16(t):
    torch.cuda.synchronize()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).ravel()


def assert_same(got, ref, what):
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, "%s: %d of %d differ, first at %d: got %#x want %#x" % (
        what, bad.size, ref.size, bad[0], got[bad[0]], ref[bad[0]])


def status_tensor(n):
    return torch.full((max(n, 1),), -1, dtype=torch.int32, device=DEV)


def statuses(st, n):
    torch.cuda.synchronize()
    return st[:n].cpu().numpy()


def table_from_oracle(ot: O.Table, index=False):
    return lt.ChunkTable.from_host(ot.comp, ot.comp_off, ot.dst_off, DEV, index=index)


# ------------------------------------------------------------ raw dequant

def _raw_int4(codes, scales, zp, rows, cols, group):
    packed = lt.pack_int4(codes)
    out = lt.dequant_int4(t_u8(packed), t_u16(scales), t_i8(zp), (rows, cols), group)
    ref = O.dequant_int4(O.pack_int4(codes), scales, zp, group)
    assert_same(host_u16(out), ref, "dequant_int4 %dx%d g%d" % (rows, cols, group))


def test_raw_int4_tiny_int4():
    w = synth.tiny_int4_1024()
    _raw_int4(w.codes, w.scales, w.zp, w.rows, w.cols, w.group)


def test_raw_int4_mlp_8192x28672_full():
    w = synth.mlp_int4_8192x28672()
    _raw_int4(w.codes, w.scales, w.zp, w.rows, w.cols, w.group)


def test_raw_int4_whole_domain():
    """every code x every zero point x every finite fp16 scale, group 16"""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    scales = h[(h & 0x7C00) != 0x7C00]
    n_groups = scales.size * 256
    sc = np.repeat(scales[None, :], 256, axis=0).ravel()
    zp = np.repeat(np.arange(-128, 128, dtype=np.int64).astype(np.int8), scales.size)
    codes = np.tile(np.arange(16, dtype=np.uint8), n_groups)
    _raw_int4(codes, sc, zp, n_groups, 16, 16)


def _group128_domain():
    """Group-128 INT4 over the whole code and zero-point domain: every code
    0..15 (eight times each, shuffled within its group) under every zero point
    -128..127, for 1024 fp16 scales that cover every exponent field 0..30 with
    both signs (subnormals and signed zeros included) at the mantissas 0, 1,
    2, 0x0FF, 0x200, 0x3FE, 0x3FF, plus finite scales drawn at random.  8192
    rows of 4096 codes (32 groups per row)."""
    rng = np.random.default_rng(128)
    fixed = [(sgn << 15) | (e << 10) | m for sgn in (0, 1) for e in range(31)
             for m in (0, 1, 2, 0x0FF, 0x200, 0x3FE, 0x3FF)]
    extra = rng.integers(0, 0x7C00, 1024 - len(fixed)) | (rng.integers(0, 2, 1024 - len(fixed)) << 15)
    scales_1 = np.array(fixed + list(extra), np.uint16)
    assert scales_1.size == 1024 and np.all((scales_1 & 0x7C00) != 0x7C00)
    n_groups = 256 * scales_1.size
    scales = np.repeat(scales_1, 256)
    zp = np.tile(np.arange(-128, 128, dtype=np.int64).astype(np.int8), scales_1.size)
    base = np.tile(np.arange(16, dtype=np.uint8), 8)
    codes = base[np.argsort(rng.random((n_groups, 128)), axis=1)]
    return codes.ravel(), scales, zp, 8192, 4096


def test_int4_group128_whole_domain_tiles_and_fused():
    """The 1 KiB-tile raw kernel and the fused group-128 write-out over every
    code x every zero point x scales of every exponent, bit for bit."""
    codes, scales, zp, rows, cols = _group128_domain()
    _raw_int4(codes, scales, zp, rows, cols, 128)
    w = synth.Int4Weight(rows, cols, 128, codes, scales, zp, synth.uniform_chunks(rows * cols // 2))
    packed = lt.pack_int4(codes)
    _fused4(lt.ChunkTable.build(packed, w.dst_off, DEV), w, "group-128 domain, packer, indexed")
    _fused4(lt.ChunkTable.build(packed, w.dst_off, DEV, index=False), w, "group-128 domain, packer, walked")
    w.zp = None
    _fused4(lt.ChunkTable.build(packed, w.dst_off, DEV), w, "group-128 domain, no zero points")


@pytest.mark.parametrize("rows,cols,group", [
    (10, 36, 6), (10, 36, 12), (10, 36, 36), (10, 36, 360), (3, 2, 2), (1, 6, 6), (7, 10, 70),
    (33, 128, 128), (64, 4096, 4096 * 64), (17, 24, 8), (5, 1000, 1000),
])
def test_raw_int4_groups_and_tails(rows, cols, group):
    rng = np.random.default_rng(rows * 1000 + cols + group)
    n = rows * cols
    codes = rng.integers(0, 16, n, dtype=np.uint8)
    scales = synth.fp16_bits(rng.uniform(-2, 2, n // group))
    zp = rng.integers(-128, 128, n // group).astype(np.int8)
    _raw_int4(codes, scales, zp, rows, cols, group)
    _raw_int4(codes, scales, None, rows, cols, group)


def _raw_int8(q, scales, zp, rows, cols, group):
    out = lt.dequant_int8(t_i8(q), t_u16(scales), t_i8(zp), (rows, cols), group)
    ref = O.dequant_int8(q, scales, zp, group)
    assert_same(host_u16(out), ref, "dequant_int8 %dx%d g%d" % (rows, cols, group))


def test_raw_int8_int8_8192():
    w = synth.int8_8192x8192()
    _raw_int8(w.q, w.scales, w.zp, w.rows, w.cols, w.group)


def test_raw_int8_domain_and_groups():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    scales = h[(h & 0x7C00) != 0x7C00]
    q = np.tile(np.arange(-128, 128, dtype=np.int64).astype(np.int8), scales.size)
    _raw_int8(q, scales, None, scales.size, 256, 256)
    rng = np.random.default_rng(3)
    zp = rng.integers(-128, 128, scales.size).astype(np.int8)
    _raw_int8(q, scales, zp, scales.size, 256, 256)
    for rows, cols, g in [(10, 36, 6), (3, 5, 5), (1, 13, 13), (9, 9, 81), (4, 24, 12)]:
        n = rows * cols
        qq = rng.integers(-128, 128, n).astype(np.int8)
        s = synth.fp16_bits(rng.uniform(-1, 1, n // g))
        z = rng.integers(-128, 128, n // g).astype(np.int8)
        _raw_int8(qq, s, z, rows, cols, g)


# ------------------------------------------------------------- decode-only

def _decode_check(table, expected, what):
    st = status_tensor(table.n_chunks)
    out = lt.decode_lz4(table, status=st)
    s = statuses(st, table.n_chunks)
    assert np.all(s == 0), "%s: chunk statuses %s" % (what, np.unique(s))
    got = out.cpu().numpy()
    bad = np.nonzero(got != expected)[0]
    assert bad.size == 0, "%s: %d bytes differ, first at %d" % (what, bad.size, bad[0])


def _seq_table(seeds, sizes):
    streams, expect = [], []
    for sd, n in zip(seeds, sizes):
        s, e = O.seqgen(int(sd), int(n))
        streams.append(s)
        expect.append(e)
    comp_off = np.cumsum([0] + [s.size for s in streams]).astype(np.uint64)
    dst_off = np.cumsum([0] + list(sizes)).astype(np.uint64)
    return O.Table(np.concatenate(streams), comp_off, dst_off), np.concatenate(expect)


def test_decode_generated_streams():
    """Generator-built streams (boundary lengths, distances 1..65535,
    overlapping matches), many per table; chunk sizes multiples of 16 except
    the last."""
    rng = np.random.default_rng(11)
    for trial in range(6):
        n = int(rng.integers(1, 300))
        sizes = list(16 * rng.integers(0, 70000 // 16, n))
        sizes[-1] = int(rng.integers(0, 70000))
        t, e = _seq_table(rng.integers(0, 2**62, n), sizes)
        _decode_check(table_from_oracle(t), e, "seqgen table %d" % trial)


@pytest.mark.parametrize("size", [65536 + 16, 200000, 262144, 700_001, 1 << 20])
def test_decode_chunks_larger_than_history(size):
    """Chunks over 64 KiB wrap the history ring; distances up to 65535."""
    t, e = _seq_table([size], [size])
    _decode_check(table_from_oracle(t), e, "big chunk %d" % size)


def _repeats(n, seed, reach):
    """Bytes with copies from up to `reach` bytes back, runs and noise."""
    rng = np.random.default_rng(seed)
    x = (rng.integers(0, 16, n, dtype=np.uint8) * 17).astype(np.uint8)
    x[::97] = 0
    for r in range(0, n - 700, 1500):
        d = int(rng.integers(1, reach))
        if r >= d:
            x[r:r + 700] = x[r - d:r - d + 700]
    return x


@pytest.mark.parametrize("size", [16384 + 16, 65536, 200000, 1 << 20])
def test_decode_short_window_chunks(size):
    """Tables that declare a window within SMALL_WINDOW decode with a 16 KiB
    history ring, which chunks over 16 KiB wrap many times; the builders'
    wait for earlier tiles follows the declared window."""
    x = _repeats(3 * size + 5, size, lt.SMALL_WINDOW)
    dst = np.array([0, size, 2 * size, 3 * size, 3 * size + 5], np.uint64)
    for win in (lt.PACK_WINDOW, 1, 1024, 7000):
        t = lt.ChunkTable.build(x, dst, DEV, max_dist=win)
        _decode_check(t, x, "window %d, chunk %d" % (win, size))
    table = lt.ChunkTable.build(x, dst, DEV, max_dist=lt.SMALL_WINDOW)
    assert table.max_dist == lt.SMALL_WINDOW
    _decode_check(table, x, "short window, chunk %d" % size)
    # the same blocks declared with any window (64 KiB history) decode alike
    t2 = lt.ChunkTable(table.comp, table.comp_off, table.dst_off, table.n_chunks,
                       table.max_chunk_bytes, table.total_bytes, table.comp_bytes, 0)
    _decode_check(t2, x, "same blocks, any window, chunk %d" % size)


def test_declared_window_is_enforced():
    """A block with a match farther back than the table's declared window
    fails with BAD_OFFSET; the other chunks are unaffected."""
    x = _repeats(4 * 65536, 9, 60000)
    dst = np.arange(5, dtype=np.uint64) * np.uint64(65536)
    ot = O.compress_table(x, dst)          # the oracle's compressor uses the full 64 KiB window
    far = []
    for i in range(4):
        blk = ot.comp[int(ot.comp_off[i]):int(ot.comp_off[i + 1])]
        far.append(max_match_distance(blk) > lt.SMALL_WINDOW)
    assert any(far)
    small = lt.ChunkTable.from_host(ot.comp, ot.comp_off, ot.dst_off, DEV, max_dist=lt.SMALL_WINDOW)
    st = status_tensor(small.n_chunks)
    out = lt.decode_lz4(small, status=st)
    s = statuses(st, small.n_chunks)
    got = out.cpu().numpy()
    for i in range(4):
        if far[i]:
            assert s[i] == lt.CHUNK_BAD_OFFSET, (i, s[i])
        else:
            assert s[i] == 0 and np.array_equal(got[65536 * i:65536 * (i + 1)], x[65536 * i:65536 * (i + 1)])


def test_decode_relu_4096x14336_full():
    a = synth.relu_4096x14336()
    _decode_check(lt.ChunkTable.build(a.data, a.dst_off, DEV), a.data, "relu_4096x14336 packer")
    _decode_check(table_from_oracle(O.compress_table(a.data, a.dst_off)), a.data, "relu_4096x14336 oracle")


def test_decode_stress_blocks():
    x = np.full(65536, 0xAB, np.uint8)
    for blk in (O.lz4_compress(x), O.lz4_store(x)):
        t = O.Table(blk, np.array([0, blk.size], np.uint64), np.array([0, 65536], np.uint64))
        _decode_check(table_from_oracle(t), x, "0xAB block %d" % blk.size)
    r = np.random.default_rng(2).integers(0, 256, 65536, dtype=np.uint8)
    blk = O.lz4_compress(r)
    t = O.Table(blk, np.array([0, blk.size], np.uint64), np.array([0, 65536], np.uint64))
    _decode_check(table_from_oracle(t), r, "all-literal block")
    # empty chunks and a zero-length block
    e = np.zeros(0, np.uint8)
    t = O.Table(np.array([0x00, 0x00], np.uint8), np.array([0, 1, 2], np.uint64), np.array([0, 0, 0], np.uint64))
    _decode_check(table_from_oracle(t), e, "empty chunks")


def _guarded_decode(ot, total, guard=4096):
    table = table_from_oracle(ot)
    buf = torch.full((total + 2 * guard,), 0xA5, dtype=torch.uint8, device=DEV)
    st = status_tensor(table.n_chunks)
    lt.decode_lz4(table, out=buf[guard:guard + max(total, 1)], status=st)
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    assert np.all(b[:guard] == 0xA5) and np.all(b[guard + total:] == 0xA5), "write outside the output"
    return statuses(st, table.n_chunks), b[guard:guard + total]


def test_decode_corrupt_streams_status_and_bounds():
    rng = np.random.default_rng(5)
    s, e = O.seqgen(99, 20000)
    # truncations of one block, each as its own 20000-byte chunk: all fail
    cuts = list(range(0, s.size, max(1, s.size // 300)))
    ot = O.Table(np.concatenate([s[:c] for c in cuts]), np.cumsum([0] + cuts).astype(np.uint64),
                 np.arange(len(cuts) + 1, dtype=np.uint64) * np.uint64(20000))
    st, _ = _guarded_decode(ot, ot.total)
    _, ost = O.decode_table(ot)
    assert np.all(st != 0) and np.all(ost != 0)
    # one flipped byte per block: the GPU reports OK exactly when the oracle
    # does, and chunks decoded OK hold the oracle's bytes
    blocks = []
    for k in range(300):
        c = s.copy()
        c[rng.integers(0, c.size)] ^= np.uint8(rng.integers(1, 256))
        blocks.append(c)
    ot = O.Table(np.concatenate(blocks), np.cumsum([0] + [b.size for b in blocks]).astype(np.uint64),
                 np.arange(len(blocks) + 1, dtype=np.uint64) * np.uint64(20000))
    st, got = _guarded_decode(ot, ot.total)
    oout, ost = O.decode_table(ot)
    assert np.array_equal(st == 0, ost == 0)
    for i in np.nonzero(ost == 0)[0]:
        assert np.array_equal(got[20000 * i:20000 * (i + 1)], oout[20000 * i:20000 * (i + 1)])


def test_decode_bad_table_entries():
    data = np.arange(300000, dtype=np.uint32).astype(np.uint8)
    ot = O.compress_table(data, synth.uniform_chunks(data.size, 32768))
    bad = O.Table(ot.comp, ot.comp_off.copy(), ot.dst_off.copy())
    bad.comp_off[3] = bad.comp_off[2] - np.uint64(1)
    bad.dst_off[6] += np.uint64(8)                       # misaligned chunk start
    st, got = _guarded_decode(bad, bad.total)
    _, ost = O.decode_table(bad)
    assert st[2] == lt.CHUNK_BAD_TABLE and st[6] == lt.CHUNK_BAD_TABLE
    assert st[0] == 0 and np.array_equal(got[:32768], data[:32768])
    assert np.all((st == 0) <= (ost == 0))


# --------------------------------------------------------- sequence index

def test_index_decodes_oracle_and_generated_streams():
    """Generator-built and oracle-compressed tables decode the same with the
    sequence index; packer tables the same without it."""
    rng = np.random.default_rng(17)
    for trial in range(4):
        n = int(rng.integers(1, 200))
        sizes = list(16 * rng.integers(0, 70000 // 16, n))
        sizes[-1] = int(rng.integers(0, 70000))
        t, e = _seq_table(rng.integers(0, 2**62, n), sizes)
        _decode_check(table_from_oracle(t, index=True), e, "seqgen indexed %d" % trial)
    a = synth.relu_4096x14336()
    _decode_check(table_from_oracle(O.compress_table(a.data, a.dst_off), index=True), a.data,
                  "relu_4096x14336 oracle, indexed")
    _decode_check(lt.ChunkTable.build(a.data, a.dst_off, DEV, index=False), a.data, "relu_4096x14336 packer, walked")


def _index_case(comp, comp_off, dst_off, data, seq_off, seq_pos, what, bad):
    n = comp_off.size - 1
    t = lt.ChunkTable.from_host(comp, comp_off, dst_off, DEV, max_dist=lt.SMALL_WINDOW)
    t.set_index(seq_off, seq_pos)
    st = status_tensor(n)
    out = lt.decode_lz4(t, status=st)
    s = statuses(st, n)
    got = out.cpu().numpy()
    for i in range(n):
        lo, hi = int(dst_off[i]), int(dst_off[i + 1])
        if i in bad:
            assert s[i] != 0, "%s: chunk %d decoded with a wrong index" % (what, i)
        else:
            assert s[i] == 0 and np.array_equal(got[lo:hi], data[lo:hi]), "%s: chunk %d" % (what, i)


def test_index_that_does_not_match_fails_its_chunk():
    """A listed position off by one, a sequence missing from or added to the
    list, a list that stops early, or one that runs past the entries fails
    that chunk alone; a chunk with no entries is walked without the index."""
    w = synth.int4_weight(256, 8192, 128, 23)
    packed = lt.pack_int4(w.codes)
    comp, comp_off = lt.compress_chunks(packed, w.dst_off, max_dist=lt.SMALL_WINDOW)
    so, sp = lt.index_chunks(comp, comp_off)
    case = lambda o, p, what, bad: _index_case(comp, comp_off, w.dst_off, packed, o, p, what, bad)
    case(so, sp, "exact", set())
    p = sp.copy()
    p[int(so[1]) + 5] += 1
    case(so, p, "moved by one", {1})
    k = int(so[2]) + 7
    o = so.copy()
    o[so > k] -= 1
    case(o, np.delete(sp, k), "one missing", {2})
    k = int(so[3]) + 3
    o = so.copy()
    o[so > k] += 1
    case(o, np.insert(sp, k + 1, sp[k] + (sp[k + 1] - sp[k]) // 2), "one added", {3})
    p = sp.copy()
    p[int(so[4])] = 1
    case(so, p, "first not at 0", {4})
    cut = (int(so[6]) - int(so[5])) // 2
    o = so.copy()
    o[6:] -= cut
    case(o, np.delete(sp, np.arange(int(so[6]) - cut, int(so[6]))), "stops early", {5})
    n7 = int(so[8]) - int(so[7])
    o = so.copy()
    o[8:] -= n7
    case(o, np.delete(sp, np.arange(int(so[7]), int(so[8]))), "no entries", set())
    o = so.copy()
    o[-1] += 1
    case(o, sp, "past the entries", {so.size - 2})


# ------------------------------------------------------------ fused paths

def _fused4(table, w, what):
    st = status_tensor(table.n_chunks)
    out = lt.fused_lz4_int4(table, t_u16(w.scales), t_i8(w.zp), (w.rows, w.cols), w.group, status=st)
    s = statuses(st, table.n_chunks)
    assert np.all(s == 0), "%s: statuses %s" % (what, np.unique(s))
    ref = O.dequant_int4(O.pack_int4(w.codes), w.scales, w.zp, w.group)
    assert_same(host_u16(out), ref, what)


def test_fused_int4_tiny_int4_both_compressors():
    w = synth.tiny_int4_1024()
    packed = lt.pack_int4(w.codes)
    _fused4(lt.ChunkTable.build(packed, w.dst_off, DEV), w, "tiny_int4_1024 packer")
    _fused4(table_from_oracle(O.compress_table(O.pack_int4(w.codes), w.dst_off)), w, "tiny_int4_1024 oracle")


def test_fused_int4_mlp_8192x28672_full():
    """The benchmark's workload: 8192x28672, group 128, packer streams, with
    the sequence index (the benchmark's table) and without it."""
    w = synth.mlp_int4_8192x28672()
    packed = lt.pack_int4(w.codes)
    _fused4(lt.ChunkTable.build(packed, w.dst_off, DEV), w, "mlp_int4_8192x28672 packer, indexed")
    _fused4(lt.ChunkTable.build(packed, w.dst_off, DEV, index=False), w, "mlp_int4_8192x28672 packer, walked")


def test_launch_order_mixed_chunks_and_partial_orders():
    """A table of 16/64/256 KiB chunks decoded in its launch order (largest
    first), fused and decode-only, equals the oracle; an order that leaves
    a chunk out and holds an entry past the last chunk decodes every listed
    chunk, skips the bad entry, and leaves the missing chunk's output and
    status untouched."""
    w = synth.int4_weight(1024, 8192, 128, 78, chunking="mixed")
    packed = lt.pack_int4(w.codes)
    tb = lt.ChunkTable.build(packed, w.dst_off, DEV)
    sizes = np.diff(w.dst_off.astype(np.int64))
    assert tb.order is not None and len(set(sizes[:-1].tolist())) == 3
    order = tb.order.cpu().numpy().view(np.uint32)
    assert np.all(np.diff(sizes[order]) <= 0)
    _fused4(tb, w, "mixed chunks, largest first")
    _decode_check(tb, packed, "mixed chunks decode-only, largest first")
    gone = int(order[1])
    partial = np.concatenate([order[order != gone], [tb.n_chunks + 7]]).astype(np.uint32)
    tb.order = torch.from_numpy(partial.view(np.int32)).to(DEV)
    st = status_tensor(tb.n_chunks)
    out = torch.full((w.rows * w.cols,), 3.0, dtype=torch.float16, device=DEV)
    lt.fused_lz4_int4(tb, t_u16(w.scales), t_i8(w.zp), (w.rows, w.cols), w.group, out=out, status=st)
    s = statuses(st, tb.n_chunks)
    assert s[gone] == -1 and np.all(np.delete(s, gone) == 0)
    got = host_u16(out)
    ref = O.dequant_int4(O.pack_int4(w.codes), w.scales, w.zp, w.group)
    e0, e1 = 2 * int(w.dst_off[gone]), 2 * int(w.dst_off[gone + 1])
    assert np.all(got[e0:e1] == np.float16(3.0).view(np.uint16))
    assert_same(np.concatenate([got[:e0], got[e1:]]), np.concatenate([ref[:e0], ref[e1:]]), "partial order")


def test_fused_int4_mlp_8192x28672_oracle_stream():
    """The 8192x28672 layer in full as the oracle's greedy compressor encodes
    it (64 KiB window, 4-byte minimum matches, no declared window), through
    the fused entry point with and without the sequence index."""
    w = synth.mlp_int4_8192x28672()
    ot = O.compress_table(O.pack_int4(w.codes), w.dst_off)
    _fused4(table_from_oracle(ot), w, "mlp_int4_8192x28672 oracle stream")
    _fused4(table_from_oracle(ot, index=True), w, "mlp_int4_8192x28672 oracle stream, indexed")


@pytest.mark.parametrize("rows,cols,group,chunk", [
    (64, 4096, 128, 48 * 1024),       # ragged chunks, several tiles
    (61, 1000, 8, 1040),               # chunk not a tile multiple, ragged tail
    (10, 36, 6, 16),                   # group splits lanes' codes (slow path)
    (7, 30, 10, 48),                   # tiny chunks, odd tail bytes
    (128, 8192, 8192, 65536),          # per-row groups
    (16, 4096, 16 * 4096, 65536),      # per-tensor group
    (512, 8192, 128, "mixed"),         # 16/64/256 KiB chunks (ring wrap)
    (1, 2, 2, 16),                     # one byte
])
def test_fused_int4_shapes(rows, cols, group, chunk):
    w = synth.int4_weight(rows, cols, group, rows * 7 + cols, chunking="mixed" if chunk == "mixed" else "64k")
    if chunk != "mixed":
        w.dst_off = synth.uniform_chunks(w.packed_bytes, chunk)
    packed = lt.pack_int4(w.codes)
    _fused4(lt.ChunkTable.build(packed, w.dst_off, DEV), w, "fused %dx%d g%d" % (rows, cols, group))
    w.zp = None
    _fused4(lt.ChunkTable.build(packed, w.dst_off, DEV), w, "fused no-zp %dx%d" % (rows, cols))


def test_fused_int4_generated_streams():
    """Arbitrary LZ4 structure (overlaps, far distances) through the fused path."""
    rng = np.random.default_rng(21)
    sizes = [int(v) for v in 16 * rng.integers(1, 5000, 40)] + [1000]
    t, e = _seq_table(rng.integers(0, 2**62, len(sizes)), sizes)
    n_codes = 2 * e.size
    rows, cols, group = 1, n_codes, 8
    scales = synth.fp16_bits(rng.uniform(-1, 1, n_codes // group))
    zp = rng.integers(-128, 128, n_codes // group).astype(np.int8)
    st = status_tensor(t.n)
    out = lt.fused_lz4_int4(table_from_oracle(t), t_u16(scales), t_i8(zp), (rows, cols), group, status=st)
    assert np.all(statuses(st, t.n) == 0)
    assert_same(host_u16(out), O.dequant_int4(e, scales, zp, group), "fused seqgen")


def test_fused_int4_short_window_big_chunks():
    """Fused INT4 with 256 KiB chunks in a short-window table (ring reuse)."""
    w = synth.int4_weight(512, 4096, 128, 41)
    packed = lt.pack_int4(w.codes)
    table = lt.ChunkTable.build(packed, synth.uniform_chunks(packed.size, 262144), DEV)
    _fused4(table, w, "short window, 256 KiB chunks")


def test_fused_int8_int8_8192():
    w = synth.int8_8192x8192()
    table = lt.ChunkTable.build(w.q.view(np.uint8), w.dst_off, DEV)
    st = status_tensor(table.n_chunks)
    out = lt.fused_lz4_int8(table, t_u16(w.scales), None, (w.rows, w.cols), w.group, status=st)
    assert np.all(statuses(st, table.n_chunks) == 0)
    assert_same(host_u16(out), O.dequant_int8(w.q, w.scales, None, w.group), "int8_8192x8192 fused int8")


def test_fused_int8_small_groups_zp():
    rng = np.random.default_rng(8)
    rows, cols, group = 300, 1000, 100
    q = rng.integers(-128, 128, rows * cols).astype(np.int8)
    q[rng.random(q.size) < 0.5] = 0
    scales = synth.fp16_bits(rng.uniform(-1, 1, rows * cols // group))
    zp = rng.integers(-128, 128, rows * cols // group).astype(np.int8)
    dst_off = synth.uniform_chunks(q.size, 4096 + 16)
    table = lt.ChunkTable.build(q.view(np.uint8), dst_off, DEV)
    st = status_tensor(table.n_chunks)
    out = lt.fused_lz4_int8(table, t_u16(scales), t_i8(zp), (rows, cols), group, status=st)
    assert np.all(statuses(st, table.n_chunks) == 0)
    assert_same(host_u16(out), O.dequant_int8(q, scales, zp, group), "fused int8 g100")


# ---------------------------------------------- corrupt blocks, fused modes

def _corrupt_blocks(comp, comp_off, rng, n_bad):
    """A copy of a table's blocks with n_bad of them damaged: truncated by a
    few bytes, one byte flipped, or a byte inserted.  Returns the new blocks,
    offsets and the damaged chunk indices."""
    n = comp_off.size - 1
    bad = sorted(rng.choice(n, size=n_bad, replace=False).tolist())
    blocks = [comp[int(comp_off[i]):int(comp_off[i + 1])].copy() for i in range(n)]
    for k, i in enumerate(bad):
        b = blocks[i]
        kind = k % 3
        if kind == 0:
            b = b[:max(0, b.size - 1 - int(rng.integers(0, 8)))]
        elif kind == 1:
            b[int(rng.integers(0, b.size))] ^= np.uint8(rng.integers(1, 256))
        else:
            b = np.insert(b, int(rng.integers(0, b.size)), np.uint8(rng.integers(0, 256)))
        blocks[i] = b
    off = np.concatenate([[0], np.cumsum([b.size for b in blocks])]).astype(np.uint64)
    return np.concatenate(blocks), off, bad


@pytest.mark.parametrize("mode", ["int4", "int8"])
def test_fused_corrupt_blocks_status_and_guards(mode):
    """Damaged blocks through the fused entry points, in an output buffer with
    guard bands on both sides: nothing outside the output is written; a chunk
    the oracle cannot decode fails; a chunk reported OK holds exactly the
    dequantized oracle bytes; undamaged chunks are exact.  Tables from the
    packer with its declared 4 KiB window, with and without the sequence
    index (built from the damaged blocks), and with no declared window (where
    a chunk is OK on the GPU exactly when it is for the oracle)."""
    rng = np.random.default_rng(61 if mode == "int4" else 62)
    if mode == "int4":
        w = synth.int4_weight(384, 8192, 128, 63)
        data = lt.pack_int4(w.codes)
        n_elem, per = w.rows * w.cols, 2
        scales, zp, group = w.scales, w.zp, w.group
    else:
        R, C = 256, 8192
        q = np.clip(np.rint(rng.standard_normal(R * C) * 32.0), -127, 127).astype(np.int8)
        q.reshape(R, C)[rng.choice(R, R // 2, replace=False)] = 0
        data = q.view(np.uint8)
        n_elem, per = R * C, 1
        scales, zp, group = synth.fp16_bits(rng.uniform(1e-3, 1e-2, size=R)), None, C
    dst_off = synth.uniform_chunks(data.size)
    guard = 4096
    for window in (lt.PACK_WINDOW, 0):
        comp, comp_off = lt.compress_chunks(data, dst_off, max_dist=window)
        bcomp, boff, bad = _corrupt_blocks(comp, comp_off, rng, 12)
        ot = O.Table(bcomp, boff, dst_off)
        odec, ost = O.decode_table(ot)
        for index in (True, False):
            table = lt.ChunkTable.from_host(bcomp, boff, dst_off, DEV, max_dist=window, index=index)
            buf = torch.full((n_elem + 2 * guard,), -1, dtype=torch.int16, device=DEV)
            out = buf[guard:guard + n_elem].view(torch.float16)
            st = status_tensor(table.n_chunks)
            if mode == "int4":
                lt.fused_lz4_int4(table, t_u16(scales), t_i8(zp), (n_elem // 8192, 8192), group, out=out, status=st)
            else:
                lt.fused_lz4_int8(table, t_u16(scales), None, (n_elem // 8192, 8192), group, out=out, status=st)
            s = statuses(st, table.n_chunks)
            b = host_u16(buf)
            what = "%s window %d index %s" % (mode, window, index)
            assert np.all(b[:guard] == 0xFFFF) and np.all(b[guard + n_elem:] == 0xFFFF), what + ": write outside"
            got = b[guard:guard + n_elem]
            assert np.all(s[ost != 0] != 0), what + ": a chunk the oracle rejects decoded OK"
            if window == 0:
                assert np.array_equal(s == 0, ost == 0), what
            if mode == "int4":
                ref = O.dequant_int4(odec, scales, zp, group, n_elem)
            else:
                ref = O.dequant_int8(odec.view(np.int8), scales, None, group)
            for i in range(table.n_chunks):
                lo, hi = per * int(dst_off[i]), per * int(dst_off[i + 1])
                if i not in bad:
                    assert s[i] == 0, (what, i, s[i])
                if s[i] == 0:
                    assert np.array_equal(got[lo:hi], ref[lo:hi]), (what, i)


# ------------------------------------------------------- bounded waits

@pytest.mark.parametrize("form", ["indexed", "walked", "full_window_bytes"])
def test_bounded_waits_fail_their_chunk_and_exit(form):
    """Every wait inside the decoder polls at most spin_limit times per wave;
    a wave that runs out fails its chunk with CHUNK_STALLED and every wave
    still leaves, so the kernel ends.  Forced from the host with tiny limits:
    the launch completes, statuses are OK or STALLED only, chunks reported
    OK hold the oracle's result, nothing outside the output is written; with
    the default limit every chunk decodes."""
    guard = 4096
    if form == "full_window_bytes":
        a = synth.activation(1024, 8192, 77)
        ot = O.compress_table(a.data, a.dst_off)          # no declared window: 64 KiB history
        data, n_out, per = a.data, a.data.size, 1
    else:
        w = synth.int4_weight(512, 28672, 128, 76)
        data = lt.pack_int4(w.codes)
        n_out, per = w.rows * w.cols, 2
        ref = O.dequant_int4(O.pack_int4(w.codes), w.scales, w.zp, w.group)
    for spin in (1, 3, 16, 256, 0):
        if form == "full_window_bytes":
            table = table_from_oracle(ot)
            buf = torch.full((n_out + 2 * guard,), 0x5A, dtype=torch.uint8, device=DEV)
        else:
            table = lt.ChunkTable.build(data, w.dst_off, DEV, index=(form == "indexed"))
            buf = torch.full((n_out + 2 * guard,), 0x5A5A, dtype=torch.int16, device=DEV)
        table.spin_limit = spin
        st = status_tensor(table.n_chunks)
        out = buf[guard:guard + n_out]
        if form == "full_window_bytes":
            lt.decode_lz4(table, out=out, status=st)
        else:
            lt.fused_lz4_int4(table, t_u16(w.scales), t_i8(w.zp), (w.rows, w.cols), w.group,
                              out=out.view(torch.float16), status=st)
        s = statuses(st, table.n_chunks)
        b = buf.cpu().numpy()
        what = "%s, spin_limit %d" % (form, spin)
        assert np.all(b[:guard] == b[0]) and np.all(b[guard + n_out:] == b[0]), what + ": write outside"
        assert set(np.unique(s)) <= {lt.CHUNK_OK, lt.CHUNK_STALLED}, (what, np.unique(s))
        if spin == 0:
            assert np.all(s == lt.CHUNK_OK), what
        if spin == 1 and form != "full_window_bytes":
            assert np.any(s == lt.CHUNK_STALLED), what + ": no wait gave up"
        got = b[guard:guard + n_out]
        expect = data if form == "full_window_bytes" else ref
        got = got if form == "full_window_bytes" else got.view(np.uint16)
        d = table.host_dst_off
        for i in np.nonzero(s == lt.CHUNK_OK)[0]:
            lo, hi = per * int(d[i]), per * int(d[i + 1])
            assert np.array_equal(got[lo:hi], expect[lo:hi]), (what, i)


# ------------------------------------------------ every table class, fused

def test_every_table_class_through_the_fused_kernels():
    """The fused calls pick a kernel per table: history class (declared 4 KiB
    window, or any distance), speculative build and progress priority
    (sequence-dense indexed tables, 3.5 or more sequences per KiB; tables
    without an index take the speculative build alone), and for INT4 the
    128-code group path or the general one.  Each combination, from the
    packer's parse and the greedy one, against the oracle (groups of 128,
    64 and 448 codes: the last two take the general path, 64 is dense even
    from the packer, 448 sparse); dense tables carry the
    most-sequences-first launch order."""
    seen = set()
    for group, seed in ((128, 4401), (64, 4402), (448, 4404)):
        w = synth.int4_weight(96, 28672, group, seed)
        packed = lt.pack_int4(w.codes)
        for greedy in (False, True):
            for md in (lt.PACK_WINDOW, 0):
                for index in (True, False):
                    tb = lt.ChunkTable.build(packed, w.dst_off, DEV, max_dist=md, greedy=greedy, index=index)
                    dense = index and tb.n_seq * 2048 >= 7 * tb.total_bytes
                    assert (tb.order is not None) == dense
                    seen.add((group, md, dense, index))
                    _fused4(tb, w, "g%d %s window %d %s" % (group, "greedy" if greedy else "packer", md,
                                                          "indexed" if index else "walked"))
    # both history classes met dense and sparse indexed tables, on both INT4 paths
    assert {(g == 128, md, d) for g, md, d, i in seen if i} == {(p, md, d) for p in (False, True)
                                                               for md in (lt.PACK_WINDOW, 0) for d in (False, True)}
    rng = np.random.default_rng(4403)
    rows, cols = 64, 8192
    q = rng.integers(-100, 100, rows * cols).astype(np.int8)
    q[rng.random(q.size) < 0.7] = 0                  # short runs of zeros: a dense table
    scales = synth.fp16_bits(rng.uniform(1e-3, 1e-2, rows))
    dst_off = synth.uniform_chunks(q.size)
    for md in (lt.PACK_WINDOW, 0):
        for greedy in (False, True):
            tb = lt.ChunkTable.build(q.view(np.uint8), dst_off, DEV, max_dist=md, greedy=greedy)
            st = status_tensor(tb.n_chunks)
            out = lt.fused_lz4_int8(tb, t_u16(scales), None, (rows, cols), cols, status=st)
            assert np.all(statuses(st, tb.n_chunks) == 0)
            assert_same(host_u16(out), O.dequant_int8(q, scales, None, cols),
                        "int8 window %d %s, %.1f sequences per KiB" % (md, "greedy" if greedy else "packer",
                                                                       tb.n_seq * 1024 / tb.total_bytes))
