"""Chunk-range (partial) decode: chunks first .. first+count-1 of a resident
table into a buffer that holds only their output (page "Openai/692db884-...
(section 28)", decoding only the part an operation needs).  Each range's
output must equal the same part of the oracle's full result, bit for bit,
and a range whose bounds do not match the table must fail its end chunks and
write nothing outside the buffer.
"""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle as O
import synth
import weight_dequantization_amd as lt

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


def host_u16(t):
    torch.cuda.synchronize()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).ravel()


def assert_same(got, ref, what):
    assert got.size == ref.size, (what, got.size, ref.size)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, "%s: %d of %d differ, first at %d: got %#x want %#x" % (
        what, bad.size, ref.size, bad[0], got[bad[0]], ref[bad[0]])


def status_tensor(n):
    return torch.full((max(n, 1),), -1, dtype=torch.int32, device=DEV)


def statuses(st, n):
    torch.cuda.synchronize()
    return st[:n].cpu().numpy()


def _ranges(n):
    return [(0, 1), (n // 3, min(257, n - n // 3)), (n - 1, 1), (0, n), (n // 2, 0)]


def _int4_ranges(table, w, ref, what):
    d = table.host_dst_off
    for first, count in _ranges(table.n_chunks):
        st = status_tensor(count)
        out = lt.fused_lz4_int4_range(table, t_u16(w.scales), t_i8(w.zp), (w.rows, w.cols), w.group,
                                      first, count, status=st)
        assert np.all(statuses(st, count) == 0), (what, first, count)
        if count:
            lo, hi = 2 * int(d[first]), 2 * int(d[first + count])
            assert_same(host_u16(out), ref[lo:hi], "%s chunks %d+%d" % (what, first, count))


def test_int4_ranges_mlp_8192x28672_full():
    """The 8192x28672 layer: single chunks at both ends, a 257-chunk middle
    range, the whole table; indexed and walked."""
    w = synth.mlp_int4_8192x28672()
    packed = lt.pack_int4(w.codes)
    ref = O.dequant_int4(O.pack_int4(w.codes), w.scales, w.zp, w.group)
    for index in (True, False):
        print("mlp_int4_8192x28672 index=%s" % index, flush=True)
        _int4_ranges(lt.ChunkTable.build(packed, w.dst_off, DEV, index=index), w, ref, "mlp_int4_8192x28672 index=%s" % index)


def test_int4_ranges_mixed_chunks_oracle_stream():
    """Mixed 16/64/256 KiB chunks with a ragged last chunk, from the oracle's
    compressor (whole match window), group 64."""
    w = synth.int4_weight(640, 8192, 64, 51, chunking="mixed")
    ot = O.compress_table(O.pack_int4(w.codes), w.dst_off)
    ref = O.dequant_int4(O.pack_int4(w.codes), w.scales, w.zp, w.group)
    for index in (False, True):
        t = lt.ChunkTable.from_host(ot.comp, ot.comp_off, ot.dst_off, DEV, index=index)
        _int4_ranges(t, w, ref, "mixed index=%s" % index)


def test_int8_ranges_int8_8192():
    w = synth.int8_8192x8192()
    table = lt.ChunkTable.build(w.q.view(np.uint8), w.dst_off, DEV)
    ref = O.dequant_int8(w.q, w.scales, None, w.group)
    d = table.host_dst_off
    for first, count in _ranges(table.n_chunks):
        st = status_tensor(count)
        out = lt.fused_lz4_int8_range(table, t_u16(w.scales), None, (w.rows, w.cols), w.group, first, count,
                                      status=st)
        assert np.all(statuses(st, count) == 0), (first, count)
        if count:
            assert_same(host_u16(out), ref[int(d[first]):int(d[first + count])], "int8_8192x8192 %d+%d" % (first, count))


def test_decode_ranges_relu_4096x14336_with_guards():
    """Bytes mode on the activation workload (random-byte, 0xAB-run and
    sparse chunks): each range lands at offset 0 of its buffer and nothing
    is written past either end."""
    a = synth.relu_4096x14336()
    table = lt.ChunkTable.build(a.data, a.dst_off, DEV)
    d = table.host_dst_off
    guard = 4096
    for first, count in _ranges(table.n_chunks):
        lo, hi = int(d[first]), int(d[first + count])
        buf = torch.full((hi - lo + 2 * guard,), 0xA5, dtype=torch.uint8, device=DEV)
        st = status_tensor(count)
        lt.decode_lz4_range(table, first, count, out=buf[guard:guard + max(hi - lo, 1)], status=st)
        assert np.all(statuses(st, count) == 0), (first, count)
        b = buf.cpu().numpy()
        assert np.all(b[:guard] == 0xA5) and np.all(b[guard + hi - lo:] == 0xA5), (first, count)
        assert np.array_equal(b[guard:guard + hi - lo], a.data[lo:hi]), (first, count)


def test_range_bounds_that_do_not_match_fail_their_chunks():
    """dst_first or dst_last off by one 16-byte step: the chunk at that end
    reports LT_CHUNK_BAD_TABLE, the others decode as usual, and the buffer's
    guard bands stay untouched."""
    data = np.arange(1 << 20, dtype=np.uint32).astype(np.uint8)
    dst_off = synth.uniform_chunks(data.size, 65536)
    table = lt.ChunkTable.build(data, dst_off, DEV)
    L = lt.lib()
    first, count = 3, 6
    lo, hi = int(dst_off[first]), int(dst_off[first + count])
    guard = 4096
    for dlo, dhi, bad in ((16, 0, 0), (0, -16, count - 1), (-16, 0, 0), (0, 16, count - 1)):
        buf = torch.full((hi - lo + 2 * guard,), 0xA5, dtype=torch.uint8, device=DEV)
        st = status_tensor(count)
        t = table.as_c()
        r = L.lt_decode_lz4_range(C.byref(t), first, count, lo + dlo, hi + dhi,
                                  C.c_void_p(buf[guard:].data_ptr()), C.c_void_p(st.data_ptr()),
                                  C.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert r == lt.LT_OK
        s = statuses(st, count)
        want = np.zeros(count, np.int32)
        want[bad] = lt.CHUNK_BAD_TABLE
        assert np.array_equal(s, want), (dlo, dhi, s)
        b = buf.cpu().numpy()
        assert np.all(b[:guard] == 0xA5) and np.all(b[guard + hi - lo - min(dlo, 0) + max(dhi, 0):] == 0xA5)
        for k in range(count):
            if k != bad:
                a0, a1 = int(dst_off[first + k]), int(dst_off[first + k + 1])
                assert np.array_equal(b[guard + a0 - lo - dlo:guard + a1 - lo - dlo], data[a0:a1]), (dlo, dhi, k)
