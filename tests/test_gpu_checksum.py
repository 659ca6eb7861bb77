"""Checksums verified inside the decode (a table's xxh field): each chunk's
compressed bytes are hashed (XXH3-64) as the decoder stages them, and a
chunk whose hash differs from the stored value fails with
LT_CHUNK_CHECKSUM whatever its decode gave (the container check of "GPU
Compression Pipeline - TDD Roadmap", Phase 6.1, without a second pass over
HBM).  Stored values come from the host packer, which the CPU tests pin to
the oracle's XXH3 and to the xxhash package."""
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


def statuses(st, n):
    torch.cuda.synchronize()
    return st[:n].cpu().numpy()


def host_u16(t):
    torch.cuda.synchronize()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).ravel()


def _fused(tb, w, out=None):
    st = torch.full((tb.n_chunks,), -1, dtype=torch.int32, device=DEV)
    out = lt.fused_lz4_int4(tb, torch.from_numpy(w.scales.view(np.int16)).to(DEV), torch.from_numpy(w.zp).to(DEV),
                            (w.rows, w.cols), w.group, out=out, status=st)
    return statuses(st, tb.n_chunks), host_u16(out)


def test_checked_layer_8192x28672():
    """The benchmark layer with stored checksums: every chunk verifies and
    the output equals the oracle's, indexed and walked."""
    w = synth.mlp_int4_8192x28672()
    packed = lt.pack_int4(w.codes)
    ref = O.dequant_int4(O.pack_int4(w.codes), w.scales, w.zp, w.group)
    for index in (True, False):
        tb = lt.ChunkTable.build(packed, w.dst_off, DEV, index=index, checksum=True)
        assert tb.xxh is not None
        s, got = _fused(tb, w)
        assert np.all(s == 0), np.unique(s)
        assert np.array_equal(got, ref)


def _chunk_bytes(tb):
    return tb.comp.cpu().numpy(), tb.comp_off.cpu().numpy().view(np.uint64)


@pytest.mark.parametrize("mode", ["bytes", "int4", "int8"])
@pytest.mark.parametrize("window", [lt.PACK_WINDOW, 0])
def test_changed_bytes_fail_exactly_their_chunks(mode, window):
    """One changed compressed byte in each of several chunks (anywhere: in a
    literal, so the decode still succeeds, or in a token, offset or length)
    fails exactly those chunks with LT_CHUNK_CHECKSUM; a wrong stored value
    for intact bytes does too; every other chunk decodes to the oracle's
    output."""
    rng = np.random.default_rng({"bytes": 1, "int4": 2, "int8": 3}[mode] * 10 + (window != 0))
    if mode == "int8":
        q = np.clip(np.rint(rng.standard_normal(256 * 8192) * 32), -127, 127).astype(np.int8)
        q[:8192 * 8] = 0
        data = q.view(np.uint8)
        rows, cols, group = 256, 8192, 8192
        scales = synth.fp16_bits(rng.uniform(1e-3, 1e-2, 256))
        dst_off = synth.uniform_chunks(data.size)
    elif mode == "int4":
        w = synth.int4_weight(1024, 8192, 128, 41, chunking="mixed")
        data = lt.pack_int4(w.codes)
        dst_off = w.dst_off
    else:
        a = synth.activation(256, 8192, 42)
        data, dst_off = a.data, a.dst_off
    comp, comp_off = lt.compress_chunks(data, dst_off, max_dist=window)
    n = comp_off.size - 1
    bad = np.sort(rng.choice(n, min(6, n - 1), replace=False))
    comp2 = comp.copy()
    for i in bad[:-1]:
        a_, b_ = int(comp_off[i]), int(comp_off[i + 1])
        comp2[int(rng.integers(a_, b_))] ^= np.uint8(rng.integers(1, 256))
    tb = lt.ChunkTable.from_host(comp2, comp_off, dst_off, DEV, window, index=True, checksum=False)
    xxh = lt.checksum_chunks(comp, comp_off)            # the values of the intact bytes
    xxh[bad[-1]] ^= np.uint64(1 << 40)                  # and one wrong stored value
    tb.xxh = torch.from_numpy(xxh.view(np.int64)).to(DEV)
    st = torch.full((n,), -1, dtype=torch.int32, device=DEV)
    if mode == "bytes":
        out = lt.decode_lz4(tb, status=st)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        ref = data
        span = lambda i: (int(dst_off[i]), int(dst_off[i + 1]))
    elif mode == "int4":
        out = lt.fused_lz4_int4(tb, torch.from_numpy(w.scales.view(np.int16)).to(DEV),
                                torch.from_numpy(w.zp).to(DEV), (w.rows, w.cols), w.group, status=st)
        got = host_u16(out)
        ref = O.dequant_int4(O.pack_int4(w.codes), w.scales, w.zp, w.group)
        span = lambda i: (2 * int(dst_off[i]), 2 * int(dst_off[i + 1]))
    else:
        out = lt.fused_lz4_int8(tb, torch.from_numpy(scales.view(np.int16)).to(DEV), None, (rows, cols), group,
                                status=st)
        got = host_u16(out)
        ref = O.dequant_int8(q, scales, None, group)
        span = lambda i: (int(dst_off[i]), int(dst_off[i + 1]))
    s = statuses(st, n)
    assert np.array_equal(np.nonzero(s)[0], bad), (s[bad], np.nonzero(s)[0])
    assert np.all(s[bad] == lt.CHUNK_CHECKSUM), s[bad]
    keep = np.ones(got.size, bool)
    for i in bad:
        a_, b_ = span(i)
        keep[a_:b_] = False
    assert np.array_equal(got[keep], ref[keep])


def _ext(v):
    """Bytes of a length field's extension for a nibble value v >= 15."""
    return [255] * ((v - 15) // 255) + [(v - 15) % 255]


def _block_of_length(c, rng):
    """A valid LZ4 block of exactly c compressed bytes (c >= 16) whose decoded
    size is a multiple of 16: A literals, one match of M bytes reading the
    last (up to 64) literals, then 5 final literals; A and M are searched for.  Returns the
    block and its decoded size."""
    for A in range(1, c):
        for M in range(7, 400):
            if (A + M + 5) % 16:
                continue
            tok = [(min(A, 15) << 4) | min(M - 4, 15)]
            d = min(A, 64)   # the match reads the last literals (inside any declared window)
            body = (_ext(A) if A >= 15 else []) + [0] * A + [d, 0] + (_ext(M - 4) if M - 4 >= 15 else [])
            if len(tok) + len(body) + 1 + 5 != c:
                continue
            lits = rng.integers(0, 256, A, dtype=np.uint8)
            blk = np.array(tok + (_ext(A) if A >= 15 else []) + list(lits) + [d, 0] +
                           (_ext(M - 4) if M - 4 >= 15 else []) + [5 << 4] + list(rng.integers(0, 256, 5)),
                           np.uint8)
            assert blk.size == c
            return blk, A + M + 5
    raise AssertionError(c)


@pytest.mark.parametrize("window,index", [(lt.PACK_WINDOW, True), (lt.PACK_WINDOW, False), (0, True), (0, False)])
def test_every_hash_length_class(window, index):
    """Chunks whose compressed lengths fall in every length class of the hash
    (1 byte: an empty chunk; 6: a last chunk of 5 literals; 10-11: runs of
    zeros; 16-128; 129-240; the block form, including lengths one short of,
    equal to and one past whole 1 KiB blocks, and one past a block plus a
    stripe), verified in decode-only mode; with every stored value off by
    one bit, every chunk fails."""
    rng = np.random.default_rng(50 + window + index)
    blocks = [(O.lz4_compress(np.zeros(n, np.uint8)), n) for n in (0, 32, 256)]
    for c in (16, 17, 64, 128, 129, 200, 240, 241, 242, 300, 1023, 1024, 1025, 1087, 1088, 1089, 2047, 2048,
              2049, 3000, 4096, 9000):
        blocks.append(_block_of_length(c, rng))
    blocks.append((O.lz4_store(rng.integers(0, 256, 5, dtype=np.uint8)), 5))   # the last chunk: 5 bytes
    outs = []
    for b, n in blocks:
        st, d, _ = O.lz4_decode(b, n)
        assert st == O.OK
        outs.append(d)
    blocks = [b for b, _ in blocks]
    for d in outs[:-1]:
        assert d.size % 16 == 0
    comp = np.concatenate(blocks)
    comp_off = np.concatenate([[0], np.cumsum([b.size for b in blocks])]).astype(np.uint64)
    dst_off = np.concatenate([[0], np.cumsum([d.size for d in outs])]).astype(np.uint64)
    data = np.concatenate(outs)
    clen = np.diff(comp_off.astype(np.int64))
    for lo, hi in [(1, 3), (4, 8), (9, 16), (17, 128), (129, 240), (241, 1 << 30)]:
        assert np.any((clen >= lo) & (clen <= hi)), (lo, hi, clen)
    tb = lt.ChunkTable.from_host(comp, comp_off, dst_off, DEV, window, index=index, checksum=True)
    st = torch.full((tb.n_chunks,), -1, dtype=torch.int32, device=DEV)
    out = lt.decode_lz4(tb, status=st)
    s = statuses(st, tb.n_chunks)
    assert np.all(s == 0), (s, clen)
    assert np.array_equal(out.cpu().numpy(), data)
    tb.xxh ^= 1
    st.fill_(-1)
    lt.decode_lz4(tb, status=st)
    assert np.all(statuses(st, tb.n_chunks) == lt.CHUNK_CHECKSUM)


def test_streamed_and_range_calls_check_their_chunks():
    """The streamed entry point (checksums copied with the offsets) and a
    chunk-range call check the chunks they decode."""
    w = synth.mlp_int4_small(rows=512)
    packed = lt.pack_int4(w.codes)
    comp, comp_off = lt.compress_chunks(packed, w.dst_off, max_dist=lt.PACK_WINDOW)
    n = comp_off.size - 1
    bad = [3, 17, n - 2]
    comp2 = comp.copy()
    for i in bad:
        comp2[int(comp_off[i]) + 40] ^= 0x5A
    xxh = lt.checksum_chunks(comp, comp_off)
    ht = lt.ChunkTable.from_host(comp2, comp_off, w.dst_off, "cpu", lt.PACK_WINDOW, index=True, pin=True)
    ht.xxh = torch.from_numpy(xxh.view(np.int64)).pin_memory()
    sc = torch.from_numpy(w.scales.view(np.int16)).to(DEV)
    zp = torch.from_numpy(w.zp).to(DEV)
    st = torch.full((n,), -1, dtype=torch.int32, device=DEV)
    out = lt.stream_fused_lz4_int4(ht, sc, zp, (w.rows, w.cols), w.group, status=st)
    s = statuses(st, n)
    assert np.array_equal(np.nonzero(s)[0], bad) and np.all(s[bad] == lt.CHUNK_CHECKSUM)
    ref = O.dequant_int4(O.pack_int4(w.codes), w.scales, w.zp, w.group)
    got = host_u16(out)
    good = [i for i in range(n) if i not in bad]
    for i in good[:5] + good[-5:]:
        a_, b_ = 2 * int(w.dst_off[i]), 2 * int(w.dst_off[i + 1])
        assert np.array_equal(got[a_:b_], ref[a_:b_])
    dt = lt.ChunkTable.from_host(comp2, comp_off, w.dst_off, DEV, lt.PACK_WINDOW, index=True)
    dt.xxh = torch.from_numpy(xxh.view(np.int64)).to(DEV)
    st2 = torch.full((20,), -1, dtype=torch.int32, device=DEV)
    lt.fused_lz4_int4_range(dt, sc, zp, (w.rows, w.cols), w.group, 10, 20, status=st2)
    s2 = statuses(st2, 20)
    assert np.array_equal(np.nonzero(s2)[0], [17 - 10]) and s2[7] == lt.CHUNK_CHECKSUM


def test_gemv_checks_too():
    """The fused matrix-vector mode runs the same decoder: a changed byte
    fails its chunk with LT_CHUNK_CHECKSUM."""
    w = synth.mlp_int4_small(rows=256)
    packed = lt.pack_int4(w.codes)
    comp, comp_off = lt.compress_chunks(packed, w.dst_off, max_dist=lt.PACK_WINDOW)
    xxh = lt.checksum_chunks(comp, comp_off)
    comp[int(comp_off[5]) + 100] ^= 1
    tb = lt.ChunkTable.from_host(comp, comp_off, w.dst_off, DEV, lt.PACK_WINDOW, index=True)
    tb.xxh = torch.from_numpy(xxh.view(np.int64)).to(DEV)
    x = torch.randn(w.cols, dtype=torch.float16, device=DEV)
    st = torch.full((tb.n_chunks,), -1, dtype=torch.int32, device=DEV)
    lt.fused_lz4_int4_gemv(tb, torch.from_numpy(w.scales.view(np.int16)).to(DEV), torch.from_numpy(w.zp).to(DEV),
                           (w.rows, w.cols), w.group, x, status=st)
    s = statuses(st, tb.n_chunks)
    assert np.array_equal(np.nonzero(s)[0], [5]) and s[5] == lt.CHUNK_CHECKSUM
