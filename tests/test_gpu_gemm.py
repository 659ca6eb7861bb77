"""Decode fused with a batched product on the matrix cores: Y = X W^T with W
decoded and dequantized tile by tile and never stored (the pages' decode
plus GEMM benchmark; the roadmap's decoded tensor used in a matmul, Phase
4.1).  The table holds W's INT4 codes in 16 x 128 tiles (pack_int4_tiles).

Each fp16 product is exact in fp32 and the sums are fp32, so Y is compared
with the oracle's fp64 product within 128 fp32 unit roundoffs of
sum |w x| per element: an MFMA sums 32 products, a builder accumulates at
most a few dozen MFMA results per chunk, and the second pass adds 6 slots
per chunk over the chunks of a row block.  A one-hot X picks single columns
of W, which come out exact.  The summation order is fixed, so two calls
give identical bits.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import weight_dequantization_amd as lt

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
U = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield
    torch.cuda.synchronize()


def _setup(w, rows, cols, tiles_per_chunk=56, window=lt.PACK_WINDOW, index=True, checksum=False, zp=True):
    codes = w.codes.reshape(w.rows, w.cols)[:rows, :cols]
    data = lt.pack_int4_tiles(codes, rows, cols)
    dst_off = lt.gemm_chunks(rows, cols, tiles_per_chunk)
    comp, comp_off = lt.compress_chunks(data, dst_off, max_dist=window)
    tb = lt.ChunkTable.from_host(comp, comp_off, dst_off, DEV, window, index=index, checksum=checksum)
    ng = rows * cols // w.group
    sc = w.scales[:ng] if cols == w.cols else None
    z = (w.zp[:ng] if cols == w.cols else None) if zp else None
    return tb, O.Table(comp, comp_off, dst_off), sc, z


def _gemm(tb, sc, z, rows, cols, group, x):
    st = torch.full((tb.n_chunks,), -1, dtype=torch.int32, device=DEV)
    y = lt.fused_lz4_int4_gemm(tb, torch.from_numpy(sc.view(np.int16)).to(DEV),
                               None if z is None else torch.from_numpy(z).to(DEV), (rows, cols), group,
                               torch.from_numpy(x.view(np.int16)).to(DEV), status=st)
    torch.cuda.synchronize()
    return y.cpu().numpy(), st.cpu().numpy()


def _bound(ot, sc, z, group, rows, cols, x):
    """|Y| of the oracle's product with |W| and |X|: sum |w x| per element."""
    ax = x.copy() & np.uint16(0x7FFF)
    ref, st = O.gemm_int4_tiled(ot, sc, z, group, rows, cols, x)
    data, _ = O.decode_table(ot)
    r = np.arange(rows)[:, None]
    c = np.arange(cols)[None, :]
    byte = ((r // 16) * (cols // 128) + c // 128) * 1024 + (r % 16) * 64 + (c % 128) // 2
    codes = ((data[byte] >> (4 * (c % 2))) & 15).astype(np.uint8)
    W = O.f64_from_f16(O.dequant_int4(O.pack_int4(codes.ravel()), sc, z, group)).reshape(rows, cols)
    mag = O.f64_from_f16(ax).reshape(-1, cols) @ np.abs(W).T
    return ref, mag, st


def _check(y, ref, mag, what):
    err = np.abs(y.astype(np.float64) - ref)
    bad = np.nonzero(err > 128 * U * mag + 1e-30)
    assert bad[0].size == 0, "%s: %d elements off, worst %g of bound %g" % (
        what, bad[0].size, err[bad].max(), (128 * U * mag)[bad].max())


def test_gemm_1024_rows_of_the_layer():
    """1024 rows of the 8192 x 28672 layer (its codes, scales and zero
    points), batch 16 and 32, indexed and walked tables, checksums on."""
    w = synth.mlp_int4_small(rows=1024)
    rng = np.random.default_rng(5)
    for index in (True, False):
        tb, ot, sc, z = _setup(w, 1024, w.cols, index=index, checksum=True)
        for batch in (16, 32):
            x = O.f16_from_f64(rng.standard_normal((batch, w.cols))).reshape(batch, w.cols)
            y, st = _gemm(tb, sc, z, 1024, w.cols, w.group, x)
            assert np.all(st == 0), np.unique(st)
            ref, mag, _ = _bound(ot, sc, z, w.group, 1024, w.cols, x)
            _check(y, ref, mag, "1024 rows, batch %d, index %s" % (batch, index))


def test_gemm_full_layer_sampled_and_deterministic():
    """The whole 8192 x 28672 layer at batch 16 (2048 chunks of 56 tiles):
    32 sampled 16-row blocks against the oracle on those blocks' own tiles;
    a second call gives the same bits."""
    w = synth.mlp_int4_8192x28672()
    rows, cols = w.rows, w.cols
    tb, ot, sc, z = _setup(w, rows, cols)
    rng = np.random.default_rng(6)
    x = O.f16_from_f64(rng.standard_normal((16, cols))).reshape(16, cols)
    y, st = _gemm(tb, sc, z, rows, cols, w.group, x)
    assert np.all(st == 0)
    y2, _ = _gemm(tb, sc, z, rows, cols, w.group, x)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    comp, comp_off, dst_off = ot.comp, ot.comp_off, ot.dst_off
    per_block = (cols // 128 + 55) // 56
    gpr = cols // w.group   # groups per row
    for rb in rng.choice(rows // 16, 32, replace=False):
        c0, c1 = rb * per_block, (rb + 1) * per_block
        a, b = int(comp_off[c0]), int(comp_off[c1])
        sub = O.Table(comp[a:b], comp_off[c0:c1 + 1] - comp_off[c0], dst_off[c0:c1 + 1] - dst_off[c0])
        g0, g1 = 16 * rb * gpr, 16 * (rb + 1) * gpr
        ref, mag, s = _bound(sub, sc[g0:g1], z[g0:g1], w.group, 16, cols, x)
        assert np.all(s == 0)
        _check(y[:, 16 * rb:16 * rb + 16], ref, mag, "row block %d" % rb)


@pytest.mark.parametrize("rows,cols,group,tpc,zp,window", [
    (16, 128, 128, 1, True, lt.PACK_WINDOW), (48, 384, 128, 1, False, 0), (48, 512, 256, 2, True, 0),
    (64, 1024, 1024, 3, True, lt.PACK_WINDOW), (32, 2048, 128, 16, False, lt.PACK_WINDOW)])
def test_gemm_shapes_groups_and_chunkings(rows, cols, group, tpc, zp, window):
    w = synth.int4_weight(rows, cols, group, 70 + rows + tpc)
    tb, ot, sc, z = _setup(w, rows, cols, tiles_per_chunk=tpc, window=window, zp=zp)
    rng = np.random.default_rng(rows + cols)
    for batch in (16, 32):
        x = O.f16_from_f64(rng.standard_normal((batch, cols)) * 3).reshape(batch, cols)
        y, st = _gemm(tb, sc, z, rows, cols, group, x)
        assert np.all(st == 0)
        ref, mag, _ = _bound(ot, sc, z, group, rows, cols, x)
        _check(y, ref, mag, "%dx%d group %d" % (rows, cols, group))


def test_gemm_one_hot_columns_exact():
    """X with one 1.0 per vector picks single columns of W: exact."""
    w = synth.int4_weight(64, 512, 128, 90)
    tb, ot, sc, z = _setup(w, 64, 512, tiles_per_chunk=2)
    cols_picked = [0, 1, 7, 8, 127, 128, 200, 255, 256, 300, 383, 384, 400, 450, 510, 511]
    x = np.zeros((16, 512), np.uint16)
    for b, j in enumerate(cols_picked):
        x[b, j] = 0x3C00
    y, st = _gemm(tb, sc, z, 64, 512, 128, x)
    assert np.all(st == 0)
    ref, _, _ = _bound(ot, sc, z, 128, 64, 512, x)
    assert np.array_equal(y.astype(np.float64), ref)


def test_gemm_chunk_spanning_two_row_blocks_fails():
    """A chunk that holds tiles of two 16-row blocks is a bad table entry."""
    w = synth.int4_weight(32, 256, 128, 91)
    data = lt.pack_int4_tiles(w.codes.reshape(32, 256), 32, 256)
    dst_off = np.array([0, 1024, 3072, 4096], np.uint64)   # chunk 1 holds tiles 1 and 2 (blocks 0 and 1)
    comp, comp_off = lt.compress_chunks(data, dst_off)
    tb = lt.ChunkTable.from_host(comp, comp_off, dst_off, DEV, 0, index=True)
    x = np.zeros((16, 256), np.uint16)
    _, st = _gemm(tb, w.scales, w.zp, 32, 256, 128, x)
    assert st[1] == lt.CHUNK_BAD_TABLE and st[0] == 0 and st[2] == 0
