"""Pins of the oracle's batched product with a matrix stored in the GEMM tile
layout (decompress, then multiply: the pages' decode-plus-GEMM benchmark,
and the roadmap's decoded tensor used in a matmul, Phase 4.1).

* brute force: on a small table every Y[b, r] equals a Python-loop sum of
  w[r, c] * x[b, c] over the fp16 weights, each code found by walking the
  tiles one by one (not by the oracle's index formula);
* the same weights in the ordinary row-major layout through the GEMV oracle
  (pinned on its own) give the same Y row by row;
* a one-hot x picks out one column of W exactly.
"""
import numpy as np

import oracle as O
import synth


def _tiled(rows, cols, group, seed, zp=True):
    w = synth.int4_weight(rows, cols, group, seed)
    codes = w.codes.reshape(rows, cols)
    stream = bytearray()
    for rb in range(rows // 16):                 # tiles one by one
        for kc in range(cols // 128):
            for rr in range(16):
                row = codes[16 * rb + rr, 128 * kc:128 * kc + 128]
                stream += bytes(int(row[2 * i]) | (int(row[2 * i + 1]) << 4) for i in range(64))
    data = np.frombuffer(bytes(stream), np.uint8)
    dst_off = np.arange(0, data.size + 1, 4096, dtype=np.uint64)
    if dst_off[-1] != data.size:
        dst_off = np.append(dst_off, np.uint64(data.size))
    t = O.compress_table(data, dst_off)
    return w, t, (w.zp if zp else None)


def test_brute_force_small():
    w, t, zp = _tiled(32, 256, 128, 11)
    rng = np.random.default_rng(1)
    x = O.f16_from_f64(rng.standard_normal((3, w.cols)))
    y, st = O.gemm_int4_tiled(t, w.scales, zp, w.group, w.rows, w.cols, x)
    assert np.all(st == O.OK)
    W = O.f64_from_f16(O.dequant_int4(O.pack_int4(w.codes), w.scales, zp, w.group)).reshape(w.rows, w.cols)
    xd = O.f64_from_f16(x).reshape(3, w.cols)
    for b in range(3):
        for r in range(w.rows):
            s = 0.0
            for c in range(w.cols):
                s += float(W[r, c]) * float(xd[b, c])
            assert abs(y[b, r] - s) <= 1e-9 * max(1.0, np.abs(W[r] * xd[b]).sum()), (b, r)


def test_agrees_with_the_gemv_oracle_row_by_row():
    w, t, zp = _tiled(48, 512, 256, 12, zp=False)
    rng = np.random.default_rng(2)
    x = O.f16_from_f64(rng.standard_normal((4, w.cols)))
    y, st = O.gemm_int4_tiled(t, w.scales, zp, w.group, w.rows, w.cols, x)
    rt = O.compress_table(O.pack_int4(w.codes), np.array([0, w.rows * w.cols // 2], np.uint64))
    for b in range(4):
        yv, _ = O.gemv_int4(rt, w.scales, zp, w.group, w.rows, w.cols, x.reshape(4, w.cols)[b])
        assert np.array_equal(y[b], yv), b


def test_one_hot_picks_a_column():
    w, t, zp = _tiled(16, 384, 128, 13)
    W = O.f64_from_f16(O.dequant_int4(O.pack_int4(w.codes), w.scales, zp, w.group)).reshape(w.rows, w.cols)
    x = np.zeros((4, w.cols), np.uint16)
    for b, j in enumerate((0, 127, 128, 383)):
        x[b, j] = 0x3C00   # 1.0
    y, _ = O.gemm_int4_tiled(t, w.scales, zp, w.group, w.rows, w.cols, x)
    for b, j in enumerate((0, 127, 128, 383)):
        assert np.array_equal(y[b], W[:, j])
