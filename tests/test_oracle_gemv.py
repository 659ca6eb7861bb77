"""Pins of the oracle's matrix-vector product with the dequantized matrix
(decompress, then multiply: the pages' decode-plus-GEMM benchmarks).

* brute force: on small tables every y[r] equals a Python-loop sum of
  w[r, c] * x[c] over the fp16 weights the fused oracle gives;
* closed form: a one-hot x picks out one column of the matrix exactly;
* linearity in x.
"""
import numpy as np

import oracle as O
import synth


def _table(rows, cols, group, seed):
    w = synth.int4_weight(rows, cols, group, seed)
    t = O.compress_table(O.pack_int4(w.codes), w.dst_off)
    return w, t


def test_brute_force_small():
    w, t = _table(4, 4096, 128, 3)
    rng = np.random.default_rng(0)
    x = O.f16_from_f64(rng.standard_normal(w.cols))
    y, st = O.gemv_int4(t, w.scales, w.zp, w.group, w.rows, w.cols, x)
    assert np.all(st == O.OK)
    W = O.f64_from_f16(O.dequant_int4(O.pack_int4(w.codes), w.scales, w.zp, w.group)).reshape(w.rows, w.cols)
    xd = O.f64_from_f16(x)
    for r in range(w.rows):
        s = 0.0
        for c in range(w.cols):
            s += float(W[r, c]) * float(xd[c])
        assert abs(y[r] - s) <= 1e-9 * max(1.0, np.abs(W[r] * xd).sum()), r


def test_one_hot_picks_a_column():
    w, t = _table(8, 2048, 128, 4)
    W = O.f64_from_f16(O.dequant_int4(O.pack_int4(w.codes), w.scales, w.zp, w.group)).reshape(w.rows, w.cols)
    for j in (0, 1, 1023, 2047):
        x = np.zeros(w.cols, np.uint16)
        x[j] = 0x3C00                                   # 1.0
        y, _ = O.gemv_int4(t, w.scales, w.zp, w.group, w.rows, w.cols, x)
        assert np.array_equal(y, W[:, j])


def test_linear_in_x():
    w, t = _table(4, 2048, 256, 5)
    rng = np.random.default_rng(1)
    a = rng.integers(-8, 8, w.cols).astype(np.float64)
    b = rng.integers(-8, 8, w.cols).astype(np.float64)
    ya, _ = O.gemv_int4(t, w.scales, w.zp, w.group, w.rows, w.cols, O.f16_from_f64(a))
    yb, _ = O.gemv_int4(t, w.scales, w.zp, w.group, w.rows, w.cols, O.f16_from_f64(b))
    yab, _ = O.gemv_int4(t, w.scales, w.zp, w.group, w.rows, w.cols, O.f16_from_f64(a + b))
    assert np.allclose(ya + yb, yab, rtol=0, atol=1e-12)
