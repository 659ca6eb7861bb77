"""Codebook dequantization on the device (lt_dequant_int4_lut; the pages'
value dictionaries: small codes plus a lookup table per group) against the
oracle, bit for bit: the benchmark layer's shape, a per-tensor dictionary,
groups that are not powers of two, and ragged lengths."""
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


def host_u16(t):
    torch.cuda.synchronize()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).ravel()


def dev_u16(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).to(DEV)


def _check(codes, lut, rows, cols, group, what):
    packed = lt.pack_int4(codes)
    out = lt.dequant_int4_lut(torch.from_numpy(packed).to(DEV), dev_u16(lut), (rows, cols), group)
    ref = O.dequant_int4_lut(O.pack_int4(codes), lut, group)
    got = host_u16(out)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, "%s: %d differ, first at %d" % (what, bad.size, bad[0])


def test_mlp_8192x28672_shape_random_tables():
    """8192x28672, group 128, every table entry a random fp16 pattern."""
    w = synth.mlp_int4_8192x28672()
    rng = np.random.default_rng(0)
    lut = rng.integers(0, 65536, (w.rows * w.cols // 128, 16)).astype(np.uint16)
    _check(w.codes, lut, w.rows, w.cols, 128, "mlp_int4_8192x28672 shape")


def test_affine_tables_equal_affine_dequant():
    """A table filled from (q - zp) * s gives lt_dequant_int4's output."""
    w = synth.tiny_int4_1024()
    q = np.arange(16, dtype=np.int64)
    vals = (q[None, :] - w.zp.astype(np.int64)[:, None]) * O.f64_from_f16(w.scales)[:, None]
    lut = O.f16_from_f64(vals.ravel()).reshape(-1, 16)
    packed = torch.from_numpy(lt.pack_int4(w.codes)).to(DEV)
    a = lt.dequant_int4_lut(packed, dev_u16(lut), (w.rows, w.cols), w.group)
    b = lt.dequant_int4(packed, dev_u16(w.scales), torch.from_numpy(w.zp).to(DEV), (w.rows, w.cols), w.group)
    assert np.array_equal(host_u16(a), host_u16(b))


@pytest.mark.parametrize("rows,cols,group", [
    (1024, 1024, 1024 * 1024),   # one dictionary for the tensor
    (33, 300, 100), (64, 96, 48), (7, 8192, 16), (5, 1000, 1000), (3, 8190, 8190), (1, 24, 24),
])
def test_groups_and_tails(rows, cols, group):
    rng = np.random.default_rng(rows * 7 + cols)
    n = rows * cols
    codes = rng.integers(0, 16, n, dtype=np.uint8)
    lut = rng.integers(0, 65536, (n // group, 16)).astype(np.uint16)
    _check(codes, lut, rows, cols, group, "%dx%d g%d" % (rows, cols, group))
