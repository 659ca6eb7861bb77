"""The LT_DEBUG build (liblt_debug.so): the decoder's exec-narrowing LDS
stores (lds_set, lds_store_lanes, lds_set_entry, publish_rec) are correct
only where they are called wave-uniformly.  The debug build checks every
call and counts violations on the device; here every mode and role runs on
it (indexed and walked walks, the recorder, the hasher, six and five
builders, both history classes, the matrix-vector and matrix-product
modes) and no violation may occur.  Outputs are checked against the
oracle as well."""
import ctypes as C
import os

import numpy as np
import pytest
import torch

import oracle as O
import synth
import weight_dequantization_amd as lt

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
DEBUG_LIB = os.path.join(os.path.dirname(lt.__file__), "liblt_debug.so")


@pytest.fixture(scope="module")
def dbg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert os.path.exists(DEBUG_LIB), "liblt_debug.so is not built"
    saved_path, saved_lib = lt.LIB_PATH, lt._L
    lt.LIB_PATH, lt._L = DEBUG_LIB, None
    L = lt._lib()
    L.lt_debug_violations.restype = C.c_int
    L.lt_debug_violations.argtypes = [C.c_void_p, C.c_void_p, C.c_int]
    try:
        yield L
    finally:
        torch.cuda.synchronize()
        lt.LIB_PATH, lt._L = saved_path, saved_lib


def _violations(L):
    torch.cuda.synchronize()
    n, line = C.c_uint32(0), C.c_uint32(0)
    assert L.lt_debug_violations(C.byref(n), C.byref(line), 1) == 0
    return n.value, line.value


def test_debug_build_counts_planted_violations(dbg):
    """The checker itself: a self-test wave with two non-uniform calls is
    counted twice; the count is then cleared."""
    assert _violations(dbg) == (0, 0)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    dbg.lt_debug_selftest.restype = C.c_int
    dbg.lt_debug_selftest.argtypes = [C.c_void_p, C.c_void_p]
    assert dbg.lt_debug_selftest(C.c_void_p(sink.data_ptr()), None) == 0
    n, line = _violations(dbg)
    assert n == 2 and line > 0
    assert _violations(dbg) == (0, 0)


def test_fused_int4_indexed_walked_checked(dbg):
    w = synth.mlp_int4_small(rows=256)
    packed = lt.pack_int4(w.codes)
    ref = O.dequant_int4(O.pack_int4(w.codes), w.scales, w.zp, w.group)
    for index, checksum in ((True, False), (False, False), (True, True), (False, True)):
        tb = lt.ChunkTable.build(packed, w.dst_off, DEV, index=index, checksum=checksum)
        st = torch.full((tb.n_chunks,), -1, dtype=torch.int32, device=DEV)
        out = lt.fused_lz4_int4(tb, torch.from_numpy(w.scales.view(np.int16)).to(DEV), torch.from_numpy(w.zp).to(DEV),
                                (w.rows, w.cols), w.group, status=st)
        torch.cuda.synchronize()
        assert np.all(st.cpu().numpy() == 0)
        assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16).ravel(), ref)
        assert _violations(dbg) == (0, 0), (index, checksum)


def test_decode_activations_and_generated_streams(dbg):
    a = synth.activation(512, 8192, 71)
    for data, dst_off, window in ((a.data, a.dst_off, lt.PACK_WINDOW), (a.data, a.dst_off, 0)):
        for index in (True, False):
            tb = lt.ChunkTable.build(data, dst_off, DEV, max_dist=window, index=index)
            st = torch.full((tb.n_chunks,), -1, dtype=torch.int32, device=DEV)
            out = lt.decode_lz4(tb, status=st)
            torch.cuda.synchronize()
            assert np.all(st.cpu().numpy() == 0) and np.array_equal(out.cpu().numpy(), data)
            assert _violations(dbg) == (0, 0), (window, index)
    ot = O.compress_table(a.data, a.dst_off)
    for index in (True, False):
        tb = lt.ChunkTable.from_host(ot.comp, ot.comp_off, a.dst_off, DEV, index=index)
        st = torch.full((tb.n_chunks,), -1, dtype=torch.int32, device=DEV)
        out = lt.decode_lz4(tb, status=st)
        torch.cuda.synchronize()
        assert np.all(st.cpu().numpy() == 0) and np.array_equal(out.cpu().numpy(), a.data)
        assert _violations(dbg) == (0, 0), ("oracle stream", index)
    for seed in range(6):   # generated streams: far and overlapping matches, the 64 KiB history
        b, e = O.seqgen(400 + seed, 70000 + 9000 * seed)
        tb = lt.ChunkTable.from_host(b, np.array([0, b.size], np.uint64), np.array([0, e.size], np.uint64), DEV)
        st = torch.full((1,), -1, dtype=torch.int32, device=DEV)
        out = lt.decode_lz4(tb, status=st)
        torch.cuda.synchronize()
        assert st.cpu().numpy()[0] == 0 and np.array_equal(out.cpu().numpy(), e)
        assert _violations(dbg) == (0, 0), seed


def test_gemv_and_gemm_modes(dbg):
    w = synth.mlp_int4_small(rows=64)
    sc = torch.from_numpy(w.scales.view(np.int16)).to(DEV)
    zp = torch.from_numpy(w.zp).to(DEV)
    tb = lt.ChunkTable.build(lt.pack_int4(w.codes), w.dst_off, DEV)
    x = torch.randn(w.cols, dtype=torch.float16, device=DEV)
    lt.fused_lz4_int4_gemv(tb, sc, zp, (w.rows, w.cols), w.group, x)
    assert _violations(dbg) == (0, 0)
    gt = lt.ChunkTable.build(lt.pack_int4_tiles(w.codes.reshape(w.rows, w.cols), w.rows, w.cols),
                             lt.gemm_chunks(w.rows, w.cols), DEV)
    X = torch.randn(32, w.cols, dtype=torch.float16, device=DEV)
    st = torch.full((gt.n_chunks,), -1, dtype=torch.int32, device=DEV)
    lt.fused_lz4_int4_gemm(gt, sc, zp, (w.rows, w.cols), w.group, X, status=st)
    torch.cuda.synchronize()
    assert np.all(st.cpu().numpy() == 0)
    assert _violations(dbg) == (0, 0)
