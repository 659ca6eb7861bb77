"""The entry point that allocates nothing, against the one it varies.

lt_stream_fused_lz4_int4_static decodes a host-resident table through the
library's static device workspace on one stream; its output and chunk
statuses must equal lt_stream_fused_lz4_int4's (caller-owned staging, copy
and decode overlapped on two streams) bit for bit, on two calls in a row,
the second with a smaller table, which reuses the workspace the first left
behind.  Both are called through the C ABI (ctypes binding).
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import weight_dequantization_amd as lt

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _case(rows, cols, seed, index):
    w = synth.int4_weight(rows, cols, 128, seed)
    packed = lt.pack_int4(w.codes)
    ht = lt.ChunkTable.build(packed, w.dst_off, "cpu", pin=True, index=index)
    sc = torch.from_numpy(w.scales.view(np.int16)).to(DEV)
    zp = torch.from_numpy(w.zp).to(DEV)
    n = rows * cols
    ref = torch.full((n,), -1, dtype=torch.int16, device=DEV)
    st_ref = torch.full((ht.n_chunks,), -1, dtype=torch.int32, device=DEV)
    lt.stream_fused_lz4_int4(ht, sc, zp, (rows, cols), 128, out=ref.view(torch.float16), status=st_ref)
    got = torch.full((n,), -1, dtype=torch.int16, device=DEV)
    st = torch.full((ht.n_chunks,), -1, dtype=torch.int32, device=DEV)
    lt.stream_fused_lz4_int4_static(ht, sc, zp, (rows, cols), 128, out=got.view(torch.float16), status=st)
    torch.cuda.synchronize()
    s_ref, s = st_ref.cpu().numpy(), st.cpu().numpy()
    assert np.array_equal(s, s_ref) and np.all(s == 0), (np.unique(s), np.unique(s_ref))
    g, r = got.cpu().numpy(), ref.cpu().numpy()
    bad = np.nonzero(g != r)[0]
    assert bad.size == 0, "%d of %d outputs differ from lt_stream_fused_lz4_int4, first at %d" % (bad.size, n, bad[0])
    return w, g


def test_static_workspace_matches_streamed_entry_point_twice():
    assert torch.cuda.is_available()
    # first call: 512 x 28672 (112 chunks, indexed); second: a smaller table
    # without the index, which reuses the workspace the first call filled
    _case(512, 28672, 91, True)
    w, g = _case(96, 4096, 92, False)
    ref = O.dequant_int4(O.pack_int4(w.codes), w.scales, w.zp, 128)
    assert np.array_equal(g.view(np.uint16), ref)


def test_static_workspace_too_large_is_refused():
    """A table whose largest chunk does not fit half the workspace is
    refused before anything is enqueued."""
    n = 16
    comp = np.zeros(lt.STATIC_SCRATCH_BYTES // 2 + 64, np.uint8)
    ht = lt.ChunkTable.from_host(comp, np.array([0, comp.size], np.uint64), np.array([0, n], np.uint64), "cpu",
                                 pin=True)
    sc = torch.zeros(1, dtype=torch.int16, device=DEV)
    out = torch.empty(2 * n, dtype=torch.float16, device=DEV)
    with pytest.raises(lt.LtError) as e:
        lt.stream_fused_lz4_int4_static(ht, sc, None, (1, 2 * n), 2 * n, out=out)
    assert e.value.status == lt.LT_ERR_TOO_LARGE
