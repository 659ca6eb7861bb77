"""File-streamed copy-and-decode: the compressed bytes stay in a file and
each batch is read with pread into a pinned half while the batches before
it are copied and decoded ("GPU Compression Pipeline - TDD Roadmap", Phase
5.1, its three stages read / transfer / decompress).  The result must be the
oracle's, bit for bit, for any batching, reader count and file offset; a
file that ends early must raise LT_ERR_IO.
"""
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


def statuses(st, n):
    torch.cuda.synchronize()
    return st[:n].cpu().numpy()


def _file(tmp_path, comp, offset, name="comp.bin"):
    p = tmp_path / name
    with open(p, "wb") as f:
        f.write(b"\x5a" * offset)
        f.write(comp.tobytes())
    return str(p)


def _layer():
    w = synth.mlp_int4_small(rows=512)
    comp, comp_off = lt.compress_chunks(lt.pack_int4(w.codes), w.dst_off, max_dist=lt.PACK_WINDOW)
    return w, comp, comp_off


@pytest.mark.parametrize("per_half,threads,offset", [(1, 1, 0), (7, 4, 4096 + 7), (100, 8, 123), (512, 3, 0)])
def test_file_fused_int4_equals_oracle(tmp_path, per_half, threads, offset):
    """Any batch size (one chunk per half up to the whole table), any number
    of reader threads and any file offset give the oracle's output; with
    checksums every chunk verifies."""
    w, comp, comp_off = _layer()
    path = _file(tmp_path, comp, offset)
    ht = lt.ChunkTable.from_host(comp, comp_off, w.dst_off, "cpu", lt.PACK_WINDOW, index=True, pin=True,
                                 checksum=True)
    st = torch.full((ht.n_chunks,), -1, dtype=torch.int32, device=DEV)
    pinned = torch.empty(ht.pinned_bytes(per_half), dtype=torch.uint8, pin_memory=True)
    staging = torch.empty(ht.staging_bytes(per_half), dtype=torch.uint8, device=DEV)
    out = lt.stream_file_fused_lz4_int4(path, offset, ht, torch.from_numpy(w.scales.view(np.int16)).to(DEV),
                                        torch.from_numpy(w.zp).to(DEV), (w.rows, w.cols), w.group, status=st,
                                        pinned=pinned, staging=staging, read_threads=threads)
    s = statuses(st, ht.n_chunks)
    assert np.all(s == 0), np.unique(s)
    assert np.array_equal(host_u16(out), O.dequant_int4(O.pack_int4(w.codes), w.scales, w.zp, w.group))


def test_file_decode_and_int8(tmp_path):
    """Decode-only on the activation workload (with its stress chunks) and
    fused INT8 on an INT8 matrix, both from files, default buffers."""
    a = synth.activation(512, 8192, 61)
    comp, comp_off = lt.compress_chunks(a.data, a.dst_off, max_dist=lt.PACK_WINDOW)
    ht = lt.ChunkTable.from_host(comp, comp_off, a.dst_off, "cpu", lt.PACK_WINDOW, index=True, pin=True)
    st = torch.full((ht.n_chunks,), -1, dtype=torch.int32, device=DEV)
    out = lt.stream_file_decode_lz4(_file(tmp_path, comp, 16, "act.bin"), 16, ht, status=st)
    assert np.all(statuses(st, ht.n_chunks) == 0)
    assert np.array_equal(out.cpu().numpy(), a.data)
    rng = np.random.default_rng(62)
    q = np.clip(np.rint(rng.standard_normal(256 * 8192) * 32), -127, 127).astype(np.int8)
    q[: 8192 * 100] = 0
    scales = synth.fp16_bits(rng.uniform(1e-3, 1e-2, 256))
    dst_off = synth.uniform_chunks(q.size)
    comp, comp_off = lt.compress_chunks(q.view(np.uint8), dst_off, max_dist=lt.PACK_WINDOW)
    ht = lt.ChunkTable.from_host(comp, comp_off, dst_off, "cpu", lt.PACK_WINDOW, index=True, pin=True)
    st = torch.full((ht.n_chunks,), -1, dtype=torch.int32, device=DEV)
    out = lt.stream_file_fused_lz4_int8(_file(tmp_path, comp, 0, "q.bin"), 0, ht,
                                        torch.from_numpy(scales.view(np.int16)).to(DEV), None, (256, 8192), 8192,
                                        status=st)
    assert np.all(statuses(st, ht.n_chunks) == 0)
    assert np.array_equal(host_u16(out), O.dequant_int8(q, scales, None, 8192))


def test_file_that_ends_early_raises(tmp_path):
    """A file shorter than the table says: LT_ERR_IO (the batches before the
    short read stay enqueued and finish normally)."""
    w, comp, comp_off = _layer()
    path = _file(tmp_path, comp[: comp.size // 2], 0)
    ht = lt.ChunkTable.from_host(comp, comp_off, w.dst_off, "cpu", lt.PACK_WINDOW, index=True, pin=True)
    # the caller's buffers outlive the copies still in flight when the call raises
    staging = torch.empty(ht.staging_bytes(8), dtype=torch.uint8, device=DEV)
    pinned = torch.empty(ht.pinned_bytes(8), dtype=torch.uint8, pin_memory=True)
    with pytest.raises(lt.LtError) as e:
        lt.stream_file_fused_lz4_int4(path, 0, ht, torch.from_numpy(w.scales.view(np.int16)).to(DEV),
                                      torch.from_numpy(w.zp).to(DEV), (w.rows, w.cols), w.group,
                                      staging=staging, pinned=pinned)
    assert e.value.status == lt.LT_ERR_IO
    torch.cuda.synchronize()
    del staging, pinned
