"""Per-chunk XXH3-64 of compressed bytes on the device, without decoding
(lt_verify_chunks; the block checksum of "GPU Compression Pipeline - TDD
Roadmap", Phase 6.1): every computed value equals the oracle's, a changed
stored byte is reported at exactly its chunk, and bad offsets fail their
chunk.
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


def u32(t, n):
    torch.cuda.synchronize()
    return t[:n].cpu().numpy().view(np.uint32)


def u64(t, n):
    torch.cuda.synchronize()
    return t[:n].cpu().numpy().view(np.uint64)


def dev_u64(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint64).view(np.int64)).to(DEV)


def test_mlp_8192x28672_checksums_and_single_flips():
    """The benchmark layer's 1792 packer blocks: computed values equal the
    oracle's; the host packer's values verify; one flipped byte in each of
    several chunks fails exactly those chunks."""
    w = synth.mlp_int4_8192x28672()
    comp, comp_off = lt.compress_chunks(lt.pack_int4(w.codes), w.dst_off, max_dist=lt.PACK_WINDOW)
    table = lt.ChunkTable.from_host(comp, comp_off, w.dst_off, DEV)
    ref = O.xxh3_chunks(comp, comp_off)
    got, _ = lt.verify_chunks(table)
    assert np.array_equal(u64(got, table.n_chunks), ref)
    expect = dev_u64(lt.checksum_chunks(comp, comp_off))
    _, st = lt.verify_chunks(table, expect)
    assert np.all(u32(st, table.n_chunks) == 0)
    rng = np.random.default_rng(4)
    bad = np.sort(rng.choice(table.n_chunks, 12, replace=False))
    for i in bad:
        a, b = int(comp_off[i]), int(comp_off[i + 1])
        p = int(rng.integers(a, b))
        table.comp[p] ^= int(rng.integers(1, 256))
    got, st = lt.verify_chunks(table, expect)
    s = u32(st, table.n_chunks)
    assert np.array_equal(np.nonzero(s)[0], bad) and np.all(s[bad] == lt.CHUNK_CHECKSUM)
    assert np.array_equal(u64(got, table.n_chunks), O.xxh3_chunks(table.comp.cpu().numpy(), comp_off))


@pytest.mark.parametrize("shift", [0, 1, 7, 15])
def test_arbitrary_offsets_and_alignment(shift):
    """Chunk boundaries at any byte (empty chunks, every length class of the
    hash: 1-3, 4-8, 9-16, 17-128, 129-240 bytes and the block form, lengths
    next to whole blocks and stripes, chunks of up to 300000 bytes), with the
    table's base address itself 0..15 bytes past a 16-byte boundary."""
    rng = np.random.default_rng(10 + shift)
    sizes = [0, 1, 2, 3, 4, 5, 8, 9, 13, 15, 16, 17, 31, 32, 33, 64, 65, 96, 97, 127, 128, 129, 200, 239, 240, 241,
             255, 256, 1023, 1024, 1025, 1088, 2047, 2048, 2049, 4095, 4096, 4097, 65536, 65551, 300000, 0, 9]
    sizes += list(rng.integers(0, 70000, 40))
    comp_off = np.cumsum([0] + sizes).astype(np.uint64)
    data = rng.integers(0, 256, int(comp_off[-1]), dtype=np.uint8)
    data[1000:200000] = 0
    store = torch.zeros(data.size + 64, dtype=torch.uint8, device=DEV)
    store[shift:shift + data.size] = torch.from_numpy(data).to(DEV)
    base = store[shift:shift + data.size]
    table = lt.ChunkTable(base, torch.from_numpy(comp_off.view(np.int64)).to(DEV),
                          torch.from_numpy(comp_off.view(np.int64)).to(DEV), len(sizes), 1 << 20,
                          int(comp_off[-1]), int(comp_off[-1]))
    got, _ = lt.verify_chunks(table)
    assert np.array_equal(u64(got, len(sizes)), O.xxh3_chunks(data, comp_off))


def test_bad_offsets_fail_their_chunk():
    data = np.arange(10000, dtype=np.uint32).astype(np.uint8)
    comp_off = np.array([0, 100, 50, 3000, 20000, 10000], np.uint64)   # decreasing, then past the end
    table = lt.ChunkTable(torch.from_numpy(data).to(DEV), torch.from_numpy(comp_off.view(np.int64)).to(DEV),
                          torch.from_numpy(comp_off.view(np.int64)).to(DEV), 5, 1 << 20, 10000, 10000)
    expect = dev_u64(np.zeros(5, np.uint64))
    got, st = lt.verify_chunks(table, expect)
    s = u32(st, 5)
    assert s[1] == lt.CHUNK_BAD_TABLE and s[3] == lt.CHUNK_BAD_TABLE and s[4] == lt.CHUNK_BAD_TABLE, s
    assert s[0] == lt.CHUNK_CHECKSUM and s[2] == lt.CHUNK_CHECKSUM      # zero is not their hash
    g = u64(got, 5)
    assert g[0] == O.xxh3_64(data[0:100]) and g[2] == O.xxh3_64(data[50:3000])
