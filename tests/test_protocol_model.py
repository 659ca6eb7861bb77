"""The chunk decoder's LDS protocol, modelled on the CPU under random
interleavings (tests/protocol_model.py), over the workloads' own blocks:
the 8192x28672 layer's distributions (host packer, 4 KiB declared window,
16 KiB history class), the ReLU activations with their stress chunks (host
packer in the 16 KiB class; the oracle's greedy compressor in the 64 KiB
class), generator-built streams with far and overlapping matches and chunks
over 64 KiB, and all-literal and long-run blocks; each with and without the
sequence index and on several schedules.  Every read must see landed,
unoverwritten input, live records and final history; no schedule may
deadlock; the decode must equal the expected bytes.  Every case runs
again with the byte-output kernel's speculative build (a tile whose sources
are not built yet is built at once, then its copies are made again after the
wait).  The model is also shown to catch planted protocol mistakes.
"""
import numpy as np
import pytest

import oracle as O
import synth
import weight_dequantization_amd as lt
from protocol_model import Chunk, ProtocolError


def _chunks(comp, comp_off, dst_off, src, picks):
    so, sp = lt.index_chunks(comp, comp_off)
    for i in picks:
        blk = comp[int(comp_off[i]):int(comp_off[i + 1])]
        yield (i, blk, src[int(dst_off[i]):int(dst_off[i + 1])].tobytes(), sp[int(so[i]):int(so[i + 1])])


def _run(blk, expect, idx, hlog, dmax, seeds, what):
    """Returns how many tiles were built speculatively."""
    nspec = 0
    for seed in seeds:
        for indexed in (True, False):
            for spec in (False, True):
                c = Chunk(blk, len(expect), index=idx if indexed else None, hlog=hlog, dmax=dmax, head=seed % 16,
                          seed=seed, spec=spec)
                st, out, _ = c.run()
                assert st == 0, (what, seed, indexed, spec, st)
                assert out == expect, (what, seed, indexed, spec)
                assert all(v == 1 for v in c.built), (what, seed, indexed, spec)
                nspec += c.nspec
    return nspec


def test_weight_layer_chunks():
    w = synth.mlp_int4_small(rows=64)
    packed = lt.pack_int4(w.codes)
    comp, comp_off = lt.compress_chunks(packed, w.dst_off, max_dist=lt.PACK_WINDOW)
    n = w.dst_off.size - 1
    for i, blk, expect, idx in _chunks(comp, comp_off, w.dst_off, packed, range(0, n, max(1, n // 6))):
        _run(blk, expect, idx, 14, lt.PACK_WINDOW, (1, 2, 3), "weight chunk %d" % i)


def test_activation_chunks_with_stress_blocks():
    a = synth.activation(1024, 8192, 1104)
    picks = sorted(set(a.stress["random"] + a.stress["all_ab"] + a.stress["ab_run"] + [0, 1, 100]))
    comp, comp_off = lt.compress_chunks(a.data, a.dst_off, max_dist=lt.PACK_WINDOW)
    nspec = 0
    for i, blk, expect, idx in _chunks(comp, comp_off, a.dst_off, a.data, picks):
        nspec += _run(blk, expect, idx, 14, lt.PACK_WINDOW, (4, 5), "activation chunk %d, packer" % i)
    ot = O.compress_table(a.data, a.dst_off)
    for i, blk, expect, idx in _chunks(ot.comp, ot.comp_off, a.dst_off, a.data, picks):
        nspec += _run(blk, expect, idx, 16, 65535, (6, 7), "activation chunk %d, oracle compressor" % i)
    assert nspec > 0   # the speculative build was taken


@pytest.mark.parametrize("target", [5000, 70000, 262144])
def test_generated_streams(target):
    for seed in range(3):
        blk, expect = O.seqgen(1000 + seed + target, target)
        idx = lt.index_chunks(blk, np.array([0, blk.size], np.uint64))[1]
        _run(blk, expect.tobytes(), idx, 16, 65535, (seed,), "seqgen %d/%d" % (target, seed))


def test_all_literal_and_long_run_blocks():
    r = np.random.default_rng(9).integers(0, 256, 65536, dtype=np.uint8)
    x = np.full(65536, 0xAB, np.uint8)
    for data, what in ((r, "random"), (x, "0xAB")):
        for blk in (O.lz4_compress(data), O.lz4_store(data)):
            idx = lt.index_chunks(blk, np.array([0, blk.size], np.uint64))[1]
            _run(blk, data.tobytes(), idx, 16, 65535, (1, 2), what)
            _run(blk, data.tobytes(), idx, 14, 65535, (3,), what + " (16 KiB class, any window)")


def _fault_caught(fault, blk, expect, idx, hlog, dmax, seeds):
    """How many schedules of a model with a planted mistake end in a
    detected violation, a deadlock or a wrong decode."""
    caught = 0
    for seed in range(seeds):
        c = Chunk(blk, len(expect), index=idx, hlog=hlog, dmax=dmax, seed=seed, fault=fault)
        try:
            _, out, _ = c.run()
            caught += out != expect
        except ProtocolError:
            caught += 1
    return caught


def test_model_catches_planted_mistakes():
    """Each planted protocol mistake is caught on some schedule (each case
    pairs a history class with a window its blocks keep to)."""
    w = synth.mlp_int4_small(rows=64)
    packed = lt.pack_int4(w.codes)
    p64, p256 = packed[:65536], packed[:262144]
    b64, o64 = lt.compress_chunks(p64, np.array([0, p64.size], np.uint64), max_dist=lt.PACK_WINDOW)
    i64 = lt.index_chunks(b64, o64)[1]
    for fault in ("no_window", "early_need"):
        assert _fault_caught(fault, b64, p64.tobytes(), i64, 14, lt.PACK_WINDOW, 4) >= 3, fault
    # a speculatively built tile whose copies are made again without waiting
    # for their sources
    a = synth.activation(1024, 8192, 1104)
    ab, ao = lt.compress_chunks(a.data, a.dst_off, max_dist=lt.PACK_WINDOW)
    caught = 0
    for i, blk, expect, idx in _chunks(ab, ao, a.dst_off, a.data, a.stress["ab_run"][:2] + [0, 1]):
        for seed in range(3):
            c = Chunk(blk, len(expect), index=idx, hlog=14, dmax=lt.PACK_WINDOW, seed=seed, spec=True,
                      fault="spec_no_wait")
            try:
                _, out, _ = c.run()
                caught += out != expect
            except ProtocolError:
                caught += 1
    assert caught >= 1
    # a slot reused while the tile that held it is still being written out
    b256, o256 = lt.compress_chunks(p256, np.array([0, p256.size], np.uint64), max_dist=lt.PACK_WINDOW)
    i256 = lt.index_chunks(b256, o256)[1]
    assert _fault_caught("no_write_rule", b256, p256.tobytes(), i256, 14, lt.PACK_WINDOW, 10) >= 1
    assert _fault_caught(None, b256, p256.tobytes(), i256, 14, lt.PACK_WINDOW, 3) == 0
    g, e = O.seqgen(5, 262144)
    gidx = lt.index_chunks(g, np.array([0, g.size], np.uint64))[1]
    assert _fault_caught("no_slot_rule", g, e.tobytes(), gidx, 16, 65535, 3) == 3
    # a 20,000-byte literal run, longer than the 8 KiB input ring, then a match
    r = np.random.default_rng(3).integers(0, 256, 20000, dtype=np.uint8)
    d = np.concatenate([r, r[:3000]])
    db = O.lz4_compress(d)
    assert _fault_caught("no_split", db, d.tobytes(), None, 16, 65535, 2) == 2
    assert _fault_caught(None, db, d.tobytes(), None, 16, 65535, 2) == 0


def test_checksum_hasher():
    """With checksums the hasher reads every compressed byte once it has
    landed and before it is reloaded, on indexed and walked layer blocks,
    activation stress blocks and long generated streams; a hasher that
    never announces its position is caught."""
    w = synth.mlp_int4_small(rows=64)
    packed = lt.pack_int4(w.codes)
    comp, comp_off = lt.compress_chunks(packed, w.dst_off, max_dist=lt.PACK_WINDOW)
    a = synth.activation(1024, 8192, 1104)
    acomp, aoff = lt.compress_chunks(a.data, a.dst_off, max_dist=lt.PACK_WINDOW)
    g, e = O.seqgen(77, 262144)
    cases = [(comp, comp_off, w.dst_off, packed, [0, 3], 14, lt.PACK_WINDOW),
             (acomp, aoff, a.dst_off, a.data, a.stress["random"][:1] + a.stress["ab_run"][:1], 14, lt.PACK_WINDOW),
             (g, np.array([0, g.size], np.uint64), np.array([0, e.size], np.uint64), e, [0], 16, 65535)]
    for cb, co, do, src, picks, hlog, dmax in cases:
        for i, blk, expect, idx in _chunks(cb, co, do, src, picks):
            for seed in (1,):
                for indexed in (True, False):
                    c = Chunk(blk, len(expect), index=idx if indexed else None, hlog=hlog, dmax=dmax, seed=seed,
                              checksum=True)
                    st, out, _ = c.run()
                    assert st == 0 and out == expect and c.hashed, (i, seed, indexed)
    b = comp[int(comp_off[0]):int(comp_off[1])]
    caught = 0
    for seed in range(6):
        c = Chunk(b, int(w.dst_off[1]), index=None, hlog=14, dmax=lt.PACK_WINDOW, seed=seed, checksum=True,
                  fault="hasher_silent")
        try:
            c.run()
        except ProtocolError:
            caught += 1
            break
    assert caught >= 1


def test_static_tile_assignment():
    """The matrix-product mode's static tiles (builder b takes b, b + nb, ...)
    keep every rule and cannot deadlock, on layer blocks in the GEMM layout's
    chunk size (56 KiB) with both history classes, indexed and walked."""
    w = synth.mlp_int4_small(rows=64)
    codes = w.codes.reshape(w.rows, w.cols)
    data = lt.pack_int4_tiles(codes, w.rows, w.cols)
    dst_off = lt.gemm_chunks(w.rows, w.cols)
    for window, hlog in ((lt.PACK_WINDOW, 14), (0, 16)):
        comp, comp_off = lt.compress_chunks(data, dst_off, max_dist=window)
        for i, blk, expect, idx in _chunks(comp, comp_off, dst_off, data, [0, 5]):
            for indexed in (True, False):
                c = Chunk(blk, len(expect), index=idx if indexed else None, hlog=hlog,
                          dmax=window or 65535, seed=3, static_tiles=True)
                st, out, _ = c.run()
                assert st == 0 and out == expect and all(v == 1 for v in c.built), (i, indexed, hlog)
