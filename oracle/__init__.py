"""CPU oracle for just-in-time tensor decompression (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``libltref.so`` (plain C built
with gcc from ``ltref.c``) with numpy arrays.  It shares no code with the HIP
library in ``weight_dequantization_amd`` and never imports it.

What it computes (every function is the plain definition, written from):

* fp16 rounding: IEEE 754 binary16 / binary64 bit fields, nearest-even.
* LZ4 block decode / greedy compress / all-literal store: the public LZ4 block
  format (the pages name LZ4 for compressed weight blocks - "GPU Compression
  Pipeline - TDD Roadmap", Phase 2.1 and Phase 3.1 - without defining it).
* INT4 packing, low nibble first, and dequantization (q - zp) * scale to fp16:
  the roadmap's Phase 1.1 (INT4) and Phase 1.2 (INT8) worked examples.
* fused = dequantize(decode(table)): the roadmap's CPU reference for its fused
  kernel (Phase 2.1).
* matrix-vector product with the dequantized matrix, y = W x in fp64 from the
  fp16 weights that fused_int4 gives (decompress, then multiply: the pages'
  decode-plus-GEMM benchmarks), by a library matrix product.
* codebook dequantization: element e is entry q(e) of its group's 16-entry fp16
  table (the pages' value dictionaries of small codes plus a lookup table).
* zero-run coding of fp16 activations (per 1024-element block a nonzero bitmap,
  then the nonzero values in order): the pages' zero-run encoding of ReLU
  outputs, in the bitmap form the GPU decoder reads.
* XXH3-64 of each chunk's compressed bytes, from the hash's public
  definition: the per-block checksum the roadmap's container format names
  (Phase 6.1).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ltref.c")
_LIB = os.path.join(_HERE, "libltref.so")

OK, TRUNCATED, BAD_OFFSET, OVERRUN, SIZE_MISMATCH, BAD_TABLE = range(6)


def build(force: bool = False) -> str:
    """Compile libltref.so with gcc (plain C11, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-fPIC", "-shared",
                               "-pthread", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = C.CDLL(_LIB)
        u8p, u16p, u32p, u64p = (C.POINTER(t) for t in (C.c_uint8, C.c_uint16, C.c_uint32, C.c_uint64))
        i8p, i32p, f64p = C.POINTER(C.c_int8), C.POINTER(C.c_int32), C.POINTER(C.c_double)
        u64, u32, vp = C.c_uint64, C.c_uint32, C.c_void_p
        sig = {
            "ltref_f64_from_f16": (C.c_double, [C.c_uint16]),
            "ltref_f16_from_f64": (C.c_uint16, [C.c_double]),
            "ltref_f16_from_f64_array": (None, [vp, u64, vp]),
            "ltref_f16_from_f32bits_array": (None, [vp, u64, vp]),
            "ltref_f64_from_f16_array": (None, [vp, u64, vp]),
            "ltref_lz4_decode_block": (C.c_int, [vp, u64, vp, u64, vp]),
            "ltref_lz4_bound": (u64, [u64]),
            "ltref_lz4_store": (u64, [vp, u64, vp]),
            "ltref_lz4_compress": (u64, [vp, u64, vp]),
            "ltref_pack_int4": (None, [vp, u64, vp]),
            "ltref_unpack_int4": (None, [vp, u64, vp]),
            "ltref_dequant_int4": (None, [vp, u64, vp, vp, u64, vp]),
            "ltref_dequant_int8": (None, [vp, u64, vp, vp, u64, vp]),
            "ltref_decode_table": (u32, [vp, u64, vp, vp, u32, u64, vp, vp, C.c_int]),
            "ltref_compress_table": (u64, [vp, vp, u32, vp, u64, vp, C.c_int]),
            "ltref_fused_int4": (u32, [vp, u64, vp, vp, u32, u64, vp, vp, u64, u64, vp, vp, C.c_int]),
            "ltref_fused_int8": (u32, [vp, u64, vp, vp, u32, u64, vp, vp, u64, u64, vp, vp, C.c_int]),
            "ltref_fused_int4_chunked": (u32, [vp, u64, vp, vp, u32, u64, vp, vp, u64, vp, vp, C.c_int]),
            "ltref_seqgen": (u64, [u64, u64, vp, u64, vp, u64, vp]),
            "ltref_dequant_int4_lut": (None, [vp, u64, vp, u64, vp]),
            "ltref_zr_encode": (u64, [vp, u64, vp, vp, vp]),
            "ltref_zr_decode": (None, [vp, vp, vp, u64, u64, vp, vp]),
            "ltref_xxh3_64": (C.c_uint64, [vp, u64]),
            "ltref_xxh3_chunks": (None, [vp, vp, u32, vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------- fp16

def f16_from_f64(x) -> np.ndarray:
    x = _c(np.atleast_1d(x), np.float64)
    out = np.empty(x.size, np.uint16)
    lib().ltref_f16_from_f64_array(_p(x), x.size, _p(out))
    return out


def f16_from_f32bits(bits: np.ndarray) -> np.ndarray:
    bits = _c(bits, np.uint32)
    out = np.empty(bits.size, np.uint16)
    lib().ltref_f16_from_f32bits_array(_p(bits), bits.size, _p(out))
    return out


def f64_from_f16(h) -> np.ndarray:
    h = _c(np.atleast_1d(h), np.uint16)
    out = np.empty(h.size, np.float64)
    lib().ltref_f64_from_f16_array(_p(h), h.size, _p(out))
    return out


# -------------------------------------------------------------------- LZ4

def lz4_bound(n: int) -> int:
    return int(lib().ltref_lz4_bound(n))


def lz4_decode(block: np.ndarray, out_size: int):
    """Decode one LZ4 block to exactly out_size bytes -> (status, bytes, produced)."""
    block = _c(block, np.uint8)
    out = np.zeros(max(out_size, 1), np.uint8)
    produced = C.c_uint64(0)
    st = lib().ltref_lz4_decode_block(_p(block), block.size, _p(out), out_size, C.byref(produced))
    return int(st), out[:out_size], int(produced.value)


def lz4_compress(x: np.ndarray) -> np.ndarray:
    x = _c(x, np.uint8)
    out = np.empty(lz4_bound(x.size), np.uint8)
    n = lib().ltref_lz4_compress(_p(x), x.size, _p(out))
    return out[:n].copy()


def lz4_store(x: np.ndarray) -> np.ndarray:
    x = _c(x, np.uint8)
    out = np.empty(lz4_bound(x.size), np.uint8)
    n = lib().ltref_lz4_store(_p(x), x.size, _p(out))
    return out[:n].copy()


def seqgen(seed: int, target: int):
    """Random valid LZ4 block built side by side with its expected output."""
    stream = np.empty(2 * target + 64, np.uint8)
    expected = np.empty(max(target, 1), np.uint8)
    out_len = C.c_uint64(0)
    n = lib().ltref_seqgen(seed, target, _p(stream), stream.size, _p(expected), expected.size,
                           C.byref(out_len))
    assert n > 0
    return stream[:n].copy(), expected[:out_len.value].copy()


# ------------------------------------------------------------- INT4 / INT8

def pack_int4(codes: np.ndarray) -> np.ndarray:
    codes = _c(codes, np.uint8)
    assert codes.size % 2 == 0
    out = np.empty(codes.size // 2, np.uint8)
    lib().ltref_pack_int4(_p(codes), codes.size, _p(out))
    return out


def unpack_int4(packed: np.ndarray, n_codes: int | None = None) -> np.ndarray:
    packed = _c(packed, np.uint8)
    n = 2 * packed.size if n_codes is None else n_codes
    out = np.empty(n, np.uint8)
    lib().ltref_unpack_int4(_p(packed), n, _p(out))
    return out


def dequant_int4(packed, scales, zp, group: int, n_elem: int | None = None) -> np.ndarray:
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.uint16)
    zp = _c(zp, np.int8)
    n = 2 * packed.size if n_elem is None else n_elem
    out = np.empty(n, np.uint16)
    lib().ltref_dequant_int4(_p(packed), n, _p(scales), _p(zp), group, _p(out))
    return out


def dequant_int8(q, scales, zp, group: int) -> np.ndarray:
    q = _c(q, np.int8)
    scales = _c(scales, np.uint16)
    zp = _c(zp, np.int8)
    out = np.empty(q.size, np.uint16)
    lib().ltref_dequant_int8(_p(q), q.size, _p(scales), _p(zp), group, _p(out))
    return out


# ------------------------------------------------------------ chunk tables

class Table:
    """Host chunk table: concatenated LZ4 blocks plus prefix-sum offsets."""

    def __init__(self, comp, comp_off, dst_off):
        self.comp = _c(comp, np.uint8)
        self.comp_off = _c(comp_off, np.uint64)
        self.dst_off = _c(dst_off, np.uint64)

    @property
    def n(self):
        return self.dst_off.size - 1

    @property
    def total(self):
        return int(self.dst_off[-1])

    @property
    def comp_bytes(self):
        return int(self.comp_off[-1])


def compress_table(src: np.ndarray, dst_off: np.ndarray, threads: int = 8) -> Table:
    src = _c(src, np.uint8)
    dst_off = _c(dst_off, np.uint64)
    n = dst_off.size - 1
    cap = int(sum(lz4_bound(int(dst_off[i + 1] - dst_off[i])) for i in range(n))) + 16
    comp = np.empty(cap, np.uint8)
    comp_off = np.empty(n + 1, np.uint64)
    size = lib().ltref_compress_table(_p(src), _p(dst_off), n, _p(comp), cap, _p(comp_off), threads)
    assert size > 0 or n == 0
    return Table(comp[:size].copy(), comp_off, dst_off)


def decode_table(t: Table, threads: int = 8):
    dst = np.zeros(max(t.total, 1), np.uint8)
    status = np.empty(max(t.n, 1), np.int32)
    lib().ltref_decode_table(_p(t.comp), t.comp.size, _p(t.comp_off), _p(t.dst_off), t.n,
                             t.total, _p(dst), _p(status), threads)
    return dst[:t.total], status[:t.n]


def fused_int4(t: Table, scales, zp, group: int, n_elem: int, threads: int = 8):
    scales = _c(scales, np.uint16)
    zp = _c(zp, np.int8)
    out = np.zeros(max(n_elem, 1), np.uint16)
    status = np.empty(max(t.n, 1), np.int32)
    lib().ltref_fused_int4(_p(t.comp), t.comp.size, _p(t.comp_off), _p(t.dst_off), t.n, t.total,
                           _p(scales), _p(zp), n_elem, group, _p(out), _p(status), threads)
    return out[:n_elem], status[:t.n]


def fused_int8(t: Table, scales, zp, group: int, n_elem: int, threads: int = 8):
    scales = _c(scales, np.uint16)
    zp = _c(zp, np.int8)
    out = np.zeros(max(n_elem, 1), np.uint16)
    status = np.empty(max(t.n, 1), np.int32)
    lib().ltref_fused_int8(_p(t.comp), t.comp.size, _p(t.comp_off), _p(t.dst_off), t.n, t.total,
                           _p(scales), _p(zp), n_elem, group, _p(out), _p(status), threads)
    return out[:n_elem], status[:t.n]


def fused_int4_chunked(t: Table, scales, zp, group: int, out: np.ndarray, threads: int):
    """Chunk-parallel fused reference writing into `out` (used for timing)."""
    scales = _c(scales, np.uint16)
    zp = _c(zp, np.int8)
    status = np.empty(max(t.n, 1), np.int32)
    bad = lib().ltref_fused_int4_chunked(_p(t.comp), t.comp.size, _p(t.comp_off), _p(t.dst_off),
                                         t.n, t.total, _p(scales), _p(zp), group, _p(out),
                                         _p(status), threads)
    return int(bad), status[:t.n]


# ----------------------------------------------------------------- XXH3-64

def xxh3_64(data) -> int:
    """XXH3 64-bit hash (seed 0, default secret) of a byte buffer."""
    a = _c(np.frombuffer(bytes(data), np.uint8) if isinstance(data, (bytes, bytearray)) else data, np.uint8)
    return int(lib().ltref_xxh3_64(_p(a) if a.size else None, a.size))


def xxh3_chunks(comp: np.ndarray, comp_off: np.ndarray) -> np.ndarray:
    """One XXH3-64 per chunk over its compressed bytes, uint64 [n]."""
    comp = _c(comp, np.uint8)
    comp_off = _c(comp_off, np.uint64)
    n = comp_off.size - 1
    out = np.zeros(max(n, 1), np.uint64)
    if n > 0:
        lib().ltref_xxh3_chunks(_p(comp), _p(comp_off), n, _p(out))
    return out[:n]


# ------------------------------------------------------------- zero runs

ZR_BLOCK = 1024


def zr_encode(x: np.ndarray):
    """Zero-run coding of fp16 bits: (bitmap uint32 [32 per block],
    val_off uint64 [blocks+1], vals uint16 [nonzeros])."""
    x = _c(x, np.uint16).ravel()
    nb = (x.size + ZR_BLOCK - 1) // ZR_BLOCK
    bitmap = np.zeros(max(32 * nb, 1), np.uint32)
    val_off = np.zeros(nb + 1, np.uint64)
    vals = np.zeros(max(x.size, 1), np.uint16)
    m = lib().ltref_zr_encode(_p(x), x.size, _p(bitmap), _p(val_off), _p(vals))
    return bitmap[:32 * nb], val_off, vals[:m].copy()


def zr_decode(bitmap, val_off, vals, n: int, out=None):
    """Inverse of zr_encode; returns (out uint16 [n], status int32 [blocks])."""
    bitmap = _c(bitmap, np.uint32)
    val_off = _c(val_off, np.uint64)
    vals = _c(vals, np.uint16)
    nb = (n + ZR_BLOCK - 1) // ZR_BLOCK
    if out is None:
        out = np.zeros(max(n, 1), np.uint16)
    st = np.zeros(max(nb, 1), np.int32)
    lib().ltref_zr_decode(_p(bitmap), _p(val_off), _p(vals if vals.size else np.zeros(1, np.uint16)), n,
                          vals.size, _p(out), _p(st))
    return out[:n], st[:nb]


# ------------------------------------------------------------- codebooks

def dequant_int4_lut(packed, lut, group: int, n_elem: int | None = None) -> np.ndarray:
    """out[e] = lut[e // group][q(e)]; lut uint16 [groups, 16] of fp16 bits."""
    packed = _c(packed, np.uint8)
    lut = _c(lut, np.uint16)
    n = 2 * packed.size if n_elem is None else n_elem
    out = np.empty(max(n, 1), np.uint16)
    lib().ltref_dequant_int4_lut(_p(packed), n, _p(lut), group, _p(out))
    return out[:n]


# ---------------------------------------------------------- decode + GEMV

def gemm_int4_tiled(t: Table, scales, zp, group: int, rows: int, cols: int, x_f16) -> np.ndarray:
    """Y = X W^T in fp64 for a table whose decoded bytes hold W's INT4 codes
    in tiles of 16 rows x 128 columns (16-row blocks in order, each block's
    column tiles in order, each tile's rows of 64 bytes in turn, low nibble
    first).  Code (r, c) sits in byte ((r // 16) * (cols // 128) + c // 128)
    * 1024 + (r % 16) * 64 + (c % 128) // 2, nibble c % 2.  W is the fp16
    matrix dequant_int4 gives for the codes in row-major order; x fp16 bits
    [batch, cols]; returns (Y float64 [batch, rows], chunk statuses)."""
    data, st = decode_table(t)
    r = np.arange(rows, dtype=np.int64)[:, None]
    c = np.arange(cols, dtype=np.int64)[None, :]
    byte = ((r // 16) * (cols // 128) + c // 128) * 1024 + (r % 16) * 64 + (c % 128) // 2
    codes = (data[byte] >> (4 * (c % 2))) & 15
    W = f64_from_f16(dequant_int4(pack_int4(codes.astype(np.uint8).ravel()), scales, zp, group)).reshape(rows, cols)
    X = f64_from_f16(_c(x_f16, np.uint16)).reshape(-1, cols)
    return X @ W.T, st


def gemv_int4(t: Table, scales, zp, group: int, rows: int, cols: int, x_f16) -> np.ndarray:
    """y = W x in fp64, W = fused_int4(t) as an fp16 rows x cols matrix and
    x fp16 bits [cols]; returns (y float64 [rows], chunk statuses)."""
    w, st = fused_int4(t, scales, zp, group, rows * cols)
    W = f64_from_f16(w).reshape(rows, cols)
    return W @ f64_from_f16(_c(x_f16, np.uint16)), st
