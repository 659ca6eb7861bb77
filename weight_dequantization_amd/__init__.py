"""weight_dequantization_amd -- just-in-time decompression of compressed tensors
on AMD MI355X (gfx950).

A thin ctypes binding over ``liblt.so`` (HIP, built in-tree by
``python -m weight_dequantization_amd.build``).  The names mirror the C ABI in
``include/lt.h``; this module only marshals arguments: every step of the
decode and dequantization runs in the library's kernels.  PyTorch provides
device memory and the current stream.

Device entry points (asynchronous on torch's current stream):
    decode_lz4(table, out=None, status=None)                 -> uint8 tensor
    dequant_int4(packed, scales, zp, shape, group, out=None) -> fp16 tensor
    dequant_int8(q, scales, zp, shape, group, out=None)      -> fp16 tensor
    dequant_int4_lut(packed, lut, shape, group, out=None)   -> fp16 tensor
    fused_lz4_int4(table, scales, zp, shape, group, out=None, status=None)
    fused_lz4_int8(table, scales, zp, shape, group, out=None, status=None)
    fused_lz4_int4_gemv(table, scales, zp, shape, group, x) -> y = W x (fp32)
Zero-run coding of fp16 activations (bitmap + nonzero values per block):
    encode_zero_runs(x) -> (bitmap, val_off, vals)        (host)
    ZeroRunTensor.build(x, device); decode_zero_runs(z, out=None, status=None)
Checksums (CRC-32 per chunk of the compressed bytes, on the device):
    verify_chunks(table, expect=None) -> (got, status)
Chunk ranges (only chunks first .. first+count-1, into a buffer for them):
    decode_lz4_range(table, first, count, out=None, status=None)
    fused_lz4_int4_range(table, scales, zp, shape, group, first, count, ...)
    fused_lz4_int8_range(table, scales, zp, shape, group, first, count, ...)
Streamed entry points (the table in pinned host memory, copies overlapped
with the decode on a second stream):
    stream_decode_lz4(host_table, out=None, status=None, staging=None)
    stream_fused_lz4_int4(host_table, scales, zp, shape, group, out=None, ...)
    stream_fused_lz4_int4_static(host_table, scales, zp, shape, group, out, ...)
        (the same with the library's static workspace: allocates nothing)
Host packer (numpy in, numpy out):
    pack_int4(codes) -> packed bytes (low nibble first)
    compress_chunks(src, dst_off, threads=0, max_dist=0) -> (comp, comp_off)
    index_chunks(comp, comp_off, threads=0) -> (seq_off, seq_pos)
    checksum_chunks(comp, comp_off, threads=0) -> CRC-32 per chunk
    ChunkTable.build(src_bytes, dst_off, device) -> table resident on the GPU
    ChunkTable.build(src_bytes, dst_off, device="cpu", pin=True) -> pinned host table
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblt.so")

ABI_VERSION = 15          # LT_ABI_VERSION of the library this binding speaks to
LT_OK, LT_ERR_INVALID_ARG, LT_ERR_UNSUPPORTED, LT_ERR_LAUNCH, LT_ERR_DEVICE, LT_ERR_TOO_LARGE, LT_ERR_IO = range(7)
STATIC_SCRATCH_BYTES = 32 << 20   # LT_STATIC_SCRATCH_BYTES
(CHUNK_OK, CHUNK_TRUNCATED, CHUNK_BAD_OFFSET, CHUNK_OVERRUN, CHUNK_SIZE_MISMATCH, CHUNK_BAD_TABLE,
 CHUNK_CHECKSUM, CHUNK_STALLED) = range(8)
MAX_CHUNK_BYTES = 1 << 20
SMALL_WINDOW = 11264      # LT_SMALL_WINDOW: tables within it decode with a 16 KiB history
PACK_WINDOW = 4096        # the host packer's default match window (see ChunkTable.build)


class LtError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s" % (where, _lib().lt_status_str(status).decode()))


class LtDecodeError(RuntimeError):
    """Some chunks failed to decode; `chunks` lists (index, code)."""

    def __init__(self, chunks):
        self.chunks = chunks
        super().__init__("%d chunk(s) failed to decode, first: %s" % (len(chunks), chunks[:4]))


class _Table(C.Structure):
    _fields_ = [("comp", C.c_void_p), ("comp_off", C.c_void_p), ("dst_off", C.c_void_p),
                ("n_chunks", C.c_uint32), ("max_chunk_bytes", C.c_uint32),
                ("total_bytes", C.c_uint64), ("comp_bytes", C.c_uint64),
                ("max_dist", C.c_uint32), ("spin_limit", C.c_uint32),
                ("seq_off", C.c_void_p), ("seq_pos", C.c_void_p), ("n_seq", C.c_uint64),
                ("order", C.c_void_p), ("xxh", C.c_void_p)]


class _ZrTensor(C.Structure):
    _fields_ = [("bitmap", C.c_void_p), ("val_off", C.c_void_p), ("vals", C.c_void_p),
                ("n_elem", C.c_uint64), ("n_vals", C.c_uint64)]


ZR_BLOCK = 1024          # LT_ZR_BLOCK

_L = None


def _lib():
    global _L
    if _L is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("liblt.so is not built: run `python -m weight_dequantization_amd.build` "
                              "(or __graft_entry__.build())")
        L = C.CDLL(LIB_PATH)
        vp, u64, u32, i32 = C.c_void_p, C.c_uint64, C.c_uint32, C.c_int
        tp = C.POINTER(_Table)
        sig = {
            "lt_decode_lz4": (i32, [tp, vp, vp, vp]),
            "lt_dequant_int4": (i32, [vp, vp, vp, u64, u64, u64, vp, vp]),
            "lt_dequant_int8": (i32, [vp, vp, vp, u64, u64, u64, vp, vp]),
            "lt_dequant_int4_lut": (i32, [vp, vp, u64, u64, u64, vp, vp]),
            "lt_fused_lz4_int4": (i32, [tp, vp, vp, u64, u64, u64, vp, vp, vp]),
            "lt_fused_lz4_int8": (i32, [tp, vp, vp, u64, u64, u64, vp, vp, vp]),
            "lt_fused_lz4_int4_gemv": (i32, [tp, vp, vp, u64, u64, u64, vp, vp, vp, vp]),
            "lt_decode_lz4_range": (i32, [tp, u32, u32, u64, u64, vp, vp, vp]),
            "lt_fused_lz4_int4_range": (i32, [tp, vp, vp, u64, u64, u64, u32, u32, u64, u64, vp, vp, vp]),
            "lt_fused_lz4_int8_range": (i32, [tp, vp, vp, u64, u64, u64, u32, u32, u64, u64, vp, vp, vp]),
            "lt_stream_decode_lz4": (i32, [tp, vp, vp, vp, u64, vp, vp]),
            "lt_verify_chunks": (i32, [tp, vp, vp, vp, vp]),
            "lt_decode_zero_runs": (i32, [C.POINTER(_ZrTensor), vp, vp, vp]),
            "lt_encode_zero_runs": (i32, [vp, u64, vp, vp, vp, u64, i32]),
            "lt_checksum_chunks": (i32, [vp, vp, u32, vp, i32]),
            "lt_stream_fused_lz4_int4": (i32, [tp, vp, vp, u64, u64, u64, vp, vp, vp, u64, vp, vp]),
            "lt_stream_fused_lz4_int8": (i32, [tp, vp, vp, u64, u64, u64, vp, vp, vp, u64, vp, vp]),
            "lt_stream_file_decode_lz4": (i32, [C.c_int, u64, tp, vp, vp, vp, u64, C.c_int, vp, u64, vp, vp]),
            "lt_stream_file_fused_lz4_int4": (i32, [C.c_int, u64, tp, vp, vp, u64, u64, u64, vp, vp, vp, u64,
                                                    C.c_int, vp, u64, vp, vp]),
            "lt_stream_file_fused_lz4_int8": (i32, [C.c_int, u64, tp, vp, vp, u64, u64, u64, vp, vp, vp, u64,
                                                    C.c_int, vp, u64, vp, vp]),
            "lt_stream_fused_lz4_int4_static": (i32, [tp, vp, vp, u64, u64, u64, vp, vp, vp]),
            "lt_lz4_bound": (u64, [u64]),
            "lt_pack_int4": (i32, [vp, u64, vp]),
            "lt_compress_chunks": (i32, [vp, vp, u32, vp, u64, vp, i32, u32]),
            "lt_compress_chunks_greedy": (i32, [vp, vp, u32, vp, u64, vp, i32, u32]),
            "lt_index_chunks": (i32, [vp, vp, u32, vp, vp, u64, i32]),
            "lt_order_chunks": (i32, [vp, u32, vp]),
            "lt_order_chunks_by_sequences": (i32, [vp, vp, u32, vp]),
            "lt_gemm_workspace_bytes": (u64, [u32, u32]),
            "lt_fused_lz4_int4_gemm": (i32, [tp, vp, vp, u64, u64, u64, vp, u32, vp, vp, u64, vp, vp]),
            "lt_status_str": (C.c_char_p, [i32]),
            "lt_abi_version": (i32, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _L = L
    return _L


def lib():
    """The loaded ctypes library (raises ImportError if it is not built)."""
    return _lib()


# ----------------------------------------------------------------- host side

def _np_ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def pack_int4(codes: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.size // 2, np.uint8)
    st = _lib().lt_pack_int4(_np_ptr(codes), codes.size, _np_ptr(out))
    if st != LT_OK:
        raise LtError(st, "lt_pack_int4")
    return out


def lz4_bound(n: int) -> int:
    return int(_lib().lt_lz4_bound(n))


def compress_chunks(src: np.ndarray, dst_off: np.ndarray, threads: int = 0, max_dist: int = 0,
                    greedy: bool = False):
    """LZ4-compress each chunk independently (matches reach at most max_dist
    bytes back; 0 means the format's 65535).  greedy=True gives the plain
    greedy parse of a general-purpose compressor (4-byte matches, no run
    preference) instead of the packer's own.  Returns (comp, comp_off)."""
    src = np.ascontiguousarray(src, dtype=np.uint8)
    dst_off = np.ascontiguousarray(dst_off, dtype=np.uint64)
    n = dst_off.size - 1
    sizes = np.diff(dst_off.astype(np.int64)) if n > 0 else np.zeros(0, np.int64)
    cap = int(np.sum(sizes + sizes // 255 + 16)) + 16
    comp = np.empty(max(cap, 1), np.uint8)
    comp_off = np.empty(n + 1, np.uint64)
    fn = "lt_compress_chunks_greedy" if greedy else "lt_compress_chunks"
    st = getattr(_lib(), fn)(_np_ptr(src), _np_ptr(dst_off), n, _np_ptr(comp), cap,
                             _np_ptr(comp_off), threads, max_dist)
    if st != LT_OK:
        raise LtError(st, fn)
    return comp[:int(comp_off[-1])].copy(), comp_off


def checksum_chunks(comp: np.ndarray, comp_off: np.ndarray, threads: int = 0) -> np.ndarray:
    """XXH3-64 (seed 0) of each chunk's compressed bytes, uint64 [n]."""
    comp = np.ascontiguousarray(comp, dtype=np.uint8)
    comp_off = np.ascontiguousarray(comp_off, dtype=np.uint64)
    n = comp_off.size - 1
    xxh = np.zeros(max(n, 1), np.uint64)
    st = _lib().lt_checksum_chunks(_np_ptr(comp), _np_ptr(comp_off), max(n, 0), _np_ptr(xxh), threads)
    if st != LT_OK:
        raise LtError(st, "lt_checksum_chunks")
    return xxh[:max(n, 0)]


def encode_zero_runs(x: np.ndarray, threads: int = 0):
    """Zero-run coding of fp16 data (uint16 bits or float16): returns
    (bitmap uint32 [32 per block], val_off uint64 [blocks+1], vals uint16)."""
    x = np.ascontiguousarray(x).view(np.uint16).ravel()
    nb = (x.size + ZR_BLOCK - 1) // ZR_BLOCK
    bitmap = np.zeros(max(32 * nb, 1), np.uint32)
    val_off = np.zeros(nb + 1, np.uint64)
    L = _lib()
    st = L.lt_encode_zero_runs(_np_ptr(x), x.size, _np_ptr(bitmap), _np_ptr(val_off), None, 0, threads)
    if st != LT_OK:
        raise LtError(st, "lt_encode_zero_runs")
    vals = np.zeros(max(int(val_off[-1]), 1), np.uint16)
    st = L.lt_encode_zero_runs(_np_ptr(x), x.size, _np_ptr(bitmap), _np_ptr(val_off), _np_ptr(vals), vals.size,
                               threads)
    if st != LT_OK:
        raise LtError(st, "lt_encode_zero_runs")
    return bitmap[:32 * nb], val_off, vals[:int(val_off[-1])]


def index_chunks(comp: np.ndarray, comp_off: np.ndarray, threads: int = 0):
    """The sequence index of a chunk table: (seq_off uint64[n+1], seq_pos
    uint32[seq_off[-1]]), each chunk's sequence offsets within its block."""
    comp = np.ascontiguousarray(comp, dtype=np.uint8)
    comp_off = np.ascontiguousarray(comp_off, dtype=np.uint64)
    n = comp_off.size - 1
    seq_off = np.zeros(n + 1, np.uint64)
    L = _lib()
    st = L.lt_index_chunks(_np_ptr(comp), _np_ptr(comp_off), n, _np_ptr(seq_off), None, 0, threads)
    if st != LT_OK:
        raise LtError(st, "lt_index_chunks")
    seq_pos = np.zeros(max(int(seq_off[-1]), 1), np.uint32)
    st = L.lt_index_chunks(_np_ptr(comp), _np_ptr(comp_off), n, _np_ptr(seq_off), _np_ptr(seq_pos),
                           seq_pos.size, threads)
    if st != LT_OK:
        raise LtError(st, "lt_index_chunks")
    return seq_off, seq_pos[:int(seq_off[-1])]


def order_chunks(dst_off: np.ndarray, seq_off: np.ndarray = None) -> np.ndarray:
    """A table's launch order (uint32 [n]): chunks by decreasing decoded
    size, chunks of one size in table order, or with the sequence index's
    offsets by decreasing sequence count."""
    dst_off = np.ascontiguousarray(dst_off, np.uint64)
    n = dst_off.size - 1
    order = np.zeros(max(n, 1), np.uint32)
    if seq_off is None:
        st = _lib().lt_order_chunks(_np_ptr(dst_off), max(n, 0), _np_ptr(order))
    else:
        seq_off = np.ascontiguousarray(seq_off, np.uint64)
        if seq_off.size != dst_off.size:
            raise ValueError("seq_off must have one entry per chunk plus one")
        st = _lib().lt_order_chunks_by_sequences(_np_ptr(dst_off), _np_ptr(seq_off), max(n, 0), _np_ptr(order))
    if st != LT_OK:
        raise LtError(st, "lt_order_chunks")
    return order[:n]


# --------------------------------------------------------------- device side

def _torch():
    import torch
    return torch


def _stream_ptr(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _dptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _place(a: np.ndarray, device, pin: bool):
    torch = _torch()
    t = torch.from_numpy(a.copy())
    if pin:
        if torch.device(device).type != "cpu":
            raise ValueError("pin=True places the table in host memory: use device='cpu'")
        return t.pin_memory()
    return t.to(device)


@dataclass
class ChunkTable:
    """A chunk table resident on the GPU (see lt_chunk_table in include/lt.h)."""
    comp: object            # torch.uint8 [comp_bytes]
    comp_off: object        # torch.int64 [n+1] (read as uint64 by the library)
    dst_off: object         # torch.int64 [n+1]
    n_chunks: int
    max_chunk_bytes: int
    total_bytes: int
    comp_bytes: int
    max_dist: int = 0       # declared largest match distance (0: any)
    seq_off: object = None  # torch.int64 [n+1] (read as uint64), or None: no sequence index
    seq_pos: object = None  # torch.int32 [n_seq] (read as uint32)
    n_seq: int = 0
    host_dst_off: object = None   # numpy uint64 [n+1], kept for chunk-range calls
    spin_limit: int = 0     # polls per decoder wave before a wait gives up (0: the library's default)
    order: object = None    # torch.int32 [n] (read as uint32): launch order, or None: table order
    xxh: object = None      # torch.int64 [n] (read as uint64): expected XXH3-64 per chunk, or None: unchecked

    @classmethod
    def from_host(cls, comp: np.ndarray, comp_off: np.ndarray, dst_off: np.ndarray, device="cuda",
                  max_dist: int = 0, index: bool = False, pin: bool = False, order: bool = False,
                  checksum: bool = False):
        """Place a host-built table on `device`; with device="cpu" and
        pin=True the arrays go to pinned host memory, the form the streamed
        entry points read.  index adds the sequence index, order the launch
        order (order_chunks) when the chunks differ in size or the index
        shows a sequence-dense table (3.5 or more sequences per KiB, the
        tables the decoder builds speculatively: then chunks of one size go
        by sequence count), checksum each chunk's XXH3-64 (checksum_chunks),
        which every decode then checks."""
        comp_off = np.ascontiguousarray(comp_off, np.uint64)
        dst_off = np.ascontiguousarray(dst_off, np.uint64)
        n = dst_off.size - 1
        sizes = np.diff(dst_off.astype(np.int64)) if n > 0 else np.zeros(0, np.int64)
        comp = np.ascontiguousarray(comp, np.uint8)
        if comp.size == 0:
            comp = np.zeros(16, np.uint8)
        t = cls(_place(comp, device, pin), _place(comp_off.view(np.int64), device, pin),
                _place(dst_off.view(np.int64), device, pin),
                n, max(1, int(sizes.max())) if n > 0 else 0, int(dst_off[-1]) if n >= 0 else 0,
                int(comp_off[-1]) if comp_off.size else 0, max_dist)
        t.host_dst_off = dst_off.copy()
        seq_off = None
        if index and n > 0:
            seq_off, seq_pos = index_chunks(comp, comp_off)
            t.set_index(seq_off, seq_pos, device, pin)
        dense = seq_off is not None and int(seq_off[-1]) * 2048 >= 7 * int(dst_off[-1])
        if order and n > 0 and dense:
            t.order = _place(order_chunks(dst_off, seq_off).view(np.int32), device, pin)
        elif order and n > 0 and np.unique(sizes).size > 1:   # one size: table order already
            t.order = _place(order_chunks(dst_off).view(np.int32), device, pin)
        if checksum and n > 0:
            t.xxh = _place(checksum_chunks(comp, comp_off).view(np.int64), device, pin)
        return t

    def set_index(self, seq_off: np.ndarray, seq_pos: np.ndarray, device=None, pin: bool = None):
        """Attach a sequence index (host arrays, as index_chunks returns)."""
        device = device if device is not None else self.comp.device
        pin = self.comp.device.type == "cpu" and self.comp.is_pinned() if pin is None else pin
        seq_off = np.ascontiguousarray(seq_off, np.uint64)
        seq_pos = np.ascontiguousarray(seq_pos, np.uint32)
        self.n_seq = int(seq_pos.size)
        if seq_pos.size == 0:
            seq_pos = np.zeros(1, np.uint32)
        self.seq_off = _place(seq_off.view(np.int64), device, pin)
        self.seq_pos = _place(seq_pos.view(np.int32), device, pin)

    def pinned_bytes(self, chunks_per_half: int = 512) -> int:
        """A pinned host buffer size for the file-streaming entry points: two
        halves that each hold the compressed bytes of the largest
        `chunks_per_half` consecutive chunks (rounded up to 256 bytes)."""
        up = lambda x: (x + 255) // 256 * 256
        n = self.n_chunks
        if n == 0:
            return 2 * 256
        k = max(1, min(int(chunks_per_half), n))
        co = self.comp_off.cpu().numpy().astype(np.int64)
        return 2 * up(int(np.max(co[k:] - co[:-k])))

    def staging_bytes(self, chunks_per_half: int = 512) -> int:
        """A staging size for the streamed entry points: the table's offsets,
        checksums and index, then two halves that each hold the compressed bytes of
        the largest `chunks_per_half` consecutive chunks (the library's
        layout: every piece rounded up to 256 bytes)."""
        up = lambda x: (x + 255) // 256 * 256
        n = self.n_chunks
        if n == 0:
            return 2 * 256
        k = max(1, min(int(chunks_per_half), n))
        co = self.comp_off.cpu().numpy().astype(np.int64)
        meta = 2 * up(8 * (n + 1))
        if self.xxh is not None:
            meta += up(8 * n)
        if self.seq_off is not None:
            meta += up(8 * (n + 1)) + up(4 * int(self.seq_off[-1]))
        return meta + 2 * up(int(np.max(co[k:] - co[:-k])) + 16)

    @classmethod
    def build(cls, src: np.ndarray, dst_off: np.ndarray, device="cuda", threads: int = 0,
              max_dist: int = None, index: bool = True, pin: bool = False, greedy: bool = False,
              order: bool = True, checksum: bool = False):
        """Compress `src` chunk by chunk on the host and upload the table.  By
        default matches stay within PACK_WINDOW bytes, which the table
        declares, so the device decoder keeps a short history per chunk, and
        the table carries the sequence index, so each chunk's sequences are
        parsed side by side, and a launch order that starts the largest
        chunks first (on sequence-dense tables, then those with the most
        sequences).  greedy=True packs with the plain greedy parse
        (compress_chunks); checksum=True stores each chunk's XXH3-64, which
        every decode of the table then checks."""
        if max_dist is None:
            max_dist = PACK_WINDOW
        comp, comp_off = compress_chunks(src, dst_off, threads, max_dist, greedy)
        return cls.from_host(comp, comp_off, dst_off, device, max_dist, index, pin, order, checksum)

    @classmethod
    def build_concat(cls, srcs, dst_offs, device="cuda", **kw):
        """One table over several tensors decoded back to back, such as the
        projections of one model layer: tensor i's chunks follow tensor
        i - 1's (chunk boundaries as in dst_offs[i]), and its decoded bytes
        start at starts[i].  Chunks are independent, so this is the tensors'
        tables laid end to end; one launch over it decodes them all, and the
        launch order (largest chunks first) spans the whole set.  The
        tensors' scales and zero points go end to end likewise, so each
        tensor's groups must end where it ends.  Keyword arguments as for
        build.  Returns (table, starts)."""
        srcs = [np.ascontiguousarray(s, np.uint8).ravel() for s in srcs]
        if len(srcs) == 0 or len(srcs) != len(dst_offs):
            raise ValueError("one dst_off per tensor, at least one tensor")
        starts = np.cumsum([0] + [s.size for s in srcs]).astype(np.uint64)
        parts = []
        for i, (s, d) in enumerate(zip(srcs, dst_offs)):
            d = np.ascontiguousarray(d, np.uint64)
            if d.size < 2 or d[0] != 0 or d[-1] != s.size or np.any(np.diff(d.astype(np.int64)) <= 0):
                raise ValueError("dst_offs[%d] must rise from 0 to the tensor's size" % i)
            parts.append(d[(0 if i == 0 else 1):] + starts[i])
        table = cls.build(np.concatenate(srcs), np.concatenate(parts), device, **kw)
        return table, starts[:-1]

    def as_c(self) -> _Table:
        return _Table(self.comp.data_ptr(), self.comp_off.data_ptr(), self.dst_off.data_ptr(),
                      self.n_chunks, self.max_chunk_bytes, self.total_bytes, self.comp_bytes,
                      self.max_dist, self.spin_limit,
                      self.seq_off.data_ptr() if self.seq_off is not None else None,
                      self.seq_pos.data_ptr() if self.seq_pos is not None else None,
                      self.n_seq if self.seq_off is not None else 0,
                      self.order.data_ptr() if self.order is not None else None,
                      self.xxh.data_ptr() if self.xxh is not None else None)


def _check(st, where):
    if st != LT_OK:
        raise LtError(st, where)


def check_status(status) -> None:
    """Raise LtDecodeError if any chunk status is not OK (synchronizes)."""
    s = status.cpu().numpy()
    bad = np.nonzero(s != CHUNK_OK)[0]
    if bad.size:
        raise LtDecodeError([(int(i), int(s[i])) for i in bad])


def decode_lz4(table: ChunkTable, out=None, status=None, stream=None):
    torch = _torch()
    if out is None:
        out = torch.empty(max(table.total_bytes, 1), dtype=torch.uint8, device=table.comp.device)
    t = table.as_c()
    _check(_lib().lt_decode_lz4(C.byref(t), _dptr(out), _dptr(status), _stream_ptr(stream)),
           "lt_decode_lz4")
    return out[:table.total_bytes] if out.numel() > table.total_bytes else out


def _out_f16(out, n, device):
    torch = _torch()
    if out is None:
        out = torch.empty(n, dtype=torch.float16, device=device)
    return out


def _shape(shape):
    rows, cols = (int(shape[0]), int(shape[1])) if len(shape) == 2 else (1, int(shape[0]))
    return rows, cols


def dequant_int4(packed, scales, zp, shape, group: int, out=None, stream=None):
    rows, cols = _shape(shape)
    out = _out_f16(out, rows * cols, packed.device)
    _check(_lib().lt_dequant_int4(_dptr(packed), _dptr(scales), _dptr(zp), rows, cols, group,
                                  _dptr(out), _stream_ptr(stream)), "lt_dequant_int4")
    return out.view(rows, cols)


def dequant_int8(q, scales, zp, shape, group: int, out=None, stream=None):
    rows, cols = _shape(shape)
    out = _out_f16(out, rows * cols, q.device)
    _check(_lib().lt_dequant_int8(_dptr(q), _dptr(scales), _dptr(zp), rows, cols, group,
                                  _dptr(out), _stream_ptr(stream)), "lt_dequant_int8")
    return out.view(rows, cols)


def dequant_int4_lut(packed, lut, shape, group: int, out=None, stream=None):
    """Codebook dequant: element e is lut[e // group][q(e)]; lut is a device
    tensor of fp16 bits (int16/uint16/float16) [groups, 16]."""
    rows, cols = _shape(shape)
    out = _out_f16(out, rows * cols, packed.device)
    _check(_lib().lt_dequant_int4_lut(_dptr(packed), _dptr(lut), rows, cols, group, _dptr(out),
                                      _stream_ptr(stream)), "lt_dequant_int4_lut")
    return out.view(rows, cols)


def fused_lz4_int4(table: ChunkTable, scales, zp, shape, group: int, out=None, status=None,
                   stream=None):
    rows, cols = _shape(shape)
    out = _out_f16(out, rows * cols, table.comp.device)
    t = table.as_c()
    _check(_lib().lt_fused_lz4_int4(C.byref(t), _dptr(scales), _dptr(zp), rows, cols, group,
                                    _dptr(out), _dptr(status), _stream_ptr(stream)),
           "lt_fused_lz4_int4")
    return out.view(rows, cols)


def fused_lz4_int4_gemv(table: ChunkTable, scales, zp, shape, group: int, x, y=None, status=None,
                        stream=None):
    """y = W x with W the fp16 matrix fused_lz4_int4 would write, never
    stored: x fp16 [cols] on the device; returns y fp32 [rows]."""
    torch = _torch()
    rows, cols = _shape(shape)
    if y is None:
        y = torch.empty(rows, dtype=torch.float32, device=table.comp.device)
    t = table.as_c()
    _check(_lib().lt_fused_lz4_int4_gemv(C.byref(t), _dptr(scales), _dptr(zp), rows, cols, group, _dptr(x),
                                         _dptr(y), _dptr(status), _stream_ptr(stream)), "lt_fused_lz4_int4_gemv")
    return y


def pack_int4_tiles(codes: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """INT4 codes [rows, cols] (values 0..15, row-major) in the GEMM layout:
    tiles of 16 rows x 128 columns, the 16-row blocks in order and each
    block's column tiles in order, each tile's 16 rows of 64 bytes in turn,
    two codes per byte, low nibble first.  rows % 16 == 0, cols % 128 == 0."""
    if rows % 16 or cols % 128:
        raise ValueError("the GEMM layout needs rows % 16 == 0 and cols % 128 == 0")
    c = np.ascontiguousarray(codes, np.uint8).reshape(rows // 16, 16, cols // 128, 128)
    return pack_int4(np.ascontiguousarray(c.transpose(0, 2, 1, 3)).ravel())


def gemm_chunks(rows: int, cols: int, tiles_per_chunk: int = 56) -> np.ndarray:
    """Chunk boundaries (dst_off) for a GEMM-layout table: each 16-row
    block's cols / 128 tiles cut into chunks of tiles_per_chunk tiles (the
    block's last chunk holds the rest), so no chunk spans two blocks."""
    tpr = cols // 128
    cuts = list(range(tiles_per_chunk, tpr, tiles_per_chunk)) + [tpr]
    per = np.array(cuts, np.uint64) * 1024
    base = np.arange(rows // 16, dtype=np.uint64)[:, None] * np.uint64(tpr * 1024)
    return np.concatenate([np.zeros(1, np.uint64), (base + per[None, :]).ravel()])


def gemm_workspace_bytes(n_chunks: int, batch: int) -> int:
    return int(_lib().lt_gemm_workspace_bytes(n_chunks, batch))


def fused_lz4_int4_gemm(table: ChunkTable, scales, zp, shape, group: int, x, y=None, workspace=None, status=None,
                        stream=None):
    """Y = X W^T, with W [rows, cols] the fp16 matrix fused_lz4_int4 would
    write from the same codes, never stored: the table holds W's codes in
    the GEMM layout (pack_int4_tiles, chunked by gemm_chunks); x fp16
    [batch, cols] on the device, batch 16 or 32; returns y fp32 [batch, rows].
    The partial products go to `workspace` (allocated here when None)."""
    torch = _torch()
    rows, cols = _shape(shape)
    if x.dim() != 2 or int(x.shape[1]) != cols:
        raise ValueError("x must be [batch, cols]")
    batch = int(x.shape[0])
    dev = table.comp.device
    if y is None:
        y = torch.empty((batch, rows), dtype=torch.float32, device=dev)
    own = workspace is None
    if own:
        workspace = torch.empty(max(gemm_workspace_bytes(table.n_chunks, batch) // 4, 4), dtype=torch.float32,
                                device=dev)
    t = table.as_c()
    _check(_lib().lt_fused_lz4_int4_gemm(C.byref(t), _dptr(scales), _dptr(zp), rows, cols, group, _dptr(x), batch,
                                         _dptr(y), _dptr(workspace), workspace.numel() * 4, _dptr(status),
                                         _stream_ptr(stream)), "lt_fused_lz4_int4_gemm")
    if own:   # dropped on return while the launch still uses it
        workspace.record_stream(stream if stream is not None else torch.cuda.current_stream(dev))
    return y


def fused_lz4_int8(table: ChunkTable, scales, zp, shape, group: int, out=None, status=None,
                   stream=None):
    rows, cols = _shape(shape)
    out = _out_f16(out, rows * cols, table.comp.device)
    t = table.as_c()
    _check(_lib().lt_fused_lz4_int8(C.byref(t), _dptr(scales), _dptr(zp), rows, cols, group,
                                    _dptr(out), _dptr(status), _stream_ptr(stream)),
           "lt_fused_lz4_int8")
    return out.view(rows, cols)


# -------------------------------------------------------------- zero runs

@dataclass
class ZeroRunTensor:
    """A zero-run coded fp16 tensor resident on the GPU (lt_zr_tensor)."""
    bitmap: object          # torch.int32 [32 per block] (read as uint32)
    val_off: object         # torch.int64 [blocks+1] (read as uint64)
    vals: object            # torch.int16 [n_vals] (fp16 bits)
    n_elem: int
    n_vals: int

    @classmethod
    def build(cls, x: np.ndarray, device="cuda", threads: int = 0):
        """Encode on the host (encode_zero_runs) and upload."""
        bitmap, val_off, vals = encode_zero_runs(x, threads)
        return cls.from_host(bitmap, val_off, vals, int(np.asarray(x).size), device)

    @classmethod
    def from_host(cls, bitmap, val_off, vals, n_elem: int, device="cuda"):
        torch = _torch()
        bitmap = np.ascontiguousarray(bitmap, np.uint32)
        vals = np.ascontiguousarray(vals, np.uint16)
        n_vals = int(vals.size)
        return cls(torch.from_numpy((bitmap if bitmap.size else np.zeros(1, np.uint32)).view(np.int32).copy()).to(device),
                   torch.from_numpy(np.ascontiguousarray(val_off, np.uint64).view(np.int64).copy()).to(device),
                   torch.from_numpy((vals if vals.size else np.zeros(8, np.uint16)).view(np.int16).copy()).to(device),
                   int(n_elem), n_vals)

    def as_c(self) -> _ZrTensor:
        return _ZrTensor(self.bitmap.data_ptr(), self.val_off.data_ptr(), self.vals.data_ptr(), self.n_elem,
                         self.n_vals)


def decode_zero_runs(z: ZeroRunTensor, out=None, status=None, stream=None):
    """Expand a zero-run coded tensor into fp16 (flat [n_elem])."""
    torch = _torch()
    if out is None:
        out = torch.empty(max(z.n_elem, 1), dtype=torch.float16, device=z.bitmap.device)
    c = z.as_c()
    _check(_lib().lt_decode_zero_runs(C.byref(c), _dptr(out), _dptr(status), _stream_ptr(stream)),
           "lt_decode_zero_runs")
    return out[:z.n_elem] if out.numel() > z.n_elem else out


# --------------------------------------------------------------- checksums

def verify_chunks(table: ChunkTable, expect=None, got=None, status=None, stream=None):
    """XXH3-64 of each chunk's compressed bytes on the device, without
    decoding.  With `expect` (device int64 [n], the uint64 values
    checksum_chunks computes) each chunk's status is CHUNK_OK or
    CHUNK_CHECKSUM; returns (got, status)."""
    torch = _torch()
    dev = table.comp.device
    if got is None:
        got = torch.empty(max(table.n_chunks, 1), dtype=torch.int64, device=dev)
    if status is None and expect is not None:
        status = torch.empty(max(table.n_chunks, 1), dtype=torch.int32, device=dev)
    t = table.as_c()
    _check(_lib().lt_verify_chunks(C.byref(t), _dptr(expect), _dptr(got), _dptr(status), _stream_ptr(stream)),
           "lt_verify_chunks")
    return got, status


# -------------------------------------------------------------- chunk range

def _range_bounds(table: ChunkTable, first: int, count: int):
    if first < 0 or count < 0 or first + count > table.n_chunks:
        raise LtError(LT_ERR_INVALID_ARG, "chunk range")
    d = table.host_dst_off
    if d is None:
        d = table.dst_off.cpu().numpy().view(np.uint64)
    return int(d[first]), int(d[first + count])


def decode_lz4_range(table: ChunkTable, first: int, count: int, out=None, status=None, stream=None):
    """Decode chunks first .. first+count-1 only; `out` receives their bytes
    from offset 0 (the decoded stream's bytes dst_off[first] ..
    dst_off[first+count])."""
    torch = _torch()
    lo, hi = _range_bounds(table, first, count)
    if out is None:
        out = torch.empty(max(hi - lo, 1), dtype=torch.uint8, device=table.comp.device)
    t = table.as_c()
    _check(_lib().lt_decode_lz4_range(C.byref(t), first, count, lo, hi, _dptr(out), _dptr(status),
                                      _stream_ptr(stream)), "lt_decode_lz4_range")
    return out[:hi - lo] if out.numel() > hi - lo else out


def _fused_range(fn, name, per_byte, table, scales, zp, shape, group, first, count, out, status, stream):
    rows, cols = _shape(shape)
    lo, hi = _range_bounds(table, first, count)
    out = _out_f16(out, max(per_byte * (hi - lo), 1), table.comp.device)
    t = table.as_c()
    _check(fn(C.byref(t), _dptr(scales), _dptr(zp), rows, cols, group, first, count, lo, hi, _dptr(out),
              _dptr(status), _stream_ptr(stream)), name)
    n = per_byte * (hi - lo)
    return out[:n] if out.numel() > n else out


def fused_lz4_int4_range(table: ChunkTable, scales, zp, shape, group: int, first: int, count: int,
                         out=None, status=None, stream=None):
    """fused_lz4_int4 over chunks first .. first+count-1 only: `out` (flat)
    receives elements 2*dst_off[first] .. 2*dst_off[first+count] of the
    tensor; shape, scales and zero points describe the whole tensor."""
    return _fused_range(_lib().lt_fused_lz4_int4_range, "lt_fused_lz4_int4_range", 2, table, scales, zp,
                        shape, group, first, count, out, status, stream)


def fused_lz4_int8_range(table: ChunkTable, scales, zp, shape, group: int, first: int, count: int,
                         out=None, status=None, stream=None):
    """fused_lz4_int8 over chunks first .. first+count-1 only (elements
    dst_off[first] .. dst_off[first+count])."""
    return _fused_range(_lib().lt_fused_lz4_int8_range, "lt_fused_lz4_int8_range", 1, table, scales, zp,
                        shape, group, first, count, out, status, stream)


# ------------------------------------------------------------------ streamed

_COPY_STREAMS = {}


def _copy_stream(device):
    torch = _torch()
    key = torch.cuda.current_device() if device is None else torch.device(device).index
    if key is None:
        key = torch.cuda.current_device()
    if key not in _COPY_STREAMS:
        _COPY_STREAMS[key] = torch.cuda.Stream(device=key)      # default priority
    return _COPY_STREAMS[key]


def _stream_setup(table: ChunkTable, out_device, staging, copy_stream):
    """(staging, copy_stream, owned): owned is True when the staging buffer
    was allocated here (it must then be tied to the streams that use it)."""
    torch = _torch()
    if table.comp.device.type != "cpu":
        raise ValueError("the streamed entry points read a host table (ChunkTable.build(..., "
                         "device='cpu', pin=True))")
    owned = staging is None
    if owned:
        staging = torch.empty(table.staging_bytes(), dtype=torch.uint8, device=out_device)
    if copy_stream is None:
        copy_stream = _copy_stream(out_device)
    return staging, copy_stream, owned


def _stream_release(staging, owned, copy_stream, stream):
    """A staging buffer allocated by the binding is dropped when the call
    returns, while the copies (copy_stream) and decodes (stream) still use it:
    recording both streams keeps the caching allocator from handing its
    memory to a new tensor before that work has finished."""
    if owned:
        torch = _torch()
        staging.record_stream(copy_stream)
        staging.record_stream(stream if stream is not None else torch.cuda.current_stream(staging.device))


def stream_decode_lz4(table: ChunkTable, out=None, status=None, staging=None, copy_stream=None,
                      stream=None, device="cuda"):
    """Decode a host-resident table: batches are copied to the two halves of
    `staging` on `copy_stream` while the previous batch decodes on `stream`.
    The host arrays must stay unchanged until `stream` has passed this call."""
    torch = _torch()
    if out is None:
        out = torch.empty(max(table.total_bytes, 1), dtype=torch.uint8, device=device)
    staging, copy_stream, owned = _stream_setup(table, out.device, staging, copy_stream)
    t = table.as_c()
    _check(_lib().lt_stream_decode_lz4(C.byref(t), _dptr(out), _dptr(status), _dptr(staging),
                                       staging.numel(), _stream_ptr(copy_stream), _stream_ptr(stream)),
           "lt_stream_decode_lz4")
    _stream_release(staging, owned, copy_stream, stream)
    return out[:table.total_bytes] if out.numel() > table.total_bytes else out


def _stream_fused(name, table, scales, zp, shape, group, out, status, staging, copy_stream, stream):
    rows, cols = _shape(shape)
    out = _out_f16(out, rows * cols, scales.device)
    staging, copy_stream, owned = _stream_setup(table, out.device, staging, copy_stream)
    t = table.as_c()
    _check(getattr(_lib(), name)(C.byref(t), _dptr(scales), _dptr(zp), rows, cols, group, _dptr(out),
                                 _dptr(status), _dptr(staging), staging.numel(), _stream_ptr(copy_stream),
                                 _stream_ptr(stream)), name)
    _stream_release(staging, owned, copy_stream, stream)
    return out.view(rows, cols)


def stream_fused_lz4_int4(table: ChunkTable, scales, zp, shape, group: int, out=None, status=None,
                          staging=None, copy_stream=None, stream=None):
    """fused_lz4_int4 over a host-resident table, copies overlapped with the
    decode as in stream_decode_lz4."""
    return _stream_fused("lt_stream_fused_lz4_int4", table, scales, zp, shape, group, out, status, staging,
                         copy_stream, stream)


def stream_fused_lz4_int8(table: ChunkTable, scales, zp, shape, group: int, out=None, status=None,
                          staging=None, copy_stream=None, stream=None):
    """fused_lz4_int8 over a host-resident table, as stream_fused_lz4_int4."""
    return _stream_fused("lt_stream_fused_lz4_int8", table, scales, zp, shape, group, out, status, staging,
                         copy_stream, stream)


def _stream_file(name, fd, file_offset, table, mid, out, status, pinned, staging, copy_stream, stream, read_threads):
    """Run a file-streaming entry point.  fd is a file descriptor or a path
    (opened and closed here; the reads are done when the call returns)."""
    torch = _torch()
    staging, copy_stream, owned = _stream_setup(table, out.device, staging, copy_stream)
    own_pin = pinned is None
    if own_pin:
        pinned = torch.empty(table.pinned_bytes(), dtype=torch.uint8, pin_memory=True)
    close = isinstance(fd, (str, bytes, os.PathLike))
    if close:
        fd = os.open(fd, os.O_RDONLY)
    try:
        t = table.as_c()
        _check(getattr(_lib(), name)(fd, int(file_offset), C.byref(t), *mid, _dptr(out), _dptr(status), _dptr(pinned),
                                     pinned.numel(), int(read_threads), _dptr(staging), staging.numel(),
                                     _stream_ptr(copy_stream), _stream_ptr(stream)), name)
    finally:
        if close:
            os.close(fd)
        _stream_release(staging, owned, copy_stream, stream)
        if own_pin:   # the copies read the pinned buffer allocated here
            copy_stream.synchronize()
    return out


def stream_file_decode_lz4(fd, file_offset: int, table: ChunkTable, out=None, status=None, pinned=None,
                           staging=None, read_threads: int = 8, copy_stream=None, stream=None, device="cuda"):
    """stream_decode_lz4 with the compressed bytes read from a file (chunk
    i's at file_offset + comp_off[i]): each batch is read with pread into a
    pinned half while the batches before it are copied and decoded.  `table`
    is a host table whose comp array is not read."""
    torch = _torch()
    if out is None:
        out = torch.empty(max(table.total_bytes, 1), dtype=torch.uint8, device=device)
    _stream_file("lt_stream_file_decode_lz4", fd, file_offset, table, (), out, status, pinned, staging,
                 copy_stream, stream, read_threads)
    return out[:table.total_bytes] if out.numel() > table.total_bytes else out


def _stream_file_fused(name, fd, file_offset, table, scales, zp, shape, group, out, status, pinned, staging,
                       read_threads, copy_stream, stream):
    rows, cols = _shape(shape)
    out = _out_f16(out, rows * cols, scales.device)
    _stream_file(name, fd, file_offset, table, (_dptr(scales), _dptr(zp), rows, cols, group), out, status, pinned,
                 staging, copy_stream, stream, read_threads)
    return out.view(rows, cols)


def stream_file_fused_lz4_int4(fd, file_offset: int, table: ChunkTable, scales, zp, shape, group: int, out=None,
                               status=None, pinned=None, staging=None, read_threads: int = 8, copy_stream=None,
                               stream=None):
    """stream_fused_lz4_int4 with the compressed bytes read from a file, as
    stream_file_decode_lz4."""
    return _stream_file_fused("lt_stream_file_fused_lz4_int4", fd, file_offset, table, scales, zp, shape, group,
                              out, status, pinned, staging, read_threads, copy_stream, stream)


def stream_file_fused_lz4_int8(fd, file_offset: int, table: ChunkTable, scales, zp, shape, group: int, out=None,
                               status=None, pinned=None, staging=None, read_threads: int = 8, copy_stream=None,
                               stream=None):
    """stream_fused_lz4_int8 with the compressed bytes read from a file."""
    return _stream_file_fused("lt_stream_file_fused_lz4_int8", fd, file_offset, table, scales, zp, shape, group,
                              out, status, pinned, staging, read_threads, copy_stream, stream)


def stream_fused_lz4_int4_static(table: ChunkTable, scales, zp, shape, group: int, out=None, status=None,
                                 stream=None):
    """fused_lz4_int4 over a host-resident table through the library's static
    workspace (lt_stream_fused_lz4_int4_static): nothing is allocated by the
    call, the copies and the decode run in order on `stream`, and calls that
    overlap on one GPU race on the shared workspace."""
    if table.comp.device.type != "cpu":
        raise ValueError("the streamed entry points read a host table (ChunkTable.build(..., "
                         "device='cpu', pin=True))")
    rows, cols = _shape(shape)
    if out is None:
        raise ValueError("stream_fused_lz4_int4_static writes into a caller-owned `out` (it allocates nothing)")
    t = table.as_c()
    _check(_lib().lt_stream_fused_lz4_int4_static(C.byref(t), _dptr(scales), _dptr(zp), rows, cols, group,
                                                  _dptr(out), _dptr(status), _stream_ptr(stream)),
           "lt_stream_fused_lz4_int4_static")
    return out.view(rows, cols)
