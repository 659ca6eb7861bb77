"""Seeded synthetic inputs for the just-in-time tensor decompression path.

This module only draws random numbers and lays them out: INT4/INT8 codes,
fp16 scales, int8 zero points, ReLU activation values and the chunk
boundaries of a tensor's byte stream. It holds none of the method's
arithmetic: nothing here packs nibbles, compresses, decodes or dequantizes.
Both the CPU oracle and the HIP path take their inputs from here.

Workloads (shapes and value distributions) stand in for the real quantized
model weights and captured activations that the pages measure on and that are
not available here:

* tiny_int4_1024       INT4 weight 1024x1024, group 256, zero point 8, 30% all-zero groups
* int8_8192x8192       INT8 per-row 8192x8192, N(0,1)*32 rounded and clipped, half the rows pruned
* mlp_int4_8192x28672  INT4 MLP projection 8192x28672, group 128, zero points U{0..15},
                       codes rounded N(7.5, 3) clipped to 0..15, 20% all-zero groups
* relu_4096x14336      ReLU activations 4096x14336 fp16, max(0, N(0,1) - 1.3), with stress chunks
* llama70b_tensor      80 Llama-70B-shaped layers of INT4 projections, group 128, chunks of
                       16/64/256 KiB mixed per chunk

Scales are drawn in float64 and rounded to fp16 with numpy's round-to-nearest-even
conversion; they are returned as raw fp16 bit patterns (uint16).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

KIB = 1024
CHUNK_64K = 64 * KIB


# ---------------------------------------------------------------- primitives

def fp16_bits(x: np.ndarray) -> np.ndarray:
    """float64 draws -> fp16 bit patterns (numpy RNE conversion)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def _normal_code_table(mean: float, sd: float, lo: int = 0, hi: int = 15) -> np.ndarray:
    """Inverse-CDF table: uniform 16-bit draw -> code, so that
    P(code = k) = P(clip(rint(N(mean, sd)), lo, hi) = k) up to 2^-16."""
    def phi(x):
        return 0.5 * (1.0 + math.erf((x - mean) / (sd * math.sqrt(2.0))))
    cdf = [phi(k + 0.5) for k in range(lo, hi)] + [1.0]   # P(code <= k)
    edges = np.round(np.asarray(cdf) * 65536.0).astype(np.int64)
    table = np.empty(65536, dtype=np.uint8)
    start = 0
    for k, end in zip(range(lo, hi + 1), edges):
        table[start:end] = k
        start = max(start, int(end))
    table[start:] = hi
    return table


_TABLE_N75_3 = None


def normal_codes(rng: np.random.Generator, n: int, mean=7.5, sd=3.0) -> np.ndarray:
    """n codes distributed as clip(rint(N(mean, sd)), 0, 15), as uint8."""
    global _TABLE_N75_3
    if mean == 7.5 and sd == 3.0:
        if _TABLE_N75_3 is None:
            _TABLE_N75_3 = _normal_code_table(7.5, 3.0)
        table = _TABLE_N75_3
    else:
        table = _normal_code_table(mean, sd)
    return table[rng.integers(0, 65536, size=n, dtype=np.uint16)]


def uniform_chunks(total: int, chunk: int = CHUNK_64K) -> np.ndarray:
    """Chunk boundaries [0, chunk, 2*chunk, ..., total] (last chunk ragged)."""
    if total == 0:
        return np.zeros(1, dtype=np.uint64)
    b = np.arange(0, total, chunk, dtype=np.uint64)
    return np.append(b, np.uint64(total))


def mixed_chunks(rng: np.random.Generator, total: int,
                 sizes=(16 * KIB, 64 * KIB, 256 * KIB)) -> np.ndarray:
    """Chunk boundaries with each chunk's size drawn uniformly from `sizes`."""
    bounds = [0]
    pos = 0
    # draw more sizes than needed in one go; the minimum size bounds the count
    draws = rng.integers(0, len(sizes), size=total // min(sizes) + 2)
    i = 0
    while pos < total:
        pos = min(total, pos + sizes[int(draws[i])])
        bounds.append(pos)
        i += 1
    return np.asarray(bounds, dtype=np.uint64)


# ---------------------------------------------------------------- workloads

@dataclass
class Int4Weight:
    rows: int
    cols: int
    group: int
    codes: np.ndarray          # uint8 [rows*cols], values 0..15
    scales: np.ndarray         # uint16 fp16 bits [rows*cols/group]
    zp: np.ndarray | None      # int8 [rows*cols/group] or None
    dst_off: np.ndarray        # uint64 chunk boundaries over the packed byte stream
    seed: object = None

    @property
    def packed_bytes(self) -> int:
        return self.rows * self.cols // 2


@dataclass
class Int8Weight:
    rows: int
    cols: int
    group: int
    q: np.ndarray              # int8 [rows*cols]
    scales: np.ndarray         # uint16 fp16 bits [rows*cols/group]
    zp: np.ndarray | None
    dst_off: np.ndarray
    seed: object = None


@dataclass
class Activation:
    shape: tuple
    data: np.ndarray           # uint8 [nbytes]: the fp16 tensor's bytes, little-endian
    dst_off: np.ndarray
    stress: dict = field(default_factory=dict)
    seed: object = None


def _zero_groups(rng, codes, group, frac):
    n_groups = codes.size // group
    k = int(round(frac * n_groups))
    sel = rng.choice(n_groups, size=k, replace=False)
    codes.reshape(n_groups, group)[sel, :] = 0
    return sel


def int4_weight(rows, cols, group, seed, *, code_dist="normal", zero_frac=0.2,
                zp_mode="uniform16", scale_lo=0.005, scale_hi=0.05,
                chunking="64k") -> Int4Weight:
    rng = np.random.default_rng(seed)
    n = rows * cols
    if code_dist == "uniform":
        codes = rng.integers(0, 16, size=n, dtype=np.uint8)
    else:
        codes = normal_codes(rng, n)
    _zero_groups(rng, codes, group, zero_frac)
    n_groups = n // group
    scales = fp16_bits(rng.uniform(scale_lo, scale_hi, size=n_groups))
    if zp_mode == "uniform16":
        zp = rng.integers(0, 16, size=n_groups, dtype=np.int64).astype(np.int8)
    elif zp_mode is None:
        zp = None
    else:
        zp = np.full(n_groups, int(zp_mode), dtype=np.int8)
    packed = n // 2
    dst_off = mixed_chunks(rng, packed) if chunking == "mixed" else uniform_chunks(packed)
    return Int4Weight(rows, cols, group, codes, scales, zp, dst_off, seed)


def tiny_int4_1024() -> Int4Weight:
    """Tiny INT4 weight: 1024x1024, group 256 along rows, zp 8, codes U{0..15},
    exactly round(0.3 * 4096) = 1229 all-zero groups, 64 KiB chunks."""
    return int4_weight(1024, 1024, 256, 1001, code_dist="uniform", zero_frac=0.30,
                       zp_mode=8, scale_lo=0.005, scale_hi=0.05)


def int8_8192x8192() -> Int8Weight:
    """INT8 per-channel: 8192x8192, q = clip(rint(N(0,1)*32), -127, 127),
    exactly 4096 zero rows, per-row fp16 scales U(1e-3, 1e-2), no zero point."""
    rng = np.random.default_rng(1002)
    R = C = 8192
    q = np.clip(np.rint(rng.standard_normal(R * C) * 32.0), -127, 127).astype(np.int8)
    rows = rng.choice(R, size=R // 2, replace=False)
    q.reshape(R, C)[rows, :] = 0
    scales = fp16_bits(rng.uniform(1e-3, 1e-2, size=R))
    return Int8Weight(R, C, C, q, scales, None, uniform_chunks(R * C), 1002)


def mlp_int4_8192x28672() -> Int4Weight:
    """Fused LZ4+INT4 MLP layer: 8192x28672, group 128, zp U{0..15},
    codes clip(rint(N(7.5, 3)), 0, 15), 20% all-zero groups, 64 KiB chunks."""
    return int4_weight(8192, 28672, 128, 1003)


def mlp_int4_small(rows=256, cols=28672, seed=2003) -> Int4Weight:
    """The 8192x28672 layer's distributions at a size the oracle checks in seconds."""
    return int4_weight(rows, cols, 128, seed)


def activation(rows, cols, seed, *, stress_frac=0.01, chunk=CHUNK_64K) -> Activation:
    """ReLU activations max(0, N(0,1) - 1.3) as fp16 bytes, plus stress chunks:
    stress_frac of the chunks become uniform random bytes, as many become all
    0xAB, and as many get one 0xAB run of U[1 KiB, 48 KiB] bytes at a seeded
    position (all chosen without replacement)."""
    rng = np.random.default_rng(seed)
    y = np.maximum(0.0, rng.standard_normal(rows * cols) - 1.3)
    data = y.astype(np.float16).view(np.uint8).copy()
    dst_off = uniform_chunks(data.size, chunk)
    n_chunks = dst_off.size - 1
    k = int(round(stress_frac * n_chunks))
    stress = {}
    if k > 0 and n_chunks >= 3 * k:
        sel = rng.choice(n_chunks, size=3 * k, replace=False)
        rnd, ab, runs = sel[:k], sel[k:2 * k], sel[2 * k:]
        for c in rnd:
            a, b = int(dst_off[c]), int(dst_off[c + 1])
            data[a:b] = rng.integers(0, 256, size=b - a, dtype=np.uint8)
        for c in ab:
            a, b = int(dst_off[c]), int(dst_off[c + 1])
            data[a:b] = 0xAB
        for c in runs:
            a, b = int(dst_off[c]), int(dst_off[c + 1])
            ln = min(b - a, int(rng.integers(KIB, 48 * KIB + 1)))
            st = a + int(rng.integers(0, b - a - ln + 1))
            data[st:st + ln] = 0xAB
        stress = {"random": sorted(map(int, rnd)), "all_ab": sorted(map(int, ab)),
                  "ab_run": sorted(map(int, runs))}
    return Activation((rows, cols), data, dst_off, stress, seed)


def relu_4096x14336() -> Activation:
    """ReLU activations decode-only: 4096x14336 fp16, 1792 chunks of 64 KiB,
    18 random-byte chunks, 18 all-0xAB chunks, 18 chunks with one 0xAB run."""
    return activation(4096, 14336, 1004)


# Llama-70B-shaped projections of one decoder layer: (name, rows, cols)
LLAMA70B_LAYER = (
    ("q", 8192, 8192),
    ("k", 8192, 1024),
    ("v", 8192, 1024),
    ("o", 8192, 8192),
    ("gate", 8192, 28672),
    ("up", 8192, 28672),
    ("down", 28672, 8192),
)
N_LAYERS_70B = 80


def llama70b_tensor(layer: int, t: int) -> Int4Weight:
    """One INT4 projection of the 80-layer stack, seeded by (1005, layer, t);
    distributions as the 8192x28672 layer's, chunk sizes drawn per chunk from 16/64/256 KiB."""
    name, r, c = LLAMA70B_LAYER[t]
    return int4_weight(r, c, 128, [1005, layer, t], chunking="mixed")


WORKLOADS = {"tiny_int4_1024": tiny_int4_1024, "int8_8192x8192": int8_8192x8192,
             "mlp_int4_8192x28672": mlp_int4_8192x28672, "relu_4096x14336": relu_4096x14336}
