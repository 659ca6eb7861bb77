#!/usr/bin/env python3
"""Benchmark: fused LZ4 + INT4 -> fp16 on one MI355X.

Workload: an INT4 MLP projection 8192 x 28672, group 128, zero points U{0..15},
codes rounded N(7.5, 3) clipped to 0..15, 20% all-zero groups, packed two per
byte (low nibble first) and LZ4-compressed in independent 64 KiB chunks by the
library's host packer, matches kept within the 4096-byte window the table
declares, with the table's sequence index (seeded synthetic data; it stands
in for real quantized weights).  A step is one lt_fused_lz4_int4 call over the whole layer: chunk
lookup, compressed-byte staging, LZ4 parse, literal/match copies, nibble
unpack, group-scale dequantization and the fp16 stores, with the compressed
table, scales and zero points already resident in HBM.

Metric: GB/s (1e9 B/s) of algorithmic bytes per step = compressed bytes read
+ fp16 bytes written (scales, zero points, the offset tables and the
sequence index are reported separately as metadata), and the fraction of
the 8.0 TB/s HBM peak.  Each step's time is the GPU time between HIP events
around the launch; a 1 GiB fill before each step (outside the events) clears
L2 and the last-level cache, so no step reads input a previous one left
cached (--no-evict times the steps back to back instead).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--extra]

Prints one JSON line.  --extra adds measurements of the raw (uncompressed)
INT4 path and of plain fill/copy ceilings under "extra".
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "fused_int4_8192x28672_hbm_traffic.md")


def source_hash() -> str:
    """Hash of the HIP sources, to tell whether stored counter data is stale."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "weight_dequantization_amd", "csrc")
    for fn in sorted(os.listdir(csrc)):
        if fn.endswith((".hip", ".hpp")):
            h.update(fn.encode())
            h.update(open(os.path.join(csrc, fn), "rb").read())
    return h.hexdigest()[:16]


def stored_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when the HIP sources changed since the counters were taken."""
    try:
        kv = dict(line.split(": ", 1) for line in open(PROFILE_TRAFFIC).read().splitlines()
                  if line.startswith(("source_hash: ", "traffic_bytes_per_launch: ")))
    except OSError:
        return None
    if kv.get("source_hash", "").strip() != source_hash():
        return None
    return int(kv["traffic_bytes_per_launch"])


def cpu_baseline(w, out_gpu, chunks: int, threads: int):
    """The CPU oracle (as it stands) on a bounded sample of the workload: the
    first `chunks` 64 KiB chunks of the same layer (all 1792 by default), compressed by the oracle's
    own compressor, decoded and dequantized with `threads` host threads.  The
    sample's outputs are also compared with the GPU's."""
    import oracle as O
    packed = O.pack_int4(w.codes)
    n = min(chunks, w.dst_off.size - 1)
    d_end = int(w.dst_off[n])
    dst_off = w.dst_off[:n + 1].copy()
    t = O.compress_table(packed[:d_end], dst_off, threads=threads)
    n_elem = 2 * d_end
    n_groups = -(-n_elem // w.group)
    scales, zp = w.scales[:n_groups], w.zp[:n_groups]
    out = np.zeros(n_elem, np.uint16)
    O.fused_int4_chunked(t, scales, zp, w.group, out, threads)        # warm caches
    times = []
    for _ in range(5):
        t0 = time.perf_counter()
        bad, _ = O.fused_int4_chunked(t, scales, zp, w.group, out, threads)
        times.append(time.perf_counter() - t0)
        assert bad == 0
    sec = sorted(times)[2]
    alg = t.comp_bytes + 2 * n_elem
    mismatches = int(np.count_nonzero(out != out_gpu[:n_elem]))
    return {
        "value": round(alg / sec / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": "first %d of %d chunks (%d elements, %.1f MB algorithmic), oracle-compressed, "
                  "median of 5 runs, %.2f s each" % (n, w.dst_off.size - 1, n_elem, alg / 1e6, sec),
        "gpu_mismatches_on_sample": mismatches,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--extra", action="store_true")
    ap.add_argument("--cpu-chunks", type=int, default=1792)
    ap.add_argument("--no-evict", action="store_true",
                    help="launch the timed steps back to back, without clearing the caches between them")
    ap.add_argument("--b2b", action="store_true",
                    help="also time the steps back to back with warm caches, for reference")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode "
              "(chunks shard across GPUs with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    import weight_dequantization_amd as lt

    dev = torch.device("cuda:0")
    w = synth.mlp_int4_8192x28672()
    packed = lt.pack_int4(w.codes)
    table = lt.ChunkTable.build(packed, w.dst_off, dev)
    scales = torch.from_numpy(w.scales.view(np.int16)).to(dev)
    zp = torch.from_numpy(w.zp).to(dev)
    n_elem = w.rows * w.cols
    out = torch.empty(n_elem, dtype=torch.float16, device=dev)
    status = torch.full((table.n_chunks,), -1, dtype=torch.int32, device=dev)
    shape = (w.rows, w.cols)
    alg_bytes = table.comp_bytes + 2 * n_elem
    # scales, zero points, the two offset tables and the sequence index
    meta_bytes = 2 * w.scales.size + w.zp.size + 16 * (table.n_chunks + 1) + \
        8 * (table.n_chunks + 1) + 4 * table.n_seq

    def step():
        lt.fused_lz4_int4(table, scales, zp, shape, w.group, out=out, status=status)

    scratch = None if args.no_evict else torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    for i in range(args.warmup):
        if scratch is not None:
            scratch.fill_(i & 255)
        step()
    torch.cuda.synchronize()
    lt.check_status(status)

    # Each timed step is bracketed by HIP events on the launch stream.  Before
    # each one (outside the events) a 1 GiB fill clears L2 and the 256 MB
    # last-level cache, so no step reads input the previous one left cached.
    stream = torch.cuda.current_stream()

    def timed_steps(evict):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i, (a, b) in enumerate(ev):
            if evict:
                scratch.fill_(i & 255)
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        lt.check_status(status)
        return [a.elapsed_time(b) for a, b in ev], wall

    kern_ms, wall = timed_steps(not args.no_evict)
    avg_kern_ms = float(np.mean(kern_ms))
    ms_per_step = avg_kern_ms if not args.no_evict else wall * 1e3 / args.steps
    value = alg_bytes / (ms_per_step / 1e3) / 1e9
    achieved = alg_bytes / (avg_kern_ms / 1e3) / 1e9
    b2b_ms = None
    if args.b2b and not args.no_evict:   # for reference: the same steps back to back, caches warm
        b2b, b2b_wall = timed_steps(False)
        b2b_ms = {"mean": round(float(np.mean(b2b)), 5), "wall_per_step": round(b2b_wall * 1e3 / args.steps, 5)}

    result = {
        "metric": "fused LZ4+INT4->fp16 GB/s (compressed in + fp16 out) and % of HBM peak, 1 GPU",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded; codes ~ rounded N(7.5,3) clipped 0..15, 20% zero groups)",
        "config": {
            "workload": "fused LZ4+INT4 -> fp16, 8192x28672 MLP projection, group 128, "
                        "asymmetric int8 zero points, 64 KiB LZ4 chunks (host packer, "
                        "declared match window 4096 B, sequence index)",
            "rows": w.rows, "cols": w.cols, "group": w.group, "chunks": table.n_chunks,
            "compressed_bytes": table.comp_bytes, "fp16_bytes": 2 * n_elem,
            "algorithmic_bytes": alg_bytes, "metadata_bytes": int(meta_bytes),
            "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": stored_traffic(),
            "kernel": "lt::chunk_kernel<3, 14>", "avg_launch_ms": round(avg_kern_ms, 5),
            "min_launch_ms": round(float(np.min(kern_ms)), 5),
            "bytes_per_launch": alg_bytes,
        },
        "step_ms": {"mean": round(avg_kern_ms, 5), "median": round(float(np.median(kern_ms)), 5),
                    "p10": round(float(np.percentile(kern_ms, 10)), 5),
                    "p90": round(float(np.percentile(kern_ms, 90)), 5),
                    "caches_cleared_before_each_step": not args.no_evict,
                    "back_to_back_no_clearing": b2b_ms},
    }

    if args.extra:
        result["extra"] = extra_measurements(torch, lt, w, packed, scales, zp, dev)

    if not args.no_cpu:
        out_host = out.view(torch.int16).cpu().numpy().view(np.uint16)
        threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
        threads = max(1, min(threads, 64))
        result["cpu_baseline"] = cpu_baseline(w, out_host, args.cpu_chunks, threads)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def extra_measurements(torch, lt, w, packed, scales, zp, dev, reps=20):
    """Raw INT4 dequant on the same layer, and plain fill / copy ceilings."""
    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps
    n_elem = w.rows * w.cols
    out = torch.empty(n_elem, dtype=torch.float16, device=dev)
    pk = torch.from_numpy(packed).to(dev)
    ms_raw = timed(lambda: lt.dequant_int4(pk, scales, zp, (w.rows, w.cols), w.group, out=out))
    raw_bytes = packed.size + 2 * n_elem
    lut = torch.randint(0, 1 << 15, (n_elem // w.group, 16), dtype=torch.int16, device=dev)
    ms_lut = timed(lambda: lt.dequant_int4_lut(pk, lut, (w.rows, w.cols), w.group, out=out))
    lut_bytes = packed.size + 2 * n_elem + lut.numel() * 2
    ms_fill = timed(lambda: out.fill_(1.0))
    src = torch.empty(2 * n_elem, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    ms_copy = timed(lambda: dst.copy_(src))
    return {
        "raw_int4_GBps": round(raw_bytes / ms_raw / 1e6, 1), "raw_int4_ms": round(ms_raw, 4),
        "codebook_int4_GBps": round(lut_bytes / ms_lut / 1e6, 1), "codebook_int4_ms": round(ms_lut, 4),
        "fill_fp16_GBps": round(2 * n_elem / ms_fill / 1e6, 1),
        "copy_GBps": round(2 * 2 * n_elem / ms_copy / 1e6, 1),
        "streamed_from_host": streamed_measurements(torch, lt, w, packed, scales, zp, dev, out),
        "verify_crc32": verify_measurement(torch, lt, w, packed, dev, timed),
        "activations_4096x14336": activation_measurements(torch, lt, dev, timed),
        "gemv": gemv_measurement(torch, lt, w, packed, scales, zp, dev, out, timed),
    }


def gemv_measurement(torch, lt, w, packed, scales, zp, dev, out, timed):
    """y = W x on the same layer: the fused decode-dequant-dot kernel (the
    fp16 matrix never written) against the fused kernel writing W followed
    by torch's fp16 matrix-vector product."""
    table = lt.ChunkTable.build(packed, w.dst_off, dev)
    x = torch.randn(w.cols, dtype=torch.float16, device=dev)
    y = torch.empty(w.rows, dtype=torch.float32, device=dev)
    ms_fused = timed(lambda: lt.fused_lz4_int4_gemv(table, scales, zp, (w.rows, w.cols), w.group, x, y=y))
    W = out.view(w.rows, w.cols)
    ms_two = timed(lambda: (lt.fused_lz4_int4(table, scales, zp, (w.rows, w.cols), w.group, out=out), torch.mv(W, x)))
    res = {"fused_ms": round(ms_fused, 4), "decode_then_mv_ms": round(ms_two, 4),
           "fused_compressed_GBps": round(table.comp_bytes / ms_fused / 1e6, 1)}
    # one layer of the 80-layer Llama-70B-shaped stack (7 projections, mixed
    # 16/64/256 KiB chunks), batch-1: the seven products back to back
    import synth
    layer = []
    for t in range(len(synth.LLAMA70B_LAYER)):
        wt = synth.llama70b_tensor(0, t)
        tb = lt.ChunkTable.build(lt.pack_int4(wt.codes), wt.dst_off, dev)
        layer.append((wt, tb, torch.from_numpy(wt.scales.view(np.int16)).to(dev), torch.from_numpy(wt.zp).to(dev),
                      torch.randn(wt.cols, dtype=torch.float16, device=dev),
                      torch.empty(wt.rows, dtype=torch.float32, device=dev)))

    def one(i, stream=None):
        wt, tb, sc, z, xv, yv = layer[i]
        lt.fused_lz4_int4_gemv(tb, sc, z, (wt.rows, wt.cols), wt.group, xv, y=yv, stream=stream)

    def run_layer():
        for i in range(len(layer)):
            one(i)
    ms_layer = timed(run_layer)
    # the order a layer allows: q, k, v together (one input), then o, then
    # gate and up together, then down; side streams at default priority
    side = [torch.cuda.Stream(device=dev) for _ in range(2)]
    main = torch.cuda.current_stream()

    def together(idx):
        for s_ in side:
            s_.wait_stream(main)
        one(idx[0])
        for s_, i in zip(side, idx[1:]):
            one(i, stream=s_)
        for s_ in side[:len(idx) - 1]:
            main.wait_stream(s_)

    def run_layer_streams():
        together([0, 1, 2])
        one(3)
        together([4, 5])
        one(6)
    ms_streams = timed(run_layer_streams)
    res["llama70b_layer_ms"] = round(ms_layer, 4)
    res["llama70b_layer_concurrent_ms"] = round(ms_streams, 4)
    res["llama70b_80_layers_ms"] = round(80 * min(ms_layer, ms_streams), 3)
    res["llama70b_layer_compressed_bytes"] = int(sum(tb.comp_bytes for _, tb, *_ in layer))
    return res


def activation_measurements(torch, lt, dev, timed):
    """The ReLU activation workload (4096x14336 fp16, about 90% zeros) two
    ways: zero-run coded (bitmap + values) and LZ4 chunks, decode-only; the
    coded size and GB/s of coded input + fp16 output."""
    import synth
    a = synth.relu_4096x14336()
    x = a.data.view(np.uint16)
    bitmap, val_off, vals = lt.encode_zero_runs(x)
    z = lt.ZeroRunTensor.from_host(bitmap, val_off, vals, x.size, dev)
    out = torch.empty(x.size, dtype=torch.float16, device=dev)
    zr_in = bitmap.nbytes + val_off.nbytes + vals.nbytes
    ms_zr = timed(lambda: lt.decode_zero_runs(z, out=out))
    assert torch.equal(out.view(torch.int16).cpu(), torch.from_numpy(x.view(np.int16)))
    table = lt.ChunkTable.build(a.data, a.dst_off, dev)
    ob = out.view(torch.uint8)
    ms_lz = timed(lambda: lt.decode_lz4(table, out=ob))
    return {
        "fp16_bytes": int(a.data.size),
        "zero_runs": {"coded_bytes": int(zr_in), "ms": round(ms_zr, 4),
                      "GBps": round((zr_in + a.data.size) / ms_zr / 1e6, 1)},
        "lz4_decode_only": {"coded_bytes": int(table.comp_bytes), "ms": round(ms_lz, 4),
                            "GBps": round((table.comp_bytes + a.data.size) / ms_lz / 1e6, 1)},
    }


def verify_measurement(torch, lt, w, packed, dev, timed):
    """lt_verify_chunks (CRC-32 of every chunk's compressed bytes against the
    stored values) on the same table, as GB/s of compressed bytes."""
    comp, comp_off = lt.compress_chunks(packed, w.dst_off, max_dist=lt.PACK_WINDOW)
    table = lt.ChunkTable.from_host(comp, comp_off, w.dst_off, dev)
    expect = torch.from_numpy(lt.checksum_chunks(comp, comp_off).view(np.int32)).to(dev)
    got = torch.empty(table.n_chunks, dtype=torch.int32, device=dev)
    status = torch.empty(table.n_chunks, dtype=torch.int32, device=dev)
    ms = timed(lambda: lt.verify_chunks(table, expect, got, status))
    lt.check_status(status)
    return {"ms": round(ms, 4), "compressed_GBps": round(table.comp_bytes / ms / 1e6, 1)}


def streamed_measurements(torch, lt, w, packed, scales, zp, dev, out, reps=10, per_half=512):
    """The same layer with its chunk table in pinned host memory: the
    streamed entry point (copies of one batch overlapped with the decode of
    the one before) against copying the whole table first and then decoding,
    and the plain host-to-device copy of the compressed bytes alone.  Host
    wall clock around each call, synchronized on both sides, so every rate
    here includes PCIe."""
    import time as _t
    n_elem = w.rows * w.cols
    ht = lt.ChunkTable.build(packed, w.dst_off, "cpu", pin=True)
    staging = torch.empty(ht.staging_bytes(per_half), dtype=torch.uint8, device=dev)
    status = torch.full((ht.n_chunks,), -1, dtype=torch.int32, device=dev)
    dt = lt.ChunkTable(torch.empty_like(ht.comp, device=dev), torch.empty_like(ht.comp_off, device=dev),
                       torch.empty_like(ht.dst_off, device=dev), ht.n_chunks, ht.max_chunk_bytes,
                       ht.total_bytes, ht.comp_bytes, ht.max_dist,
                       torch.empty_like(ht.seq_off, device=dev), torch.empty_like(ht.seq_pos, device=dev),
                       ht.n_seq)
    shape = (w.rows, w.cols)

    def streamed():
        lt.stream_fused_lz4_int4(ht, scales, zp, shape, w.group, out=out, status=status, staging=staging)

    def sequential():
        for d, h in ((dt.comp, ht.comp), (dt.comp_off, ht.comp_off), (dt.dst_off, ht.dst_off),
                     (dt.seq_off, ht.seq_off), (dt.seq_pos, ht.seq_pos)):
            d.copy_(h, non_blocking=True)
        lt.fused_lz4_int4(dt, scales, zp, shape, w.group, out=out, status=status)

    def copy_only():
        dt.comp.copy_(ht.comp, non_blocking=True)

    def wall(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            t0 = _t.perf_counter()
            fn()
            torch.cuda.synchronize()
            ts.append((_t.perf_counter() - t0) * 1e3)
        return float(np.median(ts))

    ms_stream = wall(streamed)
    lt.check_status(status)
    ms_seq = wall(sequential)
    lt.check_status(status)
    ms_copy = wall(copy_only)
    inb = ht.comp_bytes + 2 * n_elem
    return {
        "chunks_per_half": per_half, "staging_bytes": staging.numel(),
        "streamed_ms": round(ms_stream, 4), "copy_then_decode_ms": round(ms_seq, 4),
        "h2d_copy_of_compressed_bytes_ms": round(ms_copy, 4),
        "h2d_GBps": round(ht.comp_bytes / ms_copy / 1e6, 2),
        "streamed_pcie_inclusive_GBps": round(inb / ms_stream / 1e6, 2),
    }


if __name__ == "__main__":
    main()
