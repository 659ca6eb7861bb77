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

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3|2|5] [--no-cpu] [--extra]

Prints one JSON line and exits non-zero when any GPU output checked in the
run differs from the oracle's or between routes.  The line also times the
same layer as plain LZ4 ("plain_lz4": the packer's blocks without the
sequence index, and greedy-parse blocks with a 64 KiB window), reports the
device footprint with the index counted in, and times the CPU oracle on the
table the GPU decodes at all host cores and at one thread.  --extra adds
the raw (uncompressed) INT4 path, plain fill/copy ceilings and the other
entry points under "extra".  --config 2 measures the 8192x8192 INT8 matrix
(fused and two-pass); --config 5 the 80-layer Llama-70B-shaped stack.
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


def _threads_all() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return max(1, min(n, 64))


def cpu_baseline(run, alg_bytes, out_gpu, n_elem, sample, runs_one=3, runs_all=5):
    """The CPU oracle (as it stands) on the same table the GPU decodes:
    `run(threads)` decodes and dequantizes it into a host buffer and returns
    (buffer, bad chunks).  Timed at all host cores (the reported value) and
    at one thread; the outputs are compared with the GPU's, element by
    element."""
    threads = _threads_all()

    def timed(th, runs):
        out, bad = run(th)                       # warm caches
        ts = []
        for _ in range(runs):
            t0 = time.perf_counter()
            out, bad = run(th)
            ts.append(time.perf_counter() - t0)
            assert bad == 0
        return out, float(np.median(ts))

    out, sec = timed(threads, runs_all)
    mismatches = int(np.count_nonzero(out[:n_elem] != out_gpu[:n_elem]))
    _, sec1 = timed(1, runs_one)
    return {
        "value": round(alg_bytes / sec / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": "%s; median of %d runs, %.3f s each" % (sample, runs_all, sec),
        "one_thread": {"value": round(alg_bytes / sec1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                       "sample": "the same, median of %d runs, %.2f s each" % (runs_one, sec1)},
        "gpu_mismatches_on_sample": mismatches,
    }


def timed_launches(torch, fn, steps, scratch, stream):
    """Kernel time of `steps` calls of fn, each bracketed by HIP events on
    `stream`; with `scratch`, a fill of it before each call (outside the
    events) clears the caches.  Returns (per-call ms, wall seconds)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, (a, b) in enumerate(ev):
        if scratch is not None:
            scratch.fill_(i & 255)
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [a.elapsed_time(b) for a, b in ev], wall


def footprint(comp_bytes, n_chunks, n_seq, meta_bytes, n_elem, packed_bytes):
    """The compressed tensor's size in device memory, with the sequence
    index and the offset tables counted in, against fp16 and packed INT4."""
    index = 8 * (n_chunks + 1) + 4 * n_seq if n_seq else 0
    offsets = 16 * (n_chunks + 1)
    total = comp_bytes + index + offsets + meta_bytes
    return {"compressed_bytes": comp_bytes, "sequence_index_bytes": index, "offset_table_bytes": offsets,
            "scale_zero_point_bytes": meta_bytes, "total_bytes": total,
            "fp16_over_total": round(2 * n_elem / total, 4),
            "packed_over_total": round((packed_bytes + meta_bytes) / total, 4)}


def plain_lz4_forms(torch, lt, packed, comp, comp_off, w, scales, zp, dev, out_ref, scratch, stream, steps):
    """The same layer as plain LZ4, without the sequence index: (i) the
    packer's blocks (4096-byte window) and (ii) the greedy parse's blocks
    (4-byte matches, 64 KiB window), the blocks a general-purpose LZ4
    compressor writes; (iii) the greedy blocks with the index added at load.
    Each is timed like the headline and its output compared bit for bit
    with the headline's."""
    n_elem = w.rows * w.cols
    gcomp, gcomp_off = lt.compress_chunks(packed, w.dst_off, greedy=True)
    forms = (
        ("packer_blocks_no_index", lambda: lt.ChunkTable.from_host(comp, comp_off, w.dst_off, dev, lt.PACK_WINDOW)),
        ("greedy_64k_window_no_index", lambda: lt.ChunkTable.from_host(gcomp, gcomp_off, w.dst_off, dev, 0)),
        ("greedy_64k_window_indexed", lambda: lt.ChunkTable.from_host(gcomp, gcomp_off, w.dst_off, dev, 0, index=True,
                                                                      order=True)),
    )
    n_seq = {False: int(lt.index_chunks(comp, comp_off)[1].size),
             True: int(lt.index_chunks(gcomp, gcomp_off)[1].size)}
    out = torch.empty_like(out_ref)
    res, bad_total = {}, 0
    for name, make in forms:
        tb = make()
        status = torch.full((tb.n_chunks,), -1, dtype=torch.int32, device=dev)

        def fn():
            lt.fused_lz4_int4(tb, scales, zp, (w.rows, w.cols), w.group, out=out, status=status)
        out.fill_(0)
        fn()
        torch.cuda.synchronize()
        lt.check_status(status)
        bad = int((out.view(torch.int16) != out_ref.view(torch.int16)).sum().item())
        bad_total += bad
        ms, _ = timed_launches(torch, fn, steps, scratch, stream)
        lt.check_status(status)
        alg = tb.comp_bytes + 2 * n_elem
        kern = float(np.mean(ms))
        res[name] = {"compressed_bytes": tb.comp_bytes, "sequences": n_seq["greedy" in name],
                     "kernel_ms": round(kern, 5), "GBps": round(alg / kern / 1e6, 2),
                     "frac": round(alg / kern / 1e6 / HBM_PEAK_GBS, 4), "mismatches_vs_headline": bad}
        del tb
    return res, bad_total


def checked_form(torch, lt, comp, comp_off, w, scales, zp, dev, out_ref, scratch, stream, steps):
    """The headline table with each chunk's XXH3-64 stored: every launch
    hashes the compressed bytes as the decoder stages them and checks them
    (no second pass over HBM).  Timed like the headline; the output is
    compared bit for bit with the headline's and every status must be OK."""
    n_elem = w.rows * w.cols
    tb = lt.ChunkTable.from_host(comp, comp_off, w.dst_off, dev, lt.PACK_WINDOW, index=True, checksum=True)
    status = torch.full((tb.n_chunks,), -1, dtype=torch.int32, device=dev)
    out = torch.empty_like(out_ref)

    def fn():
        lt.fused_lz4_int4(tb, scales, zp, (w.rows, w.cols), w.group, out=out, status=status)
    fn()
    torch.cuda.synchronize()
    lt.check_status(status)
    bad = int((out.view(torch.int16) != out_ref.view(torch.int16)).sum().item())
    ms, _ = timed_launches(torch, fn, steps, scratch, stream)
    lt.check_status(status)
    alg = tb.comp_bytes + 2 * n_elem
    kern = float(np.mean(ms))
    return {"kernel_ms": round(kern, 5), "GBps": round(alg / kern / 1e6, 2),
            "frac": round(alg / kern / 1e6 / HBM_PEAK_GBS, 4), "checksum_bytes": 8 * tb.n_chunks,
            "mismatches_vs_headline": bad}, bad


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3, choices=(2, 3, 5),
                    help="3: the 8192x28672 INT4 layer (default); 2: the 8192x8192 INT8 matrix; "
                         "5: the 80-layer Llama-70B-shaped INT4 stack")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--extra", action="store_true")
    ap.add_argument("--no-evict", action="store_true",
                    help="launch the timed steps back to back, without clearing the caches between them")
    ap.add_argument("--b2b", action="store_true",
                    help="also time the steps back to back with warm caches, for reference")
    ap.add_argument("--no-plain", action="store_true",
                    help="skip the plain-LZ4 forms of the layer (profiling runs time the headline launch alone)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="end with one device-to-device copy of the fp16 output's size, which calibrates "
                         "rocprofv3's byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode "
              "(chunks shard across GPUs with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)
    if args.config == 2:
        sys.exit(bench_int8(args))
    if args.config == 5:
        sys.exit(bench_stack(args))
    sys.exit(bench_int4_layer(args))


def bench_int4_layer(args) -> int:
    import torch

    import synth
    import weight_dequantization_amd as lt

    dev = torch.device("cuda:0")
    w = synth.mlp_int4_8192x28672()
    packed = lt.pack_int4(w.codes)
    comp, comp_off = lt.compress_chunks(packed, w.dst_off, max_dist=lt.PACK_WINDOW)
    table = lt.ChunkTable.from_host(comp, comp_off, w.dst_off, dev, lt.PACK_WINDOW, index=True)
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
    kern_ms, wall = timed_launches(torch, step, args.steps, scratch, stream)
    lt.check_status(status)
    avg_kern_ms = float(np.mean(kern_ms))
    ms_per_step = avg_kern_ms if not args.no_evict else wall * 1e3 / args.steps
    value = alg_bytes / (ms_per_step / 1e3) / 1e9
    achieved = alg_bytes / (avg_kern_ms / 1e3) / 1e9
    b2b_ms = None
    if args.b2b and not args.no_evict:   # for reference: the same steps back to back, caches warm
        b2b, b2b_wall = timed_launches(torch, step, args.steps, None, stream)
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
            "footprint": footprint(table.comp_bytes, table.n_chunks, table.n_seq,
                                   2 * w.scales.size + w.zp.size, n_elem, packed.size),
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": stored_traffic(),
            "kernel": "lt::chunk_kernel<3, 14, false, false>", "avg_launch_ms": round(avg_kern_ms, 5),
            "min_launch_ms": round(float(np.min(kern_ms)), 5),
            "bytes_per_launch": alg_bytes,
        },
        "step_ms": {"mean": round(avg_kern_ms, 5), "median": round(float(np.median(kern_ms)), 5),
                    "p10": round(float(np.percentile(kern_ms, 10)), 5),
                    "p90": round(float(np.percentile(kern_ms, 90)), 5),
                    "caches_cleared_before_each_step": not args.no_evict,
                    "back_to_back_no_clearing": b2b_ms},
    }
    bad_plain = 0
    if not args.no_plain:
        plain, bad_plain = plain_lz4_forms(torch, lt, packed, comp, comp_off, w, scales, zp, dev, out, scratch,
                                           stream, max(5, args.steps // 5))
        result["plain_lz4"] = plain
        checked, bad_checked = checked_form(torch, lt, comp, comp_off, w, scales, zp, dev, out, scratch, stream,
                                            max(10, args.steps // 2))
        result["checksum_in_decode"] = checked
        bad_plain += bad_checked
    if args.calib_copy:
        src = torch.empty(2 * n_elem, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        result["calibration_copy_bytes"] = 2 * n_elem

    if args.extra:
        result["extra"] = extra_measurements(torch, lt, w, packed, scales, zp, dev)

    bad_cpu = 0
    if not args.no_cpu:
        import oracle as O
        out_host = out.view(torch.int16).cpu().numpy().view(np.uint16)
        t = O.Table(comp, comp_off, w.dst_off)
        host = np.zeros(n_elem, np.uint16)

        def run(th):
            bad, _ = O.fused_int4_chunked(t, w.scales, w.zp, w.group, host, th)
            return host, bad
        result["cpu_baseline"] = cpu_baseline(
            run, alg_bytes, out_host, n_elem,
            "the whole layer: all %d chunks of the table the GPU decodes (%d elements, %.1f MB algorithmic)"
            % (table.n_chunks, n_elem, alg_bytes / 1e6))
        bad_cpu = result["cpu_baseline"]["gpu_mismatches_on_sample"]
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    if bad_cpu or bad_plain:
        print("GPU output differs: %d elements from the oracle, %d across the plain-LZ4 forms"
              % (bad_cpu, bad_plain), file=sys.stderr)
        return 1
    return 0


def bench_int8(args) -> int:
    """The 8192x8192 INT8 matrix (per-row scales, half the rows zero), 64 KiB
    chunks in the default table form: the fused kernel against the two-pass
    route (decode to INT8 bytes, then dequantize)."""
    import torch

    import synth
    import weight_dequantization_amd as lt

    dev = torch.device("cuda:0")
    w = synth.int8_8192x8192()
    qb = w.q.view(np.uint8)
    comp, comp_off = lt.compress_chunks(qb, w.dst_off, max_dist=lt.PACK_WINDOW)
    table = lt.ChunkTable.from_host(comp, comp_off, w.dst_off, dev, lt.PACK_WINDOW, index=True)
    scales = torch.from_numpy(w.scales.view(np.int16)).to(dev)
    n_elem = w.rows * w.cols
    shape = (w.rows, w.cols)
    out = torch.empty(n_elem, dtype=torch.float16, device=dev)
    out2 = torch.empty_like(out)
    qbuf = torch.empty(n_elem, dtype=torch.uint8, device=dev)
    status = torch.full((table.n_chunks,), -1, dtype=torch.int32, device=dev)
    status2 = torch.full_like(status, -1)
    alg = table.comp_bytes + 2 * n_elem

    def fused():
        lt.fused_lz4_int8(table, scales, None, shape, w.group, out=out, status=status)

    def decode():
        lt.decode_lz4(table, out=qbuf, status=status2)

    def dequant():
        lt.dequant_int8(qbuf.view(torch.int8), scales, None, shape, w.group, out=out2)

    scratch = None if args.no_evict else torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        fused(); decode(); dequant()
    torch.cuda.synchronize()
    lt.check_status(status)
    lt.check_status(status2)
    bad_two = int((out.view(torch.int16) != out2.view(torch.int16)).sum().item())
    ms_f, _ = timed_launches(torch, fused, args.steps, scratch, stream)
    ms_d, _ = timed_launches(torch, decode, args.steps, scratch, stream)
    ms_q, _ = timed_launches(torch, dequant, args.steps, scratch, stream)
    lt.check_status(status)
    kf, kd, kq = float(np.mean(ms_f)), float(np.mean(ms_d)), float(np.mean(ms_q))
    value = alg / kf / 1e6
    result = {
        "metric": "fused LZ4+INT8->fp16 GB/s (compressed in + fp16 out) and % of HBM peak, 1 GPU",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(kf, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded; q = clip(rint(N(0,1)*32), +-127), 4096 of 8192 rows zero, "
                "per-row fp16 scales U(1e-3, 1e-2))",
        "config": {"workload": "fused LZ4+INT8 -> fp16, 8192x8192, per-row scales, no zero point, 64 KiB LZ4 "
                               "chunks (host packer, declared match window 4096 B, sequence index)",
                   "chunks": table.n_chunks, "compressed_bytes": table.comp_bytes, "fp16_bytes": 2 * n_elem,
                   "algorithmic_bytes": alg,
                   "footprint": footprint(table.comp_bytes, table.n_chunks, table.n_seq, 2 * w.scales.size,
                                          n_elem, n_elem)},
        "roofline": {"bound": "hbm", "achieved": round(value, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "lt::chunk_kernel<2, 14, false, false>", "avg_launch_ms": round(kf, 5), "bytes_per_launch": alg},
        "two_pass": {"decode_ms": round(kd, 5), "dequant_ms": round(kq, 5), "total_ms": round(kd + kq, 5),
                     "GBps": round(alg / (kd + kq) / 1e6, 2), "fused_speedup": round((kd + kq) / kf, 3),
                     "mismatches_vs_fused": bad_two},
        "step_ms": {"caches_cleared_before_each_step": not args.no_evict},
    }
    bad_cpu = 0
    if not args.no_cpu:
        import oracle as O
        t = O.Table(comp, comp_off, w.dst_off)
        out_host = out.view(torch.int16).cpu().numpy().view(np.uint16)

        def run(th):
            o, st = O.fused_int8(t, w.scales, None, w.group, n_elem, th)
            return o, int(np.count_nonzero(st))
        result["cpu_baseline"] = cpu_baseline(
            run, alg, out_host, n_elem, "the whole matrix: all %d chunks of the table the GPU decodes"
            % table.n_chunks)
        bad_cpu = result["cpu_baseline"]["gpu_mismatches_on_sample"]
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    if bad_cpu or bad_two:
        print("GPU output differs: %d elements from the oracle, %d between the routes" % (bad_cpu, bad_two),
              file=sys.stderr)
        return 1
    return 0


def bench_stack(args) -> int:
    """The 80-layer Llama-70B-shaped INT4 stack (q, k, v, o, gate, up, down
    per layer; group 128; 16/64/256 KiB chunks drawn per chunk), resident on
    the device in the default table form and expanded layer by layer.  The
    headline decodes each layer with one lt_fused_lz4_int4 launch over a
    table of its seven projections end to end (ChunkTable.build_concat: the
    same compressed chunks, one launch order over the layer) into one fp16
    buffer; beside it, one launch per tensor into seven reused buffers, 560
    per pass.  Two distinct layers are generated (the seeds of layers 0 and
    79) and copied on the device into 80 separate allocations (even layers
    from layer 0, odd from layer 79); 80 layers of host generation would
    take far longer than a benchmark may run.  Each layer's launches are
    bracketed by HIP events; the per-tensor launches are timed one after
    another on one stream, and spread over four streams (the projections are
    independent).  No cache clearing is needed, as each layer reads and
    writes about 2 GB."""
    import torch

    import synth
    import weight_dequantization_amd as lt

    dev = torch.device("cuda:0")
    names = [n for n, _, _ in synth.LLAMA70B_LAYER]
    base, host, cat_base = {}, {}, {}
    for src in (0, 79):
        packs, dsts, scs, zps = [], [], [], []
        for t in range(len(names)):
            w = synth.llama70b_tensor(src, t)
            packed = lt.pack_int4(w.codes)
            comp, comp_off = lt.compress_chunks(packed, w.dst_off, max_dist=lt.PACK_WINDOW)
            tb = lt.ChunkTable.from_host(comp, comp_off, w.dst_off, dev, lt.PACK_WINDOW, index=True, order=True)
            base[(src, t)] = (tb, torch.from_numpy(w.scales.view(np.int16)).to(dev), torch.from_numpy(w.zp).to(dev))
            if src == 0 and t == 6:
                host["down"] = (w, comp, comp_off)
            packs.append(packed)
            dsts.append(w.dst_off)
            scs.append(w.scales)
            zps.append(w.zp)
            print("stack: layer %d %s packed and resident" % (src, names[t]), file=sys.stderr, flush=True)
        # the same layer as one table over its seven projections, end to end
        ct, _ = lt.ChunkTable.build_concat(packs, dsts, dev)
        cat_base[src] = (ct, torch.from_numpy(np.concatenate(scs).view(np.int16)).to(dev),
                         torch.from_numpy(np.concatenate(zps)).to(dev))
        del packs
        print("stack: layer %d as one table resident" % src, file=sys.stderr, flush=True)
    def clone(tb):
        return lt.ChunkTable(tb.comp.clone(), tb.comp_off.clone(), tb.dst_off.clone(), tb.n_chunks,
                             tb.max_chunk_bytes, tb.total_bytes, tb.comp_bytes, tb.max_dist,
                             tb.seq_off.clone(), tb.seq_pos.clone(), tb.n_seq, order=tb.order.clone())

    layers, cat_layers = [], []
    for layer in range(synth.N_LAYERS_70B):
        src = 0 if layer % 2 == 0 else 79
        tensors = []
        for t in range(len(names)):
            tb, sc, zp = base[(src, t)]
            tensors.append((clone(tb), sc.clone(), zp.clone()))
        layers.append(tensors)
        ct, sc, zp = cat_base[src]
        cat_layers.append((clone(ct), sc.clone(), zp.clone()))
    shapes = [(r, c) for _, r, c in synth.LLAMA70B_LAYER]
    outs = [torch.empty(r * c, dtype=torch.float16, device=dev) for r, c in shapes]
    nmax = max(tb.n_chunks for L in layers for tb, _, _ in L)
    statuses = [torch.full((nmax,), -1, dtype=torch.int32, device=dev) for _ in shapes]
    n_elem_layer = sum(r * c for r, c in shapes)
    out_cat = torch.empty(n_elem_layer, dtype=torch.float16, device=dev)
    st_cat = torch.full((max(ct.n_chunks for ct, _, _ in cat_layers),), -1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    side = [torch.cuda.Stream(device=dev) for _ in range(3)]   # default priority

    def run_layer(L):
        for t, (tb, sc, zp) in enumerate(L):
            lt.fused_lz4_int4(tb, sc, zp, shapes[t], 128, out=outs[t], status=statuses[t])

    def run_layer_concurrent(L):
        # the seven projections are independent: spread over four streams,
        # so a small launch (k, v) does not leave the GPU idle behind it
        for s_ in side:
            s_.wait_stream(stream)
        for t, (tb, sc, zp) in enumerate(L):
            lt.fused_lz4_int4(tb, sc, zp, shapes[t], 128, out=outs[t], status=statuses[t],
                              stream=None if t % 4 == 0 else side[t % 4 - 1])
        for s_ in side:
            stream.wait_stream(s_)

    def run_layer_table(C):
        # the whole layer from one table: one launch, the seven projections
        # back to back in out_cat
        ct, sc, zp = C
        lt.fused_lz4_int4(ct, sc, zp, (1, n_elem_layer), 128, out=out_cat, status=st_cat)

    def check():
        for t, (tb, _, _) in enumerate(layers[-1]):
            lt.check_status(statuses[t][:tb.n_chunks])
        lt.check_status(st_cat[:cat_layers[-1][0].n_chunks])

    print("stack: 80 layers resident, warming up", file=sys.stderr, flush=True)
    for _ in range(max(1, args.warmup)):
        for L in layers:
            run_layer(L)
        for C in cat_layers:
            run_layer_table(C)
    torch.cuda.synchronize()
    check()
    passes = max(1, min(args.steps, 5))
    layer_comp = [sum(tb.comp_bytes for tb, _, _ in L) for L in layers]
    alg_layer = np.array([cb + 2 * n_elem_layer for cb in layer_comp], np.float64)

    def time_form(run, items=None):
        items = layers if items is None else items
        for L in items[:2]:
            run(L)
        ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in items]
              for _ in range(passes)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for p in range(passes):
            for L, (a, b) in zip(items, ev[p]):
                a.record(stream)
                run(L)
                b.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        check()
        per_layer = np.array([[a.elapsed_time(b) for a, b in row] for row in ev])
        gbps = alg_layer[None, :] / per_layer / 1e6
        ms_pass = float(per_layer.sum(axis=1).mean())
        return ms_pass, {"ms_per_pass": round(ms_pass, 4), "layer_ms_mean": round(float(per_layer.mean()), 5),
                         "layer_ms_min": round(float(per_layer.min()), 5),
                         "layer_ms_max": round(float(per_layer.max()), 5),
                         "layer_GBps_mean": round(float(gbps.mean()), 2),
                         "layer_frac_mean": round(float(gbps.mean()) / HBM_PEAK_GBS, 4),
                         "wall_ms_per_pass": round(wall * 1e3 / passes, 3)}

    ms_seq, seq = time_form(run_layer)
    ms_conc, conc = time_form(run_layer_concurrent)
    ms_one, one = time_form(run_layer_table, cat_layers)
    # the one-table form decodes the same compressed chunks (laid end to end)
    assert sum(ct.comp_bytes for ct, _, _ in cat_layers) == sum(layer_comp)
    torch.cuda.synchronize()
    bad_forms = 0
    for t, o in enumerate(outs):   # the last layer, both forms: the same fp16 bytes
        e0 = sum(r * c for r, c in shapes[:t])
        bad_forms += int((out_cat[e0:e0 + o.numel()].view(torch.int16) != o.view(torch.int16)).sum().item())
    alg_pass = float(alg_layer.sum())
    value = alg_pass / ms_one / 1e6
    result = {
        "metric": "fused LZ4+INT4->fp16 GB/s over the 80-layer stack (compressed in + fp16 out), 1 GPU",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": passes, "warmup": max(1, args.warmup),
        "ms_per_step": round(ms_one, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic (seeded; two generated layers copied to 80 device allocations)",
        "config": {"workload": "80 Llama-70B-shaped INT4 layers (q, k, v, o 8192x8192 / 8192x1024; gate, up, "
                               "down 8192x28672), group 128, 16/64/256 KiB LZ4 chunks (host packer, declared "
                               "window 4096 B, sequence index, largest chunks launched first); a step is one "
                               "pass over the 80 layers, each layer decoded by one fused launch over a table of "
                               "its seven projections end to end (80 launches per pass)",
                   "compressed_bytes_resident": int(sum(layer_comp)), "fp16_bytes_per_layer": 2 * n_elem_layer},
        "roofline": {"bound": "hbm", "achieved": round(value, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "lt::chunk_kernel<3, 14, false, false>",
                     "avg_launch_ms": one["layer_ms_mean"], "bytes_per_launch": int(alg_layer.mean())},
        "layer_one_table": one,
        "layer_concurrent": conc,
        "layer_sequential": seq,
        "mismatches_between_forms": bad_forms,
    }
    bad_cpu = 0
    if not args.no_cpu:
        import oracle as O
        w, comp, comp_off = host["down"]
        tb, sc, zp = base[(0, 6)]
        st = torch.full((tb.n_chunks,), -1, dtype=torch.int32, device=dev)
        o = lt.fused_lz4_int4(tb, sc, zp, (w.rows, w.cols), 128, status=st)
        torch.cuda.synchronize()
        lt.check_status(st)
        out_host = o.view(torch.int16).cpu().numpy().view(np.uint16).ravel()
        n_elem = w.rows * w.cols
        t = O.Table(comp, comp_off, w.dst_off)
        buf = np.zeros(n_elem, np.uint16)

        def run(th):
            bad, _ = O.fused_int4_chunked(t, w.scales, w.zp, w.group, buf, th)
            return buf, bad
        result["cpu_baseline"] = cpu_baseline(
            run, int(comp_off[-1]) + 2 * n_elem, out_host, n_elem,
            "layer 0's down projection (8192x28672, %d chunks of 16/64/256 KiB), the table the GPU decodes"
            % (comp_off.size - 1), runs_one=1, runs_all=3)
        bad_cpu = result["cpu_baseline"]["gpu_mismatches_on_sample"]
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    if bad_cpu or bad_forms:
        print("GPU output differs: %d elements from the oracle, %d between the layer forms" % (bad_cpu, bad_forms),
              file=sys.stderr)
        return 1
    return 0


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
        "streamed_from_file": file_measurements(torch, lt, w, packed, scales, zp, dev, out),
        "verify_xxh3": verify_measurement(torch, lt, w, packed, dev, timed),
        "activations_4096x14336": activation_measurements(torch, lt, dev, timed),
        "gemv": gemv_measurement(torch, lt, w, packed, scales, zp, dev, out, timed),
        "gemm": gemm_measurement(torch, lt, w, packed, scales, zp, dev, out, timed),
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


def gemm_measurement(torch, lt, w, packed, scales, zp, dev, out, timed):
    """Y = X W^T on the same layer for batches of 16 and 32: the decode fused
    with the product on the matrix cores (W's codes in the GEMM tile layout,
    2048 chunks of 56 tiles; W never written) against lt_fused_lz4_int4
    writing W (the headline table) followed by torch.mm, and torch.mm alone
    on the resident fp16 W.  Back to back, without cache clearing."""
    rows, cols = w.rows, w.cols
    gt = lt.ChunkTable.build(lt.pack_int4_tiles(w.codes.reshape(rows, cols), rows, cols),
                             lt.gemm_chunks(rows, cols), dev)
    rt = lt.ChunkTable.build(packed, w.dst_off, dev)
    W = out.view(rows, cols)
    res = {"chunks": gt.n_chunks, "compressed_bytes": gt.comp_bytes}
    for batch in (16, 32):
        x = torch.randn(batch, cols, dtype=torch.float16, device=dev)
        xt = x.t().contiguous()
        y = torch.empty(batch, rows, dtype=torch.float32, device=dev)
        ws = torch.empty(lt.gemm_workspace_bytes(gt.n_chunks, batch) // 4, dtype=torch.float32, device=dev)
        ms_f = timed(lambda: lt.fused_lz4_int4_gemm(gt, scales, zp, (rows, cols), w.group, x, y=y, workspace=ws))
        ms_2 = timed(lambda: (lt.fused_lz4_int4(rt, scales, zp, (rows, cols), w.group, out=out), torch.mm(W, xt)))
        ms_mm = timed(lambda: torch.mm(W, xt))
        y2 = torch.mm(W.float(), xt.float()).t()
        rel = float((y - y2).abs().max() / y2.abs().max())
        res["batch%d" % batch] = {"fused_ms": round(ms_f, 4), "decode_then_mm_ms": round(ms_2, 4),
                                  "mm_alone_ms": round(ms_mm, 4), "speedup": round(ms_2 / ms_f, 3),
                                  "max_rel_diff_vs_fp32_mm": rel}
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
    idx_bytes = 8 * (table.n_chunks + 1) + 4 * table.n_seq
    return {
        "fp16_bytes": int(a.data.size),
        "zero_runs": {"coded_bytes": int(zr_in), "ms": round(ms_zr, 4),
                      "GBps": round((zr_in + a.data.size) / ms_zr / 1e6, 1)},
        "lz4_decode_only": {"coded_bytes": int(table.comp_bytes), "ms": round(ms_lz, 4),
                            "GBps": round((table.comp_bytes + a.data.size) / ms_lz / 1e6, 1),
                            # the sequence index and offsets the decoder reads, counted in
                            "sequence_index_bytes": idx_bytes,
                            "fp16_over_footprint": round(a.data.size / (table.comp_bytes + idx_bytes +
                                                                        16 * (table.n_chunks + 1)), 3)},
    }


def verify_measurement(torch, lt, w, packed, dev, timed):
    """lt_verify_chunks (XXH3-64 of every chunk's compressed bytes against the
    stored values, without decoding) on the same table, as GB/s of
    compressed bytes."""
    comp, comp_off = lt.compress_chunks(packed, w.dst_off, max_dist=lt.PACK_WINDOW)
    table = lt.ChunkTable.from_host(comp, comp_off, w.dst_off, dev)
    expect = torch.from_numpy(lt.checksum_chunks(comp, comp_off).view(np.int64)).to(dev)
    got = torch.empty(table.n_chunks, dtype=torch.int64, device=dev)
    status = torch.empty(table.n_chunks, dtype=torch.int32, device=dev)
    ms = timed(lambda: lt.verify_chunks(table, expect, got, status))
    lt.check_status(status)
    return {"ms": round(ms, 4), "compressed_GBps": round(table.comp_bytes / ms / 1e6, 1)}


def file_measurements(torch, lt, w, packed, scales, zp, dev, out, reps=5):
    """The layer's compressed bytes in a file (just written, so in the
    host's page cache): read, copy and decode one after another (the whole
    table as one batch) against the three stages overlapped (batches of
    64 to 512 chunks), both through the file-streaming entry point with the
    same reader (8 threads, and 1 for reference).  Host wall clock,
    synchronized on both sides: every figure includes the reads and PCIe."""
    import tempfile
    import time as _t
    comp, comp_off = lt.compress_chunks(packed, w.dst_off, max_dist=lt.PACK_WINDOW)
    ht = lt.ChunkTable.from_host(comp, comp_off, w.dst_off, "cpu", lt.PACK_WINDOW, index=True, pin=True)
    fd, path = tempfile.mkstemp(suffix=".ltcomp")
    with os.fdopen(fd, "wb") as f:
        f.write(comp.tobytes())
    status = torch.full((ht.n_chunks,), -1, dtype=torch.int32, device=dev)
    shape = (w.rows, w.cols)

    def run(per_half, threads):
        pinned = torch.empty(ht.pinned_bytes(per_half), dtype=torch.uint8, pin_memory=True)
        staging = torch.empty(ht.staging_bytes(per_half), dtype=torch.uint8, device=dev)

        def go():
            lt.stream_file_fused_lz4_int4(path, 0, ht, scales, zp, shape, w.group, out=out, status=status,
                                          pinned=pinned, staging=staging, read_threads=threads)
        go()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            t0 = _t.perf_counter()
            go()
            torch.cuda.synchronize()
            ts.append((_t.perf_counter() - t0) * 1e3)
        lt.check_status(status)
        return float(np.median(ts))

    try:
        res = {"compressed_bytes": int(comp.size), "file": "page cache (written just before)"}
        for threads in (8, 1):
            seq = run(ht.n_chunks, threads)
            best = None
            for per_half in (64, 128, 256, 512):
                ms = run(per_half, threads)
                res["t%d_streamed_%d_per_half_ms" % (threads, per_half)] = round(ms, 3)
                best = ms if best is None else min(best, ms)
            res["t%d_sequential_ms" % threads] = round(seq, 3)
            res["t%d_speedup_best" % threads] = round(seq / best, 3)
        return res
    finally:
        os.unlink(path)


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
