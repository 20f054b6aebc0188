#!/usr/bin/env python3
"""Benchmark of the IQ4_XS x Q8_1 matmul on one MI355X.

Default run: `python bench.py [--steps K] [--warmup W]`.
One *step* is the whole hot path over the decode sweep of the attention/GDN
input-projection shape, N=10240, K=5120: for each M in {1, 2, 4, 8, 16} one
iq4xs_gemm_ws call (Q8_1 quantization of X on the device, the dispatcher's
choice of path, the matmul), with all inputs resident in HBM, launched on one
stream (the host runs ahead of the device, so the time is the device's);
weight copies are rotated (>= 640 MB in total) so the 256 MB Infinity Cache
cannot serve them.  The same calls recorded into HIP graphs and replayed are
reported as graph_ms_per_step (slower here: the replay leaves larger gaps
between the ten short kernels).

Printed: one JSON line with
  value      whole-step weight bandwidth = weight bytes read / step time (GB/s)
  per_m      ms per call, weight-GB/s, int8 TOPS and % of the HBM roofline
  roofline   for the dominant kernel (the matmul launch with the largest
             duration): algorithmic bytes per launch / its average duration,
             timed with HIP events on the stream the kernel runs on
  t_m2_over_m1  per-call time at M=2 over M=1 (flat in M is the aim)
  read_probe what a plain 1 GiB read achieves here (torch.sum), beside 8 TB/s
  group      one X against a pair of decode-shape matrices: the grouped call
             (one quantization, one matmul launch) against two separate calls
  cpu_baseline  the CPU oracle (never tuned) on a bounded sample of the same
             sweep, in the same unit.
`--sweep FILE` additionally times every (shape, M, path) point of the five
workloads and writes one JSON object per point to FILE (used for the measured
dispatch table and the results tables).

Profiling helpers (the commands are recorded in the summaries under profiles/):
`--profile-run` launches the decode sweep's matmul kernels and a calibration
copy a fixed number of times (run under rocprofv3); `--summarize-pmc FETCH_DIR
WRITE_DIR --out FILE` turns the two counter runs into the traffic summary
that the `roofline.traffic` field is read from (only while the kernel source
it was measured on is unchanged).
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import iq4_xs_q8_amd as iq  # noqa: E402
import synth  # noqa: E402

METRIC = "IQ4_XS GEMM ms + weight-GB/s/int8-TOPS, % roofline, at M=1..512"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0         # MI355X dense int8 MFMA, published
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published
MALL_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_mmv_decode_n10240_k5120_traffic.txt")
COPY_BYTES = 256 << 20          # calibration copy of the profiling run
KERNEL_SOURCES = {"k_mmv": ["mmv.hip", "common.hpp", "stream.hpp"], "k_gemv": ["gemv.hip", "common.hpp"],
                  "k_mmq": ["mmq.hip", "common.hpp"], "k_mmqt": ["mmqt.hip", "common.hpp", "stream.hpp"],
                  "k_gemm_bf16": ["deq.hip", "common.hpp"]}


def kernel_name(M, N, K, path):
    """The matmul kernel a call launches (the streaming kernel serves MMQ up
    to M=32 when K/256 is even)."""
    if path == iq.PATH_GEMV:
        return "k_gemv"
    if path == iq.PATH_DEQ_BF16:
        return "k_gemm_bf16"
    nb = K // 256
    if M <= 32 and nb % 2 == 0 and N * nb * 136 < (1 << 31):
        return "k_mmv"
    return "k_mmqt" if M > 32 else "k_mmq"


def source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "iq4_xs_q8_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algo_bytes_call(M, N, K):
    """Algorithmic HBM bytes of one iq4xs_gemm call: the weights once, X read
    (4 B/element), the quantized activations written and read (1.125 B/element
    each way) and Y written."""
    return 0.53125 * N * K + (4 + 2 * 1.125) * M * K + 4 * M * N


def algo_bytes_kernel(M, N, K):
    """Algorithmic bytes of one matmul launch: weights, prepared activations
    (1 B per value + 4 B scale per 32), Y."""
    return 0.53125 * N * K + 1.125 * M * K + 4 * M * N


class Rotation:
    """Copies of one weight matrix, enough to exceed twice the MALL (a
    multiple of `group` copies)."""

    def __init__(self, W: np.ndarray, min_total=640 << 20, group=1):
        base = torch.from_numpy(W).cuda()
        n = max(2, math.ceil(min_total / base.numel()))
        n = -(-n // group) * group
        self.ws = [base] + [base.clone() for _ in range(n - 1)]
        self.i = 0

    def next(self):
        w = self.ws[self.i]
        self.i = (self.i + 1) % len(self.ws)
        return w


def time_events(fn, reps, stream):
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        fn()
    stop.record(stream)
    stop.synchronize()
    return start.elapsed_time(stop) / reps      # ms


def measure_point(rot, X, N, K, path, reps=30):
    """Per iq4xs_gemm call: ms on the device (`reps` calls over rotating
    weight copies recorded in one HIP graph and replayed, so host launch
    cost is not counted) and ms launched eagerly from the host; and ms per
    launch of the matmul kernel alone (prepared activations, Y marked as
    zeroed so that nothing else runs; its values are not used).  All from HIP
    events on the launching stream."""
    M = X.shape[0]
    Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(iq.workspace_bytes(M, N, K, path), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    call = lambda: iq.gemm(rot.next(), X, path=path, out=Y, workspace=ws)  # noqa: E731
    for _ in range(3):
        call()
    t_eager = time_events(call, reps, stream)
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        call()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            call()
    g.replay()
    t_call = time_events(g.replay, 3, stream) / reps
    del g
    t_kern = None
    if path != iq.PATH_DEQ_BF16:
        act = iq.prepare_act(X)
        Y.zero_()
        kern = lambda: iq.gemm_act(rot.next(), act, M, K, path=path, out=Y, y_zeroed=True)  # noqa: E731
        for _ in range(3):
            kern()
        t_kern = time_events(kern, reps, stream)
    return t_call, t_kern, t_eager


def measure_group(ms=(1, 8, 16), reps=20):
    """One X against two weight matrices of the decode shape (N=10240,
    K=5120; e.g. two input projections of one layer): one grouped call (one
    quantization, one matmul launch over both) against two iq4xs_gemm calls,
    both with caller workspaces.  ms per pair on the device: `reps` pairs (each on another rotated weight
    pair, past the Infinity Cache) recorded in one HIP graph and replayed, as
    for the per-call times.  (The same shape as the decode sweep, so that a
    kernel trace of the bench run averages one shape per kernel.)"""
    wl = synth.DECODE_ATTN
    N, K = wl.shapes[0]
    base = torch.from_numpy(wl.w(N, K)).cuda()
    npairs = max(2, math.ceil((640 << 20) / (2 * base.numel())))
    pairs = [(base.clone(), base.clone()) for _ in range(npairs)]
    del base
    stream = torch.cuda.current_stream()
    wb = 2 * 0.53125 * N * K
    points = []
    for M in ms:
        X = torch.from_numpy(wl.x(M, K, N=N)).cuda()
        Y = [torch.empty((M, N), dtype=torch.float32, device="cuda") for _ in range(2)]
        # caller workspaces on both sides: nothing is allocated inside the calls
        gws = torch.empty(iq.group_workspace_bytes([N, N], M, K), dtype=torch.uint8, device="cuda")
        sws = torch.empty(iq.workspace_bytes(M, N, K), dtype=torch.uint8, device="cuda")

        def grouped(i):
            a, b = pairs[i % npairs]
            iq.gemm_group([a, b], X, Y, workspace=gws)

        def separate(i):
            a, b = pairs[i % npairs]
            iq.gemm(a, X, out=Y[0], workspace=sws)
            iq.gemm(b, X, out=Y[1], workspace=sws)

        t = {}
        for name, f in (("grouped", grouped), ("separate", separate)):
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                for i in range(3):
                    f(i)
            stream.wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(reps):
                    f(i)
            g.replay()
            t[name] = time_events(g.replay, 3, stream) / reps
            del g
        points.append({"M": M, "grouped_ms": t["grouped"], "separate_ms": t["separate"],
                       "speedup": t["separate"] / t["grouped"],
                       "grouped_weight_GBs": wb / (t["grouped"] * 1e-3) / 1e9,
                       "grouped_hbm_frac": (wb + (4 + 2.25) * M * K + 8 * M * N) / (t["grouped"] * 1e-3) / 1e9
                       / HBM_PEAK_GBS})
    del pairs
    torch.cuda.empty_cache()
    return {"workload": "pair of N=10240 K=5120 matrices sharing X (grouped call vs two calls), "
                        "quantize included, graph replay", "points": points}


def read_probe(nbytes=1 << 30, reps=10):
    """What a plain read of nbytes achieves on this device (torch.sum over a
    fresh fp32 buffer, so the Infinity Cache holds at most a quarter of it):
    a reference beside the published 8 TB/s, not a kernel of this library."""
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.ones_like(x)
    stream = torch.cuda.current_stream()
    for _ in range(2):
        x.sum()
    t = time_events(lambda: (x.sum(), y.sum()), reps, stream) / 2
    del x, y
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "ms": t, "GBs": nbytes / (t * 1e-3) / 1e9, "kernel": "torch.sum (fp32, 1 GiB)"}


def point_record(N, K, M, path, t_call, t_kern, t_eager=None):
    wb = 0.53125 * N * K
    ops = 2.0 * M * N * K
    rec = {"N": N, "K": K, "M": M, "path": iq.path_name(path), "ms": t_call, "eager_ms": t_eager,
           "weight_GBs": wb / (t_call * 1e-3) / 1e9,
           "int8_TOPS": ops / (t_call * 1e-3) / 1e12,
           "hbm_frac": algo_bytes_call(M, N, K) / (t_call * 1e-3) / 1e9 / HBM_PEAK_GBS}
    if t_kern is not None:
        rec["kernel_ms"] = t_kern
        rec["kernel_GBs"] = algo_bytes_kernel(M, N, K) / (t_kern * 1e-3) / 1e9
        rec["kernel_hbm_frac"] = rec["kernel_GBs"] / HBM_PEAK_GBS
        rec["kernel_mfma_frac"] = ops / (t_kern * 1e-3) / 1e12 / INT8_PEAK_TOPS
    rec["mfma_frac"] = rec["int8_TOPS"] / INT8_PEAK_TOPS
    # impossible-throughput flag: faster than the card can move the bytes
    rec["impossible"] = bool(rec["hbm_frac"] > 1.0 or rec.get("kernel_hbm_frac", 0) > 1.0
                             or rec["mfma_frac"] > 1.0)
    return rec


def cpu_baseline(wl, N, K, ms, target_s=12.0):
    """The oracle (as it stands) on a sample of output columns of the same
    sweep; returns weight-GB/s of that sample."""
    import oracle
    o = oracle.get()
    W = wl.w(N, K)
    Xs = {M: wl.x(M, K, N=N) for M in ms}

    def run(ncols):
        Ws = np.ascontiguousarray(W[:ncols])
        t0 = time.perf_counter()
        for M in ms:
            o.gemm_q8_1(Ws, o.quantize_q8_1(Xs[M]), K)
        return time.perf_counter() - t0

    probe = 64
    t = run(probe)
    ncols = int(min(N, max(probe, probe * target_s / max(t, 1e-3))))
    reps, t = 0, 0.0
    while reps == 0 or t < target_s:      # the whole sweep can take well under target_s
        t += run(ncols)
        reps += 1
    wbytes = 0.53125 * ncols * K * len(ms) * reps
    return {"value": wbytes / t / 1e9, "unit": "weight-GB/s", "cores": o.threads(), "kind": "oracle",
            "sample": f"{ncols} of {N} output columns, every M in {list(ms)}, quantize included, "
                      f"{reps} pass(es), {t:.1f} s"}


def profile_run():
    """Fixed launches for rocprofv3: per M of the decode sweep, 20 launches
    of the matmul kernel alone (rotated weights, as in the timed step), then
    a calibration copy of COPY_BYTES, 4 times."""
    wl = synth.DECODE_ATTN
    (N, K), ms = wl.shapes[0], wl.ms
    rot = Rotation(wl.w(N, K))
    for M in ms:
        X = torch.from_numpy(wl.x(M, K, N=N)).cuda()
        act = iq.prepare_act(X)
        Y = torch.zeros((M, N), dtype=torch.float32, device="cuda")
        path = iq.dispatch(M, N, K)
        for _ in range(20):
            iq.gemm_act(rot.next(), act, M, K, path=path, out=Y, y_zeroed=True)
        torch.cuda.synchronize()
        print(f"[profile-run] M={M} {kernel_name(M, N, K, path)} x20", flush=True)
    # the copy's source must come from HBM, not from the 256 MB Infinity
    # Cache: fill four buffers, then copy the first (three later fills have
    # evicted it), once per buffer
    bufs = [torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(float(i)) for i in range(4)]
    dst = torch.empty_like(bufs[0])
    for i in range(4):
        for j in range(1, 4):
            bufs[(i + j) % 4].fill_(float(j))
        dst.copy_(bufs[i])
    torch.cuda.synchronize()
    print(f"[profile-run] copy {COPY_BYTES} bytes x4", flush=True)


def profile_shapes(specs):
    """Fixed launches for rocprofv3 at given shapes ("MxNxK", comma
    separated): per shape, 20 launches of the matmul kernel(s) alone
    (gemm_act, rotated weights), inputs of the workload the shape belongs to
    (else the prefill recipe)."""
    for spec in specs.split(","):
        M, N, K = (int(v) for v in spec.split("x"))
        wl = next((w for w in synth.WORKLOADS if (N, K) in w.shapes), synth.WORKLOADS[-1])
        rot = Rotation(wl.w(N, K))
        X = torch.from_numpy(wl.x(M, K, N=N)).cuda()
        act = iq.prepare_act(X)
        Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        path = iq.dispatch(M, N, K)
        for _ in range(20):
            iq.gemm_act(rot.next(), act, M, K, path=path, out=Y)
        torch.cuda.synchronize()
        print(f"[profile-shapes] M={M} N={N} K={K} {kernel_name(M, N, K, path)} x20", flush=True)
        del rot
        torch.cuda.empty_cache()


def _counter_rows(d):
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {d}")
    return rows


def summarize_pmc(fetch_dir, write_dir, out, cmd_fetch, cmd_write):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the matmul kernels and of
    the calibration copy -> calibrated HBM bytes per launch."""
    def per_kernel(rows, counter):
        acc = {}
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            key = ("copy" if "copyBuffer" in name else
                   "k_mmv" if "k_mmv" in name else "k_gemv" if "k_gemv" in name else
                   "k_mmqt_fix" if "k_mmqt_fix" in name else "k_mmqt" if "k_mmqt" in name else
                   "k_mmq" if "k_mmq" in name else None)
            if key is None:
                continue
            label = name.split("Cfg<")[1].split(">")[0].replace(" ", "") if "Cfg<" in name else ""
            acc.setdefault((key, label), {}).setdefault(r["Dispatch_Id"], 0.0)
            acc[(key, label)][r["Dispatch_Id"]] += float(r["Counter_Value"])
        return {k: list(v.values()) for k, v in acc.items()}
    fetch_all = per_kernel(_counter_rows(fetch_dir), "FETCH_SIZE")
    write_all = per_kernel(_counter_rows(write_dir), "WRITE_SIZE")
    # the calibration copies are the copyBuffer dispatches far above the
    # weight-copy sizes; everything else is averaged per kernel
    cf = [v for (k, _), vs in fetch_all.items() if k == "copy" for v in vs if v * 1024.0 > COPY_BYTES / 16]
    cw = [v for (k, _), vs in write_all.items() if k == "copy" for v in vs if v * 1024.0 > COPY_BYTES / 16]
    fetch = {k: sum(v) / len(v) for k, v in fetch_all.items()}
    write = {k: sum(v) / len(v) for k, v in write_all.items()}
    if not cf or not cw:
        raise SystemExit("calibration copy not found in the counter runs")
    f_scale = COPY_BYTES / (sum(cf) / len(cf) * 1024.0)       # true bytes per counted byte
    w_scale = COPY_BYTES / (sum(cw) / len(cw) * 1024.0)
    wl = synth.DECODE_ATTN
    (N, K), ms = wl.shapes[0], wl.ms
    lines = [f"# HBM traffic per launch from rocprofv3 counters, decode sweep N={N} K={K}",
             f"# fetch run: {cmd_fetch}", f"# write run: {cmd_write}",
             f"copy_bytes {COPY_BYTES}",
             f"copy_fetch_kib {sum(cf) / len(cf):.1f}  fetch_scale {f_scale:.4f}",
             f"copy_write_kib {sum(cw) / len(cw):.1f}  write_scale {w_scale:.4f}",
             f"source_hash k_mmv {source_hash('k_mmv')}",
             "# kernel config  fetch_kib  write_kib  calibrated_bytes  algorithmic_bytes(M)"]
    for (k, label), fk in sorted(fetch.items()):
        if k == "copy":
            continue
        wk = write.get((k, label), 0.0)
        total = fk * 1024.0 * f_scale + wk * 1024.0 * w_scale
        lines.append(f"traffic {k} <{label}> {fk:.1f} {wk:.1f} {total:.0f}")
    for M in ms:
        lines.append(f"algorithmic M={M} {algo_bytes_kernel(M, N, K):.0f}")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


SQ_PASSES = (("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU",
              "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES"),
             ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_LDS_BANK_CONFLICT",
              "SQ_WAIT_INST_LDS", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_ANY"))


def _sq_key(name, order, shapes):
    """Kernel label; the tile kernel's launches of a --profile-shapes run
    (20 per shape, in order) also carry their shape."""
    key = name.replace("void ", "").replace("iq4xs::(anonymous namespace)::", "").split("(")[0]
    if shapes and "k_mmqt<" in key and order is not None:
        i = order // 20
        if i < len(shapes):
            key += " [M=%d N=%d K=%d]" % shapes[i]
    return key


def _tile_order(rows, id_field):
    """Launch index of every tile-kernel dispatch (not the summing kernel)."""
    ids = sorted({int(r[id_field]) for r in rows if "k_mmqt<" in r["Kernel_Name"]})
    return {i: n for n, i in enumerate(ids)}


def summarize_sq(dirs, trace_dirs, out, cmds, specs=""):
    """Per matmul kernel (by template arguments, and shape for the tile
    kernel): the average per dispatch of the SQ counters of the given runs;
    VALU instructions per MFMA instruction, LDS bank-conflict cycles per LDS
    instruction; and, with kernel traces of the same launches, the share of
    the kernel's duration that VALU issue (instructions x 4 cycles, spread
    over 1024 SIMDs at 2.4 GHz) and the matrix cores (busy cycles over 1024
    SIMDs) take."""
    shapes = [tuple(int(v) for v in sp.split("x")) for sp in specs.split(",")] if specs else []
    per = {}
    for d in dirs:
        rows = _counter_rows(d)
        order = _tile_order(rows, "Dispatch_Id")
        for r in rows:
            name = r["Kernel_Name"]
            if not any(k in name for k in ("k_mmv", "k_gemv", "k_mmqt", "k_mmq", "k_quantize")):
                continue
            key = _sq_key(name, order.get(int(r["Dispatch_Id"])), shapes)
            per.setdefault(key, {}).setdefault(r["Counter_Name"], {}).setdefault(r["Dispatch_Id"], 0.0)
            per[key][r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    dur = {}
    for td in trace_dirs:
        files = glob.glob(os.path.join(td, "**", "*kernel_trace.csv"), recursive=True)
        rows = list(csv.DictReader(open(files[0])))
        order = _tile_order(rows, "Dispatch_Id")
        for r in rows:
            key = _sq_key(r["Kernel_Name"], order.get(int(r["Dispatch_Id"])), shapes)
            dur.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
    lines = ["# SQ counters per dispatch (averages), matmul and quantize kernels of the decode sweep and the tile shapes",
             *[f"# run: {c}" for c in cmds],
             "# VALU/MFMA: instructions; LDS-conflict: bank-conflict cycles per LDS instruction; VALU-issue and "
             "MFMA-busy: per SIMD, as a share of the kernel's average duration in the trace",
             "# kernel | " + " ".join(c for p_ in SQ_PASSES for c in p_) +
             " | VALU/MFMA  LDS-conflict  trace-us  VALU-issue  MFMA-busy"]
    for key in sorted(per):
        v = {c: sum(d.values()) / len(d) for c, d in per[key].items()}
        vals = " ".join(f"{v.get(c, float('nan')):.4g}" for p_ in SQ_PASSES for c in p_)
        valu, mfma = v.get("SQ_INSTS_VALU", 0.0), v.get("SQ_INSTS_MFMA", 0.0)
        lds, conf = v.get("SQ_INSTS_LDS", 0.0), v.get("SQ_LDS_BANK_CONFLICT", 0.0)
        d_us = sum(dur[key]) / len(dur[key]) if key in dur else float("nan")
        issue = valu * 4 / 1024 / 2.4e3 / d_us
        busy = v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / 1024 / 2.4e3 / d_us
        lines.append(f"{key} | {vals} | {valu / mfma if mfma else float('nan'):.2f}  "
                     f"{conf / lds if lds else float('nan'):.3f}  {d_us:.2f}  {issue:.2f}  {busy:.2f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_trace(trace_dir, out, cmd, title):
    """The kernel-trace statistics of a rocprofv3 --stats run as a short text
    table (kernel, calls, average / min / max microseconds, share of GPU
    time)."""
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    with open(files[0]) as fh:
        rows = list(csv.DictReader(fh))
    def short(name):
        name = name.replace("iq4xs::(anonymous namespace)::", "").replace("iq4xs::", "")
        return name.split("(")[0] if not name.startswith("void k_") else name.split("(")[0]
    lines = [f"# rocprofv3 kernel-trace statistics: {title}", f"# command: {cmd}",
             f"{'kernel':60s} {'calls':>6s} {'avg_us':>8s} {'min_us':>8s} {'max_us':>8s} {'pct':>6s}"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"{short(r['Name'])[:60]:60s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:8.2f} "
                     f"{float(r['MinNs']) / 1e3:8.2f} {float(r['MaxNs']) / 1e3:8.2f} {float(r['Percentage']):6.2f}")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_pmc_shapes(fetch_dir, write_dir, out, cmd_fetch, cmd_write, specs):
    """Per shape of a --profile-shapes run (20 launches each, in order): mean
    FETCH_SIZE / WRITE_SIZE per launch of the tile kernel and of its
    shared-tile kernel, calibrated with the copy runs of a --profile-run
    summary (TRAFFIC_FILE), against the algorithmic bytes."""
    with open(TRAFFIC_FILE) as fh:
        sc = {ln.split()[2]: float(ln.split()[3]) for ln in fh if ln.startswith("copy_") and "scale" in ln}
    f_scale, w_scale = sc["fetch_scale"], sc["write_scale"]
    def per_dispatch(d, counter):
        acc = {}
        for r in _counter_rows(d):
            if r["Counter_Name"] == counter and "k_mmqt" in r["Kernel_Name"]:
                k = (int(r["Dispatch_Id"]), "fix" if "k_mmqt_fix" in r["Kernel_Name"] else "main")
                acc[k] = acc.get(k, 0.0) + float(r["Counter_Value"])
        return acc
    fd, wd = per_dispatch(fetch_dir, "FETCH_SIZE"), per_dispatch(write_dir, "WRITE_SIZE")
    shapes = [tuple(int(v) for v in sp.split("x")) for sp in specs.split(",")]
    lines = ["# HBM traffic per launch of the tile kernel from rocprofv3 counters (20 launches per shape)",
             f"# fetch run: {cmd_fetch}", f"# write run: {cmd_write}",
             f"# scales from the copy calibration of {os.path.basename(TRAFFIC_FILE)}: fetch x{f_scale:.4f}, write x{w_scale:.4f}",
             f"source_hash k_mmqt {source_hash('k_mmqt')}",
             "# M N K  kernel  fetch_MB  write_MB  calibrated_MB  algorithmic_MB (W + planes + Y)"]
    # dispatches in launch order: 20 tile-kernel launches per shape, each
    # followed by its summing kernel where the shape has one
    sums = {}
    n_main = -1
    for (i, part) in sorted(set(fd) | set(wd)):
        if part == "main":
            n_main += 1
        shape = n_main // 20
        acc = sums.setdefault((shape, part), [0.0, 0.0, 0])
        acc[0] += fd.get((i, part), 0.0)
        acc[1] += wd.get((i, part), 0.0)
        acc[2] += 1
    for (shape, part), (f, w, cnt) in sorted(sums.items(), key=lambda kv: (kv[0][1] != "main", kv[0][0])):
        if shape >= len(shapes):
            continue
        M, N, K = shapes[shape]
        fb = f / cnt * 1024.0 * f_scale
        wb = w / cnt * 1024.0 * w_scale
        lines.append(f"{M} {N} {K}  {'k_mmqt' if part == 'main' else 'k_mmqt_fix'}  {fb / 1e6:.1f}  {wb / 1e6:.1f}  "
                     f"{(fb + wb) / 1e6:.1f}  {algo_bytes_kernel(M, N, K) / 1e6 if part == 'main' else 0:.1f}")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def traffic_for(kernel, label):
    """Calibrated bytes per launch from the committed summary, or None when
    the summary is missing or the kernel source changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as fh:
        lines = fh.read().splitlines()
    if f"source_hash {kernel} {source_hash(kernel)}" not in lines:
        return None
    for ln in lines:
        parts = ln.split()
        if len(parts) == 6 and parts[0] == "traffic" and parts[1] == kernel and parts[2] == f"<{label}>":
            return float(parts[5])
    return None


def run_sweep(path_out):
    """Every (shape, M, path) point of the five workloads -> JSONL."""
    with open(path_out, "w") as f:
        for wl in synth.WORKLOADS:
            for (N, K) in wl.shapes:
                rot = Rotation(wl.w(N, K))
                for M in wl.ms:
                    X = torch.from_numpy(wl.x(M, K, N=N)).cuda()
                    paths = [iq.PATH_AUTO, iq.PATH_MMQ]
                    if M <= 4:
                        paths.append(iq.PATH_GEMV)
                    if M >= 32:
                        paths.append(iq.PATH_DEQ_BF16)
                    for p in paths:
                        rec = point_record(N, K, M, p, *measure_point(rot, X, N, K, p, reps=20))
                        rec["workload"] = wl.name
                        if p == iq.PATH_AUTO:
                            rec["auto"] = iq.path_name(iq.dispatch(M, N, K))
                        f.write(json.dumps(rec) + "\n")
                        f.flush()
                        print(f"[sweep] {wl.cid} N={N} K={K} M={M} {rec['path']}: {rec['ms']:.4f} ms "
                              f"{rec['weight_GBs']:.0f} GB/s", flush=True)
                del rot
                torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sweep", default=None, help="also time every workload point -> JSONL")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-run", action="store_true", help="fixed launches for rocprofv3")
    ap.add_argument("--profile-shapes", default=None, help="MxNxK,...: fixed launches for rocprofv3")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR")
    ap.add_argument("--summarize-pmc-shapes", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "SHAPES"))
    ap.add_argument("--summarize-sq", nargs="+", metavar="DIR", help="SQ counter runs -> instruction mix")
    ap.add_argument("--trace-dir", default=None, help="kernel-trace runs of the same launches, comma-separated")
    ap.add_argument("--shapes", default="", help="MxNxK,... of the --profile-shapes runs")
    ap.add_argument("--cmd", default="")
    ap.add_argument("--title", default="")
    ap.add_argument("--out", default=TRAFFIC_FILE)
    ap.add_argument("--cmd-fetch", default="")
    ap.add_argument("--cmd-write", default="")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, args.out, args.cmd_fetch, args.cmd_write)
        return
    if args.summarize_pmc_shapes:
        if args.out == TRAFFIC_FILE:
            raise SystemExit("--summarize-pmc-shapes needs its own --out")
        summarize_pmc_shapes(*args.summarize_pmc_shapes[:2], args.out, args.cmd_fetch, args.cmd_write,
                             args.summarize_pmc_shapes[2])
        return
    if args.summarize_sq:
        if args.out == TRAFFIC_FILE:
            raise SystemExit("--summarize-sq needs its own --out")
        summarize_sq(args.summarize_sq, [d for d in (args.trace_dir or "").split(",") if d], args.out,
                     [c for c in args.cmd.split(";;") if c], args.shapes)
        return
    if args.summarize_trace:
        if args.out == TRAFFIC_FILE:
            raise SystemExit("--summarize-trace needs its own --out")
        summarize_trace(args.summarize_trace, args.out, args.cmd, args.title)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the matmul is built and measured on a single MI355X "
              "(multi-GPU sharding is a design note only); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.profile_run:
        profile_run()
        return
    if args.profile_shapes:
        profile_shapes(args.profile_shapes)
        return

    wl = synth.DECODE_ATTN
    (N, K), ms = wl.shapes[0], wl.ms
    rot = Rotation(wl.w(N, K), group=len(ms))
    Xs = {M: torch.from_numpy(wl.x(M, K, N=N)).cuda() for M in ms}
    Ys = {M: torch.empty((M, N), dtype=torch.float32, device="cuda") for M in ms}
    wss = {M: torch.empty(iq.workspace_bytes(M, N, K), dtype=torch.uint8, device="cuda") for M in ms}

    # One step = one iq4xs_gemm_ws call per M (quantization + matmul) on one
    # stream.  The same calls recorded into a HIP graph per group of weight
    # copies, as a decode loop might replay them, are timed beside it.
    def step_on(ws_list):
        for M, w in zip(ms, ws_list):
            iq.gemm(w, Xs[M], out=Ys[M], workspace=wss[M])

    groups = [rot.ws[i:i + len(ms)] for i in range(0, len(rot.ws), len(ms))]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step_on(groups[0])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for grp in groups:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step_on(grp)
        graphs.append(g)
    stream = torch.cuda.current_stream()

    def timed(fn, steps, warmup):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for i in range(steps):
            fn(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / steps, time.perf_counter() - t0

    step_ms, wall = timed(lambda i: step_on(groups[i % len(groups)]), args.steps, args.warmup)
    graph_ms, _ = timed(lambda i: graphs[i % len(graphs)].replay(), args.steps, args.warmup)
    wbytes = 0.53125 * N * K * len(ms)
    value = wbytes / (step_ms * 1e-3) / 1e9

    per_m = []
    for M in ms:
        path = iq.dispatch(M, N, K)
        per_m.append(point_record(N, K, M, path, *measure_point(rot, Xs[M], N, K, path)))
    dom = max(per_m, key=lambda r: r["kernel_ms"])
    dom_kernel = kernel_name(dom["M"], N, K, iq.PATHS[dom["path"]])
    achieved = algo_bytes_kernel(dom["M"], N, K) / (dom["kernel_ms"] * 1e-3) / 1e9
    label = {1: "1,4,8,3,false", 2: "1,4,8,3,true", 4: "2,4,8,3,true", 8: "4,8,4,3,false",
             16: "8,16,4,3,false"}.get(dom["M"], "") if dom_kernel == "k_mmv" else ""
    traffic = traffic_for(dom_kernel, label)
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS,
                "traffic": None if traffic is None else traffic / (dom["kernel_ms"] * 1e-3) / 1e9,
                "traffic_bytes_per_launch": traffic,
                "kernel": dom_kernel, "M": dom["M"],
                "bytes_per_launch": algo_bytes_kernel(dom["M"], N, K),
                "avg_launch_ms": dom["kernel_ms"]}

    out = {"metric": METRIC, "value": value, "unit": "weight-GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": step_ms,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
           "data": "synthetic (seeded IQ4_XS weights, N(0,1) activations with 1% outlier channels)",
           "config": {"workload": "IQ4_XS x Q8_1 GEMM decode sweep, attention/GDN input projection "
                                  "N=10240 K=5120, M in {1,2,4,8,16}, quantize included",
                      "N": N, "K": K, "M": list(ms), "weight_copies": len(rot.ws)},
           "wall_s": wall, "graph_ms_per_step": graph_ms,
           "graph_weight_GBs": wbytes / (graph_ms * 1e-3) / 1e9, "per_m": per_m, "roofline": roofline}
    del graphs
    by_m = {r["M"]: r for r in per_m}
    if 1 in by_m and 2 in by_m:
        out["t_m2_over_m1"] = by_m[2]["ms"] / by_m[1]["ms"]
    out["group"] = measure_group()
    out["read_probe"] = read_probe()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, N, K, ms)
    if args.sweep:
        del rot
        torch.cuda.empty_cache()
        run_sweep(args.sweep)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
