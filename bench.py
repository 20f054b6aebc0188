#!/usr/bin/env python3
"""Benchmark of the IQ4_XS x Q8_1 matmul on one MI355X.

Default run: `python bench.py [--steps K] [--warmup W]`.
One *step* is one pass of the whole hot path over the five synthetic
workloads, M = 1..512: one iq4xs_gemm call (Q8_1 quantization of X on the
device, the measured dispatcher's choice of path, the matmul) for every
point of
  - a single 2048 x 2048 GEMM at M=4;
  - the attention/GDN input projection N=10240 K=5120, decode M in {1,2,4,8,16};
  - the MLP gate/up shape N=17408 K=5120, M in {8,16,32,64,96};
  - the MLP down shape N=5120 K=17408, M in {1,12,32,64,96};
  - the prefill sweep: nine (N, K) shapes x M in {64,128,256,512}
(52 calls), all inputs resident in HBM, launched back to back on one stream
(the host runs ahead, so the time is the device's); every shape's weights
are rotated over copies of >= 640 MB, so the 256 MB Infinity Cache cannot
serve them.

Printed: one JSON line with
  value        whole-step weight bandwidth = weight bytes of all 52 calls / step time
  int8_TOPS    2*sum(M*N*K) / step time
  points       per (shape, M): ms per call (graph replay, quantization included),
               ms of the matmul kernel(s) alone, weight-GB/s, int8 TOPS, the
               fractions of the HBM and int8-MFMA rooflines, the bound that
               binds (the larger of bytes/8 TB/s and ops/5 POP/s), the kernel
  roofline     the dominant kernel (largest share of the step's kernel time):
               algorithmic work per launch / its average duration, timed with
               HIP events on the stream it runs on
  rooflines    the same for the dominant point of each matmul kernel
  probes       this device's own ceilings: a stream read (28 MB, 95 MB, 1 GiB,
               rotated past the Infinity Cache), a stream write, back-to-back
               int8 and bf16 matrix-core instructions
  group        one X against a pair of decode-shape matrices: grouped call vs two calls
  formats      a few points with IQ4_NL and Q4_0 weights
  fused_bf16x3 the fused bf16 paths (BF16X3, and DEQ_BF16) at every prefill
               point, beside the path the table picks there
  cpu_baseline the CPU oracle (never tuned) on a bounded column sample of the
               same 52 points, in the same unit.
`--sweep FILE` times every (shape, M, path) point and writes one JSON object
per point to FILE (the input of the dispatch-table calibration).

Profiling helpers (the commands are recorded in the summaries under
profiles/): `--profile-points` launches every point's call with a marker
kernel between points (run under rocprofv3 --kernel-trace; `--check-trace`
then checks that every call launched the quantizer and the matmul kernel its
path names); `--profile-run` / `--profile-shapes` launch matmul kernels and
the read / write probes of known bytes a fixed number of times (run under
rocprofv3 --pmc; `--summarize-pmc*` turns FETCH_SIZE / WRITE_SIZE into
calibrated bytes per launch).
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import re
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
PROBE_BYTES = 1 << 30           # calibration read / write of the profiling runs
# launches per shape of the profiling runs: warm-up (the first few calls on
# rotated weights run up to 30% slower), then the measured ones; the
# summaries keep the measured ones
PROFILE_WARM, PROFILE_RUNS = 10, 20
PROFILE_GROUP = PROFILE_WARM + PROFILE_RUNS


def _measured(seq):
    """The measured launches of one kernel's launches in a profiling run."""
    return seq[PROFILE_WARM:] if len(seq) >= PROFILE_GROUP else seq
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_mmv_decode_n10240_k5120_traffic.txt")
TILE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_mmqt_tile_shapes_traffic.txt")
KERNEL_SOURCES = {"k_mmv": ["mmv.hip", "common.hpp", "stream.hpp"], "k_gemv": ["gemv.hip", "common.hpp"],
                  "k_mmq": ["mmq.hip", "common.hpp"], "k_mmqt": ["mmqt.hip", "common.hpp", "stream.hpp"],
                  "k_gemm_x3": ["fused.hip", "common.hpp", "stream.hpp"],
                  "k_gemm_deq": ["fused.hip", "common.hpp", "stream.hpp"]}
# Exact formulation on the matrix cores: per (output, 32-wide sub-block) the
# int8 MFMA does 32 MACs (0.031 cycles per SIMD at 2048 ops/cycle) and the
# fp32 rescale three VALU instructions (0.1875 cycles at 16 lanes/cycle,
# packed fp32 off): the tile kernel cannot pass 1/6 of the int8 peak.
VALU_CEILING_FRAC = (64 / 2048) / (3 * 4 / 64)


def kernel_name(M, N, K, path):
    """The matmul kernel a call launches (the streaming kernel serves MMQ up
    to M=32 when K/256 is even; --check-trace verifies this against the
    rocprofv3 trace)."""
    if path == iq.PATH_GEMV:
        return "k_gemv"
    if path == iq.PATH_BF16X3:
        return "k_gemm_x3"
    if path == iq.PATH_DEQ_BF16:
        return "k_gemm_deq"
    nb = K // 256
    if M <= 32 and nb % 2 == 0 and N * nb * 136 < (1 << 31):
        return "k_mmv"
    return "k_mmqt" if M > 32 and N * nb * 136 < (1 << 31) else "k_mmq"


def source_hash(kernel):
    """Hash of a kernel's source files with comments and whitespace taken out,
    so that a profile stays valid across edits of the comments only."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "iq4_xs_q8_amd", "csrc", f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
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


def sweep_points():
    """(workload, N, K, M) of the 52 calls of one step."""
    return [(wl, N, K, M) for wl in synth.WORKLOADS for (N, K) in wl.shapes for M in wl.ms]


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


def time_graph(fn, reps, stream):
    """ms per call of `reps` calls of fn captured in one HIP graph and
    replayed (no host launch gaps between short kernels)."""
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        fn()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    t = time_events(g.replay, 3, stream) / reps
    del g
    return t


def time_events(fn, reps, stream):
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        fn()
    stop.record(stream)
    stop.synchronize()
    return start.elapsed_time(stop) / reps      # ms


def measure_point(rot, X, N, K, path, reps=20, fmt=iq.FMT_IQ4_XS):
    """Per call: ms on the device (`reps` calls over rotating weight copies
    recorded in one HIP graph and replayed, so host launch cost is not
    counted) and ms launched eagerly; and ms per launch of the matmul
    kernel(s) alone (prepared activations, Y marked as zeroed so that nothing
    else runs; its values are not used).  All from HIP events on the
    launching stream."""
    M = X.shape[0]
    Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    if fmt == iq.FMT_IQ4_XS:
        ws = torch.empty(iq.workspace_bytes(M, N, K, path), dtype=torch.uint8, device="cuda")
        call = lambda: iq.gemm(rot.next(), X, path=path, out=Y, workspace=ws)  # noqa: E731
    else:
        ws = torch.empty(iq.fmt_workspace_bytes(fmt, M, N, K, path), dtype=torch.uint8, device="cuda")
        call = lambda: iq.gemm_fmt(rot.next(), X, fmt, path=path, out=Y, workspace=ws)  # noqa: E731
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
    if path not in (iq.PATH_DEQ_BF16, iq.PATH_BF16X3) and fmt == iq.FMT_IQ4_XS:
        act = iq.prepare_act(X)
        Y.zero_()
        # the partial-tile scratch from the caller: the launch allocates
        # nothing and is replayed from a graph like the calls (no host gaps
        # between short kernels)
        kws = torch.empty(iq.act_workspace_bytes(M, N, K, path), dtype=torch.uint8, device="cuda")
        kern = lambda: iq.gemm_act(rot.next(), act, M, K, path=path, out=Y, y_zeroed=True,  # noqa: E731
                                   workspace=kws)
        for _ in range(3):
            kern()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            kern()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                kern()
        g.replay()
        t_kern = time_events(g.replay, 3, stream) / reps
        del g
    return t_call, t_kern, t_eager


def point_record(N, K, M, path, t_call, t_kern, t_eager=None):
    """Per point: ms, weight-GB/s, int8 TOPS, the fraction of each roofline
    and the one that binds.  Algorithmic bytes and ops (2*M*N*K) per call;
    with the kernel alone, its own algorithmic bytes."""
    wb = 0.53125 * N * K
    ops = 2.0 * M * N * K
    t_hbm = algo_bytes_call(M, N, K) / (HBM_PEAK_GBS * 1e9) * 1e3      # ms at the HBM peak
    t_mfma = ops / (INT8_PEAK_TOPS * 1e12) * 1e3                         # ms at the int8 peak
    rec = {"N": N, "K": K, "M": M, "path": iq.path_name(path), "ms": t_call, "eager_ms": t_eager,
           "weight_GBs": wb / (t_call * 1e-3) / 1e9,
           "int8_TOPS": ops / (t_call * 1e-3) / 1e12,
           "hbm_frac": t_hbm / t_call, "mfma_frac": t_mfma / t_call,
           "bound": "hbm" if t_hbm >= t_mfma else "mfma",
           "roofline_frac": max(t_hbm, t_mfma) / t_call}
    if t_kern is not None:
        tk_hbm = algo_bytes_kernel(M, N, K) / (HBM_PEAK_GBS * 1e9) * 1e3
        rec["kernel_ms"] = t_kern
        rec["kernel_GBs"] = algo_bytes_kernel(M, N, K) / (t_kern * 1e-3) / 1e9
        rec["kernel_hbm_frac"] = tk_hbm / t_kern
        rec["kernel_mfma_frac"] = t_mfma / t_kern
        rec["kernel_roofline_frac"] = max(tk_hbm, t_mfma) / t_kern
    rec["kernel"] = kernel_name(M, N, K, path)
    # impossible-throughput flag: faster than the card can move the bytes or
    # do the operations ("V100TPS engine log", opening section)
    rec["impossible"] = bool(rec["hbm_frac"] > 1.0 or rec["mfma_frac"] > 1.0 or
                             rec.get("kernel_hbm_frac", 0) > 1.0 or rec.get("kernel_mfma_frac", 0) > 1.0)
    return rec


def measure_group(ms=(1, 8, 16), reps=20):
    """One X against two weight matrices of the decode shape (N=10240,
    K=5120; e.g. two input projections of one layer): one grouped call (one
    quantization, one matmul launch over both) against two iq4xs_gemm calls,
    both with caller workspaces.  ms per pair on the device: `reps` pairs
    (each on another rotated weight pair, past the Infinity Cache) recorded
    in one HIP graph and replayed, as for the per-call times."""
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


def probes(reps=10):
    """This device's own ceilings, from the library's measurement kernels:
    stream reads of 28 MB (one decode-shape weight matrix), 95 MB and 1 GiB,
    each buffer rotated with others so that >= 768 MB lie between two reads
    of it (the Infinity Cache holds 256 MB); a 1 GiB stream write; and
    back-to-back int8 and bf16 MFMA instructions on every SIMD.  Reads and
    writes are replayed from a HIP graph, as the matmul calls are."""
    stream = torch.cuda.current_stream()
    sink = torch.empty(65536, dtype=torch.int32, device="cuda")
    out = {"read": [], "write": None, "mfma": {}}
    for nbytes in (27_852_800, 95_027_200, 1 << 30):
        n = max(2, math.ceil((1 << 30) * 0.75 / nbytes) + 1)
        bufs = [torch.full((nbytes,), i, dtype=torch.uint8, device="cuda") for i in range(n)]
        k = [0]

        def rd():
            iq.probe_read(bufs[k[0] % n], sink, grid=4096)
            k[0] += 1
        for _ in range(n):
            rd()
        t = time_graph(rd, reps * n if nbytes < (1 << 30) else reps, stream)
        out["read"].append({"bytes": nbytes, "ms": t, "GBs": nbytes / (t * 1e-3) / 1e9,
                            "frac_of_8TBs": nbytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, "buffers": n})
        del bufs
    buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    iq.probe_write(buf)
    t = time_graph(lambda: iq.probe_write(buf), reps, stream)
    out["write"] = {"bytes": 1 << 30, "ms": t, "GBs": (1 << 30) / (t * 1e-3) / 1e9}
    del buf
    torch.cuda.empty_cache()
    grid, iters = 2048, 2000
    res = torch.empty(grid * 256, dtype=torch.int32, device="cuda")
    resf = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    for kind, name, flops, peak, o in ((iq.PROBE_MFMA_I8, "int8", 65536, INT8_PEAK_TOPS, res),
                                       (iq.PROBE_MFMA_BF16, "bf16", 32768, BF16_PEAK_TFLOPS, resf)):
        iq.probe_mfma(kind, 10, o, grid)
        t = time_events(lambda: iq.probe_mfma(kind, iters, o, grid), 3, stream)
        rate = grid * 4 * 4 * iters * flops / (t * 1e-3) / 1e12
        out["mfma"][name] = {"T_per_s": rate, "published_peak": peak, "frac": rate / peak,
                             "instructions_per_wave": 4 * iters, "waves": grid * 4}
    # matrix-core and vector-ALU work on the same SIMDs (one workgroup of
    # eight wavefronts per compute unit; 2 MFMAs and 96 FMAs per iteration)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    mixo = torch.empty(cus * 512, dtype=torch.int32, device="cuda")
    t = {}
    for mode, name in ((iq.PROBE_MIX_MFMA, "mfma"), (iq.PROBE_MIX_VALU, "valu"), (iq.PROBE_MIX_SAME, "same"),
                       (iq.PROBE_MIX_SPLIT, "split")):
        iq.probe_mix(mode, 10, mixo, cus)
        t[name] = time_events(lambda: iq.probe_mix(mode, 1000, mixo, cus), 3, stream)
    out["mfma_beside_valu"] = {
        "ms": t, "iterations": 1000, "per_iteration": "2 v_mfma_i32_32x32x32_i8 + 96 v_fma_f32",
        # 1.0: the two kinds of work add up; 0.5 (same) would be full overlap
        "same_over_sum": t["same"] / (t["mfma"] + t["valu"]),
        # each SIMD gets half of 'same': 1.0 = adds up, max/sum = full overlap
        "split_over_half_sum": t["split"] / (0.5 * (t["mfma"] + t["valu"]))}
    return out


def cpu_baseline(points, target_s=12.0):
    """The oracle (as it stands, all host threads) on a column sample of the
    same 52 calls (quantization included), in weight-GB/s of the sample.  The
    sample is the same fraction of every point's output columns, sized so the
    pass takes about target_s."""
    import oracle
    o = oracle.get()
    cache = {}

    def run(frac):
        t = 0.0
        wbytes = 0.0
        for wl, N, K, M in points:
            ncols = max(1, int(round(frac * N)))
            key = (wl.cid, N, K)
            if key not in cache:
                cache.clear()
                cache[key] = wl.w(N, K)
            W = np.ascontiguousarray(cache[key][:ncols])
            X = wl.x(M, K, N=N)
            t0 = time.perf_counter()
            o.gemm_q8_1(W, o.quantize_q8_1(X), K)
            t += time.perf_counter() - t0
            wbytes += 0.53125 * ncols * K
        return t, wbytes

    # grow the sample until one pass takes at least a quarter of target_s,
    # then size it to target_s (each pass has a fixed cost per call)
    frac = 2e-4
    t, _ = run(frac)
    while t < target_s / 4 and frac < 1.0:
        frac = min(1.0, frac * 4)
        t, _ = run(frac)
    frac = min(1.0, frac * target_s / max(t, 1e-3))
    t, wbytes = run(frac)
    return {"value": wbytes / t / 1e9, "unit": "weight-GB/s", "cores": o.threads(), "kind": "oracle",
            "sample": f"{frac * 100:.3f}% of the output columns of each of the {len(points)} calls "
                      f"(at least one), quantize included, {t:.1f} s"}


def dominant_rooflines(recs):
    """Per matmul kernel, the point where it takes the most time: its
    algorithmic work per launch over the kernel's average duration against
    the roofline that binds at that point (HBM below M ~ 166, int8 MFMA
    above); the headline entry is the kernel with the largest share of the
    step's kernel time."""
    by_kernel = {}
    for r in recs:
        if r.get("kernel_ms") is None:
            continue
        by_kernel.setdefault(r["kernel"], []).append(r)
    out = []
    for k, rs in by_kernel.items():
        r = max(rs, key=lambda r: r["kernel_ms"])
        M, N, K = r["M"], r["N"], r["K"]
        if r["kernel_hbm_frac"] >= r["kernel_mfma_frac"]:
            ent = {"bound": "hbm", "achieved": algo_bytes_kernel(M, N, K) / (r["kernel_ms"] * 1e-3) / 1e9,
                   "peak": HBM_PEAK_GBS, "unit": "GB/s", "work_per_launch": algo_bytes_kernel(M, N, K),
                   "work_unit": "bytes (0.53125 per weight + 1.125 per activation + 4 per output)"}
        else:
            ent = {"bound": "mfma", "achieved": 2.0 * M * N * K / (r["kernel_ms"] * 1e-3) / 1e12,
                   "peak": INT8_PEAK_TOPS, "unit": "TFLOP/s", "op": "int8 multiply-add = 2 ops",
                   "work_per_launch": 2.0 * M * N * K, "work_unit": "int8 ops (2*M*N*K)",
                   "valu_ceiling_frac": VALU_CEILING_FRAC}
        ent["frac"] = ent["achieved"] / ent["peak"]
        ent.update({"kernel": k, "M": M, "N": N, "K": K, "avg_launch_ms": r["kernel_ms"],
                    "share_of_kernel_time": sum(x["kernel_ms"] for x in rs) /
                    sum(x["kernel_ms"] for x in recs if x.get("kernel_ms") is not None)})
        ent["traffic_bytes_per_launch"] = traffic_for(k, M, N, K)
        ent["traffic"] = (None if ent["traffic_bytes_per_launch"] is None else
                          ent["traffic_bytes_per_launch"] / (r["kernel_ms"] * 1e-3) / 1e9)
        out.append(ent)
    out.sort(key=lambda e: -e["share_of_kernel_time"])
    return out


def fused_points(recs, reps=10):
    """The fused bf16 paths at every prefill point, per call (quantization
    included, graph replay) beside the point's own path: BF16X3 (compensated,
    within the per-row bound; three bf16 products per term, 6*M*N*K flops)
    and DEQ_BF16 (the plain bf16 formulation, one product, 2*M*N*K flops),
    against the bf16 MFMA peak."""
    by = {(r["N"], r["K"], r["M"]): r for r in recs}
    out = []
    for (N, K) in synth.PREFILL.shapes:
        rot = Rotation(synth.PREFILL.w(N, K))
        for M in synth.PREFILL.ms:
            X = torch.from_numpy(synth.PREFILL.x(M, K, N=N)).cuda()
            t_call, _, _ = measure_point(rot, X, N, K, iq.PATH_BF16X3, reps=reps)
            t_plain, _, _ = measure_point(rot, X, N, K, iq.PATH_DEQ_BF16, reps=reps)
            flops = 6.0 * M * N * K
            ent = {"N": N, "K": K, "M": M, "ms": t_call, "bf16_TFLOPs": flops / (t_call * 1e-3) / 1e12,
                   "bf16_frac": flops / (t_call * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                   "int8_equiv_TOPS": 2.0 * M * N * K / (t_call * 1e-3) / 1e12,
                   "deq_bf16_ms": t_plain,
                   "deq_bf16_TFLOPs": 2.0 * M * N * K / (t_plain * 1e-3) / 1e12}
            if (N, K, M) in by:
                ent["auto_ms"] = by[(N, K, M)]["ms"]
                ent["auto_path"] = by[(N, K, M)]["path"]
                ent["speedup_vs_auto"] = by[(N, K, M)]["ms"] / t_call
            out.append(ent)
        del rot
        torch.cuda.empty_cache()
    return out


def format_points(reps=20):
    """A few points with IQ4_NL and Q4_0 weights (iq4xs_gemm_fmt, AUTO)."""
    out = []
    for fmt, name in ((iq.FMT_IQ4_NL, "IQ4_NL"), (iq.FMT_Q4_0, "Q4_0")):
        for wl, M in ((synth.DECODE_ATTN, 1), (synth.DECODE_ATTN, 16), (synth.MLP_UP, 64), (synth.MLP_DOWN, 96)):
            N, K = wl.shapes[0]
            rot = Rotation(synth.weights18((wl.cid, N, K, 0), N, K))
            X = torch.from_numpy(wl.x(M, K, N=N)).cuda()
            t_call, _, _ = measure_point(rot, X, N, K, iq.PATH_AUTO, reps=reps, fmt=fmt)
            wb = 0.5625 * N * K
            out.append({"format": name, "N": N, "K": K, "M": M, "ms": t_call,
                        "weight_GBs": wb / (t_call * 1e-3) / 1e9,
                        "hbm_frac": (wb + 6.25 * M * K + 4 * M * N) / (t_call * 1e-3) / 1e9 / HBM_PEAK_GBS,
                        "int8_TOPS": 2.0 * M * N * K / (t_call * 1e-3) / 1e12})
            del rot
            torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------- profiling
def _marker(i, buf):
    """A tiny write-probe launch whose position in a kernel trace separates
    the dispatches of consecutive points."""
    iq.probe_write(buf, value=i, grid=1)


def profile_points():
    """For --check-trace under rocprofv3 --kernel-trace: every point's full
    iq4xs_gemm call (AUTO) twice, a marker launch before each point."""
    marker = torch.empty(256, dtype=torch.uint8, device="cuda")
    plan = []
    cur = None
    for i, (wl, N, K, M) in enumerate(sweep_points()):
        if cur != (wl.cid, N, K):
            W = torch.from_numpy(wl.w(N, K)).cuda()
            cur = (wl.cid, N, K)
        X = torch.from_numpy(wl.x(M, K, N=N)).cuda()
        Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        _marker(i, marker)
        for _ in range(2):
            iq.gemm(W, X, out=Y)
        torch.cuda.synchronize()
        path = iq.dispatch(M, N, K)
        plan.append({"point": i, "M": M, "N": N, "K": K, "path": iq.path_name(path),
                     "kernel": kernel_name(M, N, K, path), "calls": 2})
        print(f"[profile-points] {i} M={M} N={N} K={K} {iq.path_name(path)}", flush=True)
    _marker(len(plan), marker)
    torch.cuda.synchronize()
    return plan


def check_trace(trace_dir, out, cmd):
    """Between consecutive marker launches of a --profile-points trace: the
    kernels each call launched.  Every call must launch the quantizer and a
    matmul kernel of its path, and the matmul kernel must be the one
    kernel_name() (which the roofline entries use) names."""
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {trace_dir}")
    rows = sorted(csv.DictReader(open(files[0])), key=lambda r: int(r["Start_Timestamp"]))

    def short(n):
        # "ns::(anonymous namespace)::k_name<...>(args)" -> "k_name"
        n = n.replace("void ", "").replace("(anonymous namespace)", "anon")
        return n.split("(")[0].split("<")[0].split("::")[-1].strip()
    groups, cur = [], None
    for r in rows:
        k = short(r["Kernel_Name"])
        if k == "k_probe_write":
            if cur is not None:
                groups.append(cur)
            cur = []
        elif cur is not None:
            cur.append((k, (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3))
    pts = sweep_points()
    families = {"GEMV": {"k_gemv"}, "MMQ": {"k_mmv", "k_mmqt", "k_mmq"}, "DEQ_BF16": {"k_gemm_deq"},
                "BF16X3": {"k_gemm_x3"}}
    lines = ["# kernels launched per call, from a rocprofv3 kernel trace of bench.py --profile-points",
             f"# command: {cmd}",
             "# every call of every point launches the quantizer and a matmul kernel of the path the",
             "# dispatcher names, and that kernel is the one the benchmark's roofline entries attribute",
             "# point  M  N  K  path  expected  launched (per call)  matmul-us (mean)  ok"]
    bad = 0
    if len(groups) != len(pts):
        raise SystemExit(f"{len(groups)} marker groups, {len(pts)} points")
    for i, ((wl, N, K, M), g) in enumerate(zip(pts, groups)):
        names = [k for k, _ in g]
        path = iq.path_name(iq.dispatch(M, N, K))
        expect = kernel_name(M, N, K, iq.PATHS[path])
        per_call = names[:len(names) // 2]
        mat = [k for k in per_call if k.startswith(("k_gemv", "k_mmv", "k_mmqt", "k_mmq", "k_gemm_x3", "k_gemm_deq"))]
        ok = (len(names) % 2 == 0 and names[:len(names) // 2] == names[len(names) // 2:] and
              per_call[0] == "k_quantize" and mat and mat[0] == expect and mat[0] in families[path])
        bad += not ok
        mus = [d for k, d in g if k == expect]
        lines.append(f"{i:3d} {M:4d} {N:6d} {K:6d}  {path:8s} {expect:7s} {'+'.join(per_call):40s} "
                     f"{sum(mus) / max(len(mus), 1):9.2f}  {'ok' if ok else 'MISMATCH'}")
    lines.append(f"# {len(pts) - bad} of {len(pts)} points ok")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    if bad:
        raise SystemExit(f"{bad} points launched other kernels than expected")


def _probe_pair():
    """The calibration read and write of known bytes (PROBE_BYTES each),
    four times, the read buffer evicted from the Infinity Cache in between by
    writes to three others."""
    bufs = [torch.empty(PROBE_BYTES, dtype=torch.uint8, device="cuda") for _ in range(4)]
    sink = torch.empty(65536, dtype=torch.int32, device="cuda")
    for i in range(4):
        for j in range(1, 4):
            iq.probe_write(bufs[(i + j) % 4], value=j)
        torch.cuda.synchronize()
        iq.probe_read(bufs[i], sink)
        torch.cuda.synchronize()
    print(f"[profile] read and write probes of {PROBE_BYTES} bytes", flush=True)
    del bufs
    torch.cuda.empty_cache()


def profile_run():
    """Fixed launches for rocprofv3: per M of the decode sweep, PROFILE_WARM
    then PROFILE_RUNS launches of the matmul kernel alone (rotated weights, as
    in the timed step), then the calibration probes."""
    wl = synth.DECODE_ATTN
    (N, K), ms = wl.shapes[0], wl.ms
    rot = Rotation(wl.w(N, K))
    for M in ms:
        X = torch.from_numpy(wl.x(M, K, N=N)).cuda()
        act = iq.prepare_act(X)
        Y = torch.zeros((M, N), dtype=torch.float32, device="cuda")
        path = iq.dispatch(M, N, K)
        for _ in range(PROFILE_GROUP):
            iq.gemm_act(rot.next(), act, M, K, path=path, out=Y, y_zeroed=True)
        torch.cuda.synchronize()
        print(f"[profile-run] M={M} {kernel_name(M, N, K, path)} x{PROFILE_GROUP}", flush=True)
    del rot
    torch.cuda.empty_cache()
    _probe_pair()


def profile_shapes(specs):
    """Fixed launches for rocprofv3 at given shapes ("MxNxK", comma
    separated): per shape, PROFILE_WARM then PROFILE_RUNS launches of the matmul kernel(s) alone
    (gemm_act, rotated weights), inputs of the workload the shape belongs to
    (else the prefill recipe); then the calibration probes.  "MxNxK:PATH"
    forces a path and launches whole calls (for the paths gemm_act does not
    take: their quantize kernel shows in the trace beside the matmul)."""
    for spec in specs.split(","):
        shape, _, pname = spec.partition(":")
        M, N, K = (int(v) for v in shape.split("x"))
        wl = next((w for w in synth.WORKLOADS if (N, K) in w.shapes), synth.WORKLOADS[-1])
        rot = Rotation(wl.w(N, K))
        X = torch.from_numpy(wl.x(M, K, N=N)).cuda()
        Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        if pname:
            path = iq.PATHS[pname]
            ws = torch.empty(iq.workspace_bytes(M, N, K, path), dtype=torch.uint8, device="cuda")
            for _ in range(PROFILE_GROUP):
                iq.gemm(rot.next(), X, path=path, out=Y, workspace=ws)
        else:
            act = iq.prepare_act(X)
            path = iq.dispatch(M, N, K)
            for _ in range(PROFILE_GROUP):
                iq.gemm_act(rot.next(), act, M, K, path=path, out=Y)
        torch.cuda.synchronize()
        print(f"[profile-shapes] M={M} N={N} K={K} {kernel_name(M, N, K, path)} x{PROFILE_GROUP}", flush=True)
        del rot
        torch.cuda.empty_cache()
    _probe_pair()


def _counter_rows(d):
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {d}")
    return rows


def _probe_scales(fetch_rows, write_rows):
    """true bytes per counted byte: FETCH_SIZE of the read probe and
    WRITE_SIZE of the write probe over their known sizes (the probes of
    PROBE_BYTES; the small marker writes are ignored)."""
    def per(rows, counter, kname):
        acc = {}
        for r in rows:
            if r["Counter_Name"] == counter and kname in r["Kernel_Name"]:
                acc[r["Dispatch_Id"]] = acc.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        return [v for v in acc.values() if v * 1024.0 > PROBE_BYTES / 16]
    f = per(fetch_rows, "FETCH_SIZE", "k_probe_read")
    w = per(write_rows, "WRITE_SIZE", "k_probe_write")
    if not f or not w:
        raise SystemExit("calibration probes not found in the counter runs")
    fk, wk = sum(f) / len(f), sum(w) / len(w)
    return fk, wk, PROBE_BYTES / (fk * 1024.0), PROBE_BYTES / (wk * 1024.0)


def summarize_pmc(fetch_dir, write_dir, out, cmd_fetch, cmd_write):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the decode sweep's matmul
    kernels, calibrated by the read and write probes -> HBM bytes per launch."""
    fr, wr = _counter_rows(fetch_dir), _counter_rows(write_dir)

    def per_kernel(rows, counter):
        acc = {}
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            key = ("k_mmv" if "k_mmv" in name else "k_gemv" if "k_gemv" in name else None)
            if key is None:
                continue
            label = name.split("Cfg<")[1].split(">")[0].replace(" ", "") if "Cfg<" in name else ""
            acc.setdefault((key, label), {}).setdefault(int(r["Dispatch_Id"]), 0.0)
            acc[(key, label)][int(r["Dispatch_Id"])] += float(r["Counter_Value"])
        out = {}
        for k, v in acc.items():
            vals = _measured([v[i] for i in sorted(v)])
            out[k] = sum(vals) / len(vals)
        return out
    fk, wk, f_scale, w_scale = _probe_scales(fr, wr)
    fetch, write = per_kernel(fr, "FETCH_SIZE"), per_kernel(wr, "WRITE_SIZE")
    wl = synth.DECODE_ATTN
    (N, K), ms = wl.shapes[0], wl.ms
    lines = [f"# HBM traffic per launch from rocprofv3 counters, decode sweep N={N} K={K}",
             f"# fetch run: {cmd_fetch}", f"# write run: {cmd_write}",
             f"# calibration: a read of {PROBE_BYTES} bytes (probe_read, plain 16-byte loads) and a write of",
             f"# {PROBE_BYTES} bytes (probe_write, plain 16-byte stores), each buffer evicted from the Infinity Cache",
             f"probe_bytes {PROBE_BYTES}",
             f"probe_fetch_kib {fk:.1f}  fetch_scale {f_scale:.4f}",
             f"probe_write_kib {wk:.1f}  write_scale {w_scale:.4f}",
             f"source_hash k_mmv {source_hash('k_mmv')}",
             f"source_hash k_gemv {source_hash('k_gemv')}",
             "# kernel config  fetch_kib  write_kib  calibrated_bytes"]
    for (k, label), f in sorted(fetch.items()):
        w = write.get((k, label), 0.0)
        lines.append(f"traffic {k} <{label}> {f:.1f} {w:.1f} {f * 1024.0 * f_scale + w * 1024.0 * w_scale:.0f}")
    for M in ms:
        lines.append(f"algorithmic M={M} {algo_bytes_kernel(M, N, K):.0f}")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_fused(trace_dir, fetch_dir, write_dir, out, cmds, spec):
    """One shape of a --profile-shapes run with a fused bf16 path forced
    ("MxNxK:BF16X3" or "MxNxK:DEQ_BF16"): the fused kernel's and the
    quantizer's durations from the kernel trace, the fused kernel's HBM bytes
    per launch from the counter runs (calibrated by their probes), its
    algorithmic bytes and its bf16 rate at the trace's average duration
    (BF16X3: three products per term, 6*M*N*K flops, both activation planes
    read; DEQ_BF16: one product, 2*M*N*K, the hi plane)."""
    shape, _, pname = spec.partition(":")
    M, N, K = (int(v) for v in shape.split("x"))
    x3 = pname != "DEQ_BF16"
    kern = "k_gemm_x3" if x3 else "k_gemm_deq"
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {trace_dir}")
    durs = {}
    for r in csv.DictReader(open(files[0])):
        for k in (kern, "k_quantize"):
            if k in r["Kernel_Name"]:
                durs.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
    fr, wr = _counter_rows(fetch_dir), _counter_rows(write_dir)
    fk, wk, f_scale, w_scale = _probe_scales(fr, wr)

    def per_launch(rows, counter):
        acc = {}
        for r in rows:
            if r["Counter_Name"] == counter and kern in r["Kernel_Name"]:
                i = int(r["Dispatch_Id"])
                acc[i] = acc.get(i, 0.0) + float(r["Counter_Value"])
        vals = _measured([acc[i] for i in sorted(acc)])
        return sum(vals) / len(vals) if vals else float("nan")
    f_kib, w_kib = per_launch(fr, "FETCH_SIZE"), per_launch(wr, "WRITE_SIZE")
    traffic = f_kib * 1024.0 * f_scale + w_kib * 1024.0 * w_scale
    ms_rows = -(-M // 256) * 256
    act = 4.0 if x3 else 2.0
    algo = 0.53125 * N * K + act * ms_rows * K + 4.0 * M * N
    flops = (6.0 if x3 else 2.0) * M * N * K
    durs = {k: _measured(v) for k, v in durs.items()}
    d = durs.get(kern, [float("nan")])
    avg = sum(d) / len(d)
    title = "compensated-bf16 kernel (BF16X3 path)" if x3 else "plain bf16 kernel (DEQ_BF16 path)"
    lines = [f"# fused {title}, M={M} N={N} K={K}: kernel trace and HBM counters ({PROFILE_RUNS} whole calls "
             f"after {PROFILE_WARM} of warm-up, rotated weights)",
             *[f"# command: {c}" for c in cmds],
             f"source_hash {kern} {source_hash(kern)}",
             f"# calibration by the runs' own probes ({PROBE_BYTES} bytes read / written): fetch x{f_scale:.4f}, "
             f"write x{w_scale:.4f}",
             "# kernel  calls  avg_us  min_us  max_us"]
    for k, v in sorted(durs.items()):
        lines.append(f"{k} {len(v)} {sum(v) / len(v):.2f} {min(v):.2f} {max(v):.2f}")
    lines += [f"{kern} fetch_kib {f_kib:.1f} write_kib {w_kib:.1f} traffic_bytes_per_launch {traffic:.0f}",
              f"{kern} algorithmic_bytes_per_launch {algo:.0f} (weights 0.53125/weight, activation planes "
              f"{act:.0f} B per element of the padded rows, Y)",
              f"{kern} traffic/algorithmic {traffic / algo:.2f}",
              f"{kern} bf16 TFLOP/s at avg {flops / (avg * 1e-6) / 1e12:.0f} "
              f"({flops / (avg * 1e-6) / 1e12 / BF16_PEAK_TFLOPS * 100:.1f}% of 2.5 PFLOP/s)"]
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_pmc_shapes(fetch_dir, write_dir, out, cmd_fetch, cmd_write, specs):
    """Per shape of a --profile-shapes run (PROFILE_GROUP launches each, in
    order, the first PROFILE_WARM left out): mean
    FETCH_SIZE / WRITE_SIZE per launch of the tile kernel and of its
    shared-tile kernel, calibrated by the probes of the same runs, against
    the algorithmic bytes."""
    fr, wr = _counter_rows(fetch_dir), _counter_rows(write_dir)
    fk, wk, f_scale, w_scale = _probe_scales(fr, wr)

    def per_dispatch(rows, counter):
        acc = {}
        for r in rows:
            if r["Counter_Name"] == counter and "k_mmqt" in r["Kernel_Name"]:
                k = (int(r["Dispatch_Id"]), "fix" if "k_mmqt_fix" in r["Kernel_Name"] else "main")
                acc[k] = acc.get(k, 0.0) + float(r["Counter_Value"])
        return acc
    fd, wd = per_dispatch(fr, "FETCH_SIZE"), per_dispatch(wr, "WRITE_SIZE")
    shapes = [tuple(int(v) for v in sp.split("x")) for sp in specs.split(",")]
    lines = [f"# HBM traffic per launch of the tile kernel from rocprofv3 counters ({PROFILE_RUNS} launches per "
             f"shape after {PROFILE_WARM} of warm-up)",
             f"# fetch run: {cmd_fetch}", f"# write run: {cmd_write}",
             f"# calibration by the runs' own probes ({PROBE_BYTES} bytes read / written): "
             f"fetch x{f_scale:.4f} ({fk:.1f} KiB counted), write x{w_scale:.4f} ({wk:.1f} KiB counted)",
             f"source_hash k_mmqt {source_hash('k_mmqt')}",
             "# M N K  kernel  fetch_MB  write_MB  calibrated_MB  algorithmic_MB (W + planes + Y)"]
    sums = {}
    n_main = -1
    for (i, part) in sorted(set(fd) | set(wd)):
        if part == "main":
            n_main += 1
        shape = n_main // PROFILE_GROUP
        if n_main % PROFILE_GROUP < PROFILE_WARM:
            continue
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


def traffic_for(kernel, M, N, K):
    """Calibrated HBM bytes per launch of `kernel` at (M, N, K) from the
    committed counter summaries, or None when there is none for that point or
    the kernel's source changed since it was measured."""
    if kernel in ("k_mmv", "k_gemv") and os.path.exists(TRAFFIC_FILE) and (N, K) == (10240, 5120):
        lines = open(TRAFFIC_FILE).read().splitlines()
        if f"source_hash {kernel} {source_hash(kernel)}" not in lines:
            return None
        labels = {1: "1,4,8,3,false,0", 2: "1,4,8,3,true,0", 4: "2,4,8,3,true,0", 8: "4,8,4,3,false,0",
                  16: "8,16,4,3,false,0"}
        want = f"<{labels.get(M, '')}>" if kernel == "k_mmv" else "<>"
        for ln in lines:
            p = ln.split()
            if len(p) == 6 and p[0] == "traffic" and p[1] == kernel and p[2] == want:
                return float(p[5])
        return None
    if kernel == "k_mmqt" and os.path.exists(TILE_TRAFFIC_FILE):
        lines = open(TILE_TRAFFIC_FILE).read().splitlines()
        if f"source_hash k_mmqt {source_hash('k_mmqt')}" not in lines:
            return None
        total = 0.0
        found = False
        for ln in lines:
            p = ln.split()
            if len(p) == 8 and p[:3] == [str(M), str(N), str(K)]:
                total += float(p[6]) * 1e6
                found = True
        return total if found else None
    return None


SQ_PASSES = (("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU",
              "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES"),
             ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_LDS_BANK_CONFLICT",
              "SQ_WAIT_INST_LDS", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_ANY"))


def _sq_key(name, order, shapes):
    """Kernel label; the tile kernel's launches of a --profile-shapes run
    (PROFILE_GROUP per shape, in order) also carry their shape."""
    key = name.replace("void ", "").replace("iq4xs::(anonymous namespace)::", "").split("(")[0]
    if shapes and "k_mmqt<" in key and order is not None:
        i = order // PROFILE_GROUP
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
    SIMDs) take; and the same two shares at the clock the run implies
    (SQ_BUSY_CYCLES counted once per shader engine, 32 of them), with their
    sum: near 1 when VALU and matrix-core issue do not overlap."""
    shapes = [tuple(int(v) for v in sp.split(":")[0].split("x")) for sp in specs.split(",")] if specs else []
    per = {}
    for d in dirs:
        rows = _counter_rows(d)
        order = _tile_order(rows, "Dispatch_Id")
        for r in rows:
            name = r["Kernel_Name"]
            if not any(k in name for k in ("k_mmv", "k_gemv", "k_mmqt", "k_mmq", "k_quantize", "k_gemm_x3",
                                           "k_gemm_deq")):
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
            dur.setdefault(key, []).append((int(r["Start_Timestamp"]), (int(r["End_Timestamp"]) -
                                                                          int(r["Start_Timestamp"])) * 1e-3))
    dur = {k: _measured([d for _, d in sorted(v)]) for k, v in dur.items()}
    lines = ["# SQ counters per dispatch (averages), matmul and quantize kernels of the decode sweep and the tile shapes",
             *[f"# run: {c}" for c in cmds],
             "# VALU/MFMA: instructions; LDS-conflict: bank-conflict cycles per LDS instruction; VALU-issue and "
             "MFMA-busy: per SIMD, as a share of the kernel's average duration in the trace",
             "# kernel | " + " ".join(c for p_ in SQ_PASSES for c in p_) +
             " | VALU/MFMA  LDS-conflict  trace-us  VALU-issue  MFMA-busy | clock-GHz  VALU-issue  MFMA-busy  sum"]
    for key in sorted(per):
        v = {}
        for c, d in per[key].items():
            vals = _measured([d[i] for i in sorted(d, key=int)])
            v[c] = sum(vals) / len(vals)
        vals = " ".join(f"{v.get(c, float('nan')):.4g}" for p_ in SQ_PASSES for c in p_)
        valu, mfma = v.get("SQ_INSTS_VALU", 0.0), v.get("SQ_INSTS_MFMA", 0.0)
        lds, conf = v.get("SQ_INSTS_LDS", 0.0), v.get("SQ_LDS_BANK_CONFLICT", 0.0)
        d_us = sum(dur[key]) / len(dur[key]) if key in dur else float("nan")
        issue = valu * 4 / 1024 / 2.4e3 / d_us
        busy = v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / 1024 / 2.4e3 / d_us
        clk = v.get("SQ_BUSY_CYCLES", float("nan")) / 32 / d_us / 1e3      # GHz
        issue_c, busy_c = issue * 2.4 / clk, busy * 2.4 / clk
        lines.append(f"{key} | {vals} | {valu / mfma if mfma else float('nan'):.2f}  "
                     f"{conf / lds if lds else float('nan'):.3f}  {d_us:.2f}  {issue:.2f}  {busy:.2f} | "
                     f"{clk:.2f}  {issue_c:.2f}  {busy_c:.2f}  {issue_c + busy_c:.2f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")




def summarize_trace(trace_dir, out, cmd, title):
    """The kernel trace of a rocprofv3 run as a short text table (kernel,
    calls, average / min / max microseconds, share of GPU time), the
    warm-up launches of each matmul kernel left out."""
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {trace_dir}")
    with open(files[0]) as fh:
        rows = sorted(csv.DictReader(fh), key=lambda r: int(r["Start_Timestamp"]))

    def short(name):
        name = name.replace("void ", "").replace("iq4xs::(anonymous namespace)::", "").replace("iq4xs::", "")
        return name.replace("(anonymous namespace)::", "").split("(")[0]
    per = {}
    for r in rows:
        per.setdefault(short(r["Kernel_Name"]), []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
    per = {k: (_measured(v) if k.startswith(("k_mmv", "k_gemv", "k_mmqt", "k_mmq", "k_gemm")) else v)
           for k, v in per.items()}
    total = sum(sum(v) for v in per.values())
    lines = [f"# rocprofv3 kernel-trace statistics: {title}", f"# command: {cmd}",
             f"# matmul kernels: the last {PROFILE_RUNS} of each {PROFILE_GROUP} launches (warm-up left out)",
             f"{'kernel':60s} {'calls':>6s} {'avg_us':>8s} {'min_us':>8s} {'max_us':>8s} {'pct':>6s}"]
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{k[:60]:60s} {len(v):6d} {sum(v) / len(v):8.2f} {min(v):8.2f} {max(v):8.2f} "
                     f"{100.0 * sum(v) / total:6.2f}")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_trace_shapes(trace_dir, out, cmd, specs):
    """Per shape of a --profile-shapes kernel trace (PROFILE_GROUP launches per
    shape, in order, the first PROFILE_WARM left out): the tile kernel's and
    its summing kernel's durations."""
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {trace_dir}")
    rows = sorted(csv.DictReader(open(files[0])), key=lambda r: int(r["Start_Timestamp"]))
    shapes = [tuple(int(v) for v in sp.split("x")) for sp in specs.split(",")]
    per, n_main = {}, -1
    for r in rows:
        name = r["Kernel_Name"]
        if "k_mmqt" not in name:
            continue
        part = "k_mmqt_fix" if "k_mmqt_fix" in name else "k_mmqt"
        if part == "k_mmqt":
            n_main += 1
        if n_main % PROFILE_GROUP < PROFILE_WARM:
            continue
        per.setdefault((n_main // PROFILE_GROUP, part), []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
    lines = [f"# tile-kernel durations per shape from a rocprofv3 kernel trace ({PROFILE_RUNS} launches per shape "
             f"after {PROFILE_WARM} of warm-up, gemm_act, rotated weights)", f"# command: {cmd}",
             f"source_hash k_mmqt {source_hash('k_mmqt')}",
             "# M N K  kernel  calls  avg_us  min_us  max_us"]
    for (i, part), d in sorted(per.items()):
        if i < len(shapes):
            M, N, K = shapes[i]
            lines.append(f"{M} {N} {K}  {part}  {len(d)}  {sum(d) / len(d):.2f}  {min(d):.2f}  {max(d):.2f}")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def run_sweep(path_out):
    """Every (shape, M, path) point of the five workloads -> JSONL (with the
    device's compute-unit count, which the dispatch table records)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
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
                    if M >= 64:
                        paths.append(iq.PATH_BF16X3)
                    for p in paths:
                        rec = point_record(N, K, M, p, *measure_point(rot, X, N, K, p, reps=20))
                        rec["workload"] = wl.name
                        rec["cus"] = cus
                        if p == iq.PATH_AUTO:
                            rec["auto"] = iq.path_name(iq.dispatch(M, N, K))
                        f.write(json.dumps(rec) + "\n")
                        f.flush()
                        print(f"[sweep] {wl.cid} N={N} K={K} M={M} {rec['path']}: {rec['ms']:.4f} ms "
                              f"{rec['weight_GBs']:.0f} GB/s", flush=True)
                del rot
                torch.cuda.empty_cache()


def summarize_sweep(jsonl, out, cmd):
    """A --sweep JSONL as a compact text table (one line per shape, M and
    path: us per call and us of the matmul kernel alone), the record behind
    the dispatch table; iq4_xs_q8_amd.calibrate reads this table as well."""
    recs = [json.loads(line) for line in open(jsonl)]
    cus = sorted({r.get("cus") for r in recs if r.get("cus")})
    lines = ["# per-call device time of every (shape, M, path) point of the five workloads",
             f"# command: {cmd}", f"# compute units: {','.join(map(str, cus))}",
             "# N K M path us_per_call us_kernel"]
    for r in recs:
        if r["path"] == "AUTO":
            continue
        k = r.get("kernel_ms")
        lines.append(f"{r['N']} {r['K']} {r['M']} {r['path']} {r['ms'] * 1e3:.2f} "
                     f"{'-' if k is None else f'{k * 1e3:.2f}'}")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"{len(lines) - 4} points -> {out}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--sweep", default=None, help="also time every workload point and path -> JSONL")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-run", action="store_true", help="fixed launches for rocprofv3 --pmc")
    ap.add_argument("--profile-shapes", default=None, help="MxNxK,...: fixed launches for rocprofv3")
    ap.add_argument("--profile-points", action="store_true", help="every point's call, markers between")
    ap.add_argument("--check-trace", metavar="TRACE_DIR")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR")
    ap.add_argument("--summarize-pmc-shapes", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "SHAPES"))
    ap.add_argument("--summarize-sq", nargs="+", metavar="DIR", help="SQ counter runs -> instruction mix")
    ap.add_argument("--summarize-sweep", metavar="JSONL")
    ap.add_argument("--summarize-fused", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-trace-shapes", nargs=2, metavar=("TRACE_DIR", "SHAPES"))
    ap.add_argument("--trace-dir", default=None, help="kernel-trace runs of the same launches, comma-separated")
    ap.add_argument("--shapes", default="", help="MxNxK,... of the --profile-shapes runs")
    ap.add_argument("--cmd", default="")
    ap.add_argument("--title", default="")
    ap.add_argument("--out", default=None)
    ap.add_argument("--cmd-fetch", default="")
    ap.add_argument("--cmd-write", default="")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, args.out or TRAFFIC_FILE, args.cmd_fetch, args.cmd_write)
        return
    for flag in ("summarize_pmc_shapes", "summarize_sq", "summarize_trace", "check_trace", "summarize_sweep",
                 "summarize_fused"):
        if getattr(args, flag) and not args.out:
            raise SystemExit(f"--{flag.replace('_', '-')} needs --out")
    if args.summarize_pmc_shapes:
        summarize_pmc_shapes(*args.summarize_pmc_shapes[:2], args.out, args.cmd_fetch, args.cmd_write,
                             args.summarize_pmc_shapes[2])
        return
    if args.summarize_sq:
        summarize_sq(args.summarize_sq, [d for d in (args.trace_dir or "").split(",") if d], args.out,
                     [c for c in args.cmd.split(";;") if c], args.shapes)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.out, args.cmd, args.title)
        return
    if args.summarize_fused:
        summarize_fused(*args.summarize_fused, args.out, [c for c in args.cmd.split(";;") if c], args.shapes)
        return
    if args.summarize_sweep:
        summarize_sweep(args.summarize_sweep, args.out, args.cmd)
        return
    if args.summarize_trace_shapes:
        if not args.out:
            raise SystemExit("--summarize-trace-shapes needs --out")
        summarize_trace_shapes(args.summarize_trace_shapes[0], args.out, args.cmd, args.summarize_trace_shapes[1])
        return
    if args.check_trace:
        check_trace(args.check_trace, args.out, args.cmd)
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
    if args.profile_points:
        profile_points()
        return

    t_setup = time.perf_counter()
    pts = sweep_points()
    rots, calls = {}, []
    for wl, N, K, M in pts:
        if (wl.cid, N, K) not in rots:
            rots[(wl.cid, N, K)] = Rotation(wl.w(N, K))
        X = torch.from_numpy(wl.x(M, K, N=N)).cuda()
        Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        ws = torch.empty(iq.workspace_bytes(M, N, K), dtype=torch.uint8, device="cuda")
        calls.append((rots[(wl.cid, N, K)], X, Y, ws))
    print(f"[bench] {len(pts)} points, {sum(len(r.ws) for r in rots.values())} weight copies, "
          f"setup {time.perf_counter() - t_setup:.1f} s", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()

    # One step = one iq4xs_gemm_ws call per point (quantization + dispatch +
    # matmul), in workload order, on one stream.
    def step():
        for rot, X, Y, ws in calls:
            iq.gemm(rot.next(), X, out=Y, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = ev0.elapsed_time(ev1) / args.steps
    wbytes = sum(0.53125 * N * K for _, N, K, _ in pts)
    ops = sum(2.0 * M * N * K for _, N, K, M in pts)
    value = wbytes / (step_ms * 1e-3) / 1e9
    print(f"[bench] step {step_ms:.3f} ms ({value:.0f} weight-GB/s)", file=sys.stderr, flush=True)

    recs = []
    for (wl, N, K, M), (rot, X, _, _) in zip(pts, calls):
        path = iq.dispatch(M, N, K)
        r = point_record(N, K, M, path, *measure_point(rot, X, N, K, path))
        r["workload"] = wl.name
        recs.append(r)
    del calls
    print("[bench] per-point times done", file=sys.stderr, flush=True)
    rl = dominant_rooflines(recs)
    by = {(r["N"], r["K"], r["M"]): r for r in recs}
    out = {"metric": METRIC, "value": value, "unit": "weight-GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": step_ms,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
           "data": "synthetic (seeded IQ4_XS weights; N(0,1) activations, 1% outlier channels x20 on the "
                   "decode shape, sigma 0.5 on the MLP-down shape)",
           "config": {"workload": "IQ4_XS x Q8_1 GEMM sweep M=1..512: 2048x2048 at M=4; N=10240 K=5120 at "
                                  "M=1,2,4,8,16; N=17408 K=5120 at M=8..96; N=5120 K=17408 at M=1..96; nine "
                                  "prefill shapes up to N=248320 at M=64,128,256,512 (52 calls per step, "
                                  "quantize included)",
                      "points": len(pts), "weight_bytes_per_step": wbytes,
                      "weight_copies": sum(len(r.ws) for r in rots.values())},
           "int8_TOPS": ops / (step_ms * 1e-3) / 1e12, "wall_s": wall,
           "roofline": dict(rl[0]), "rooflines": rl, "points": recs}
    del rots
    torch.cuda.empty_cache()
    if (10240, 5120, 1) in by and (10240, 5120, 2) in by:
        out["t_m2_over_m1"] = by[(10240, 5120, 2)]["ms"] / by[(10240, 5120, 1)]["ms"]
    out["probes"] = probes()
    print("[bench] probes done", file=sys.stderr, flush=True)
    out["group"] = measure_group()
    out["formats"] = format_points()
    print("[bench] group and formats done", file=sys.stderr, flush=True)
    out["fused_bf16x3"] = fused_points(recs)
    print("[bench] fused path points done", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(pts)
    if args.sweep:
        torch.cuda.empty_cache()
        run_sweep(args.sweep)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
