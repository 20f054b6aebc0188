"""Turn a measured sweep into the dispatch table behind IQ4XS_PATH_AUTO.

Usage:  python -m iq4_xs_q8_amd.calibrate SWEEP [OUT.txt]

SWEEP is what `bench.py --sweep` writes on the device (JSONL), or its text
summary (`bench.py --summarize-sweep`, kept under profiles/): one record per
(workload shape, M, path) with the per-call device time `ms` (quantization
included, calls replayed from a HIP graph so that host launch cost is not
counted, weights rotated past the Infinity Cache).  The table ("V100TPS engine log",
mmvq vs dequant+GEMM table: the band boundaries are measured, not
hard-coded) is written as

  * per measured shape, bands of consecutive measured M whose fastest exact
    path (GEMV or MMQ) is the GEMV, each band reaching up to the next
    measured M minus one;
  * per measured shape, a BF16X3 band from the smallest measured M from
    which the fused compensated-bf16 path is faster than GEMV and MMQ at
    every larger measured M (it meets the same per-row bound as they do);
  * per measured shape, a DEQ_BF16 band from the smallest measured M from
    which the bf16 path is fastest at every larger measured M (these bands
    only apply with IQ4XS_ALLOW_BF16=1: the bf16 path is not exact);
  * for unmeasured shapes, GEMV for M <= 4 up to the largest N at which the
    GEMV won every measured M <= 4 point;
  * MMQ for everything else.
The output goes to OUT.txt (default: stdout); the library embeds
csrc/dispatch_gfx950.txt at build time.
"""

from __future__ import annotations

import collections
import json
import sys

BIG = 1000000000


def load(path):
    """(N, K) -> M -> {path: ms}, and the compute-unit count the sweep ran on
    (None when its records do not say).  Reads the JSONL of a sweep run or
    its text summary (bench.py --summarize-sweep: "N K M path us_per_call
    us_kernel" lines and a "# compute units: C" line)."""
    best = collections.defaultdict(dict)
    cus = set()
    for line in open(path):
        line = line.strip()
        if not line:
            continue
        if line.startswith("#"):
            if line.startswith("# compute units:") and line.split(":")[1].strip():
                cus.update(int(c) for c in line.split(":")[1].split(","))
            continue
        if line.startswith("{"):
            r = json.loads(line)
            if "cus" in r:
                cus.add(int(r["cus"]))
            if r["path"] == "AUTO":
                continue
            best[(r["N"], r["K"])].setdefault(r["M"], {})[r["path"]] = r["ms"]
        else:
            N, K, M, p, us = line.split()[:5]
            best[(int(N), int(K))].setdefault(int(M), {})[p] = float(us) * 1e-3
    if len(cus) > 1:
        raise SystemExit(f"sweep mixes devices with {sorted(cus)} compute units")
    return best, (cus.pop() if cus else None)


def table(best, arch="gfx950", cus=None):
    lines = [f"# Dispatch table for IQ4XS_PATH_AUTO on {arch}, written by iq4_xs_q8_amd/calibrate.py",
             "# from a bench.py --sweep run (per-call device ms from graph replays, quantization included).",
             "# band <path> <M_lo> <M_hi> <N> <K>; first match wins.", f"arch {arch}"]
    if cus is not None:
        lines.append(f"cus {cus}")
    gemv_ok_n = []                           # shapes where the GEMV won every measured M <= 4
    gemv_lost_n = []
    for (N, K), pts in sorted(best.items()):
        ms = sorted(pts)
        exact = {m: min((t, p) for p, t in pts[m].items() if p in ("GEMV", "MMQ"))[1] for m in ms}
        small = [m for m in ms if m <= 4 and "GEMV" in pts[m]]
        if small:
            (gemv_ok_n if all(exact[m] == "GEMV" for m in small) else gemv_lost_n).append(N)
        i = 0
        while i < len(ms):
            if exact[ms[i]] != "GEMV":
                i += 1
                continue
            j = i
            while j + 1 < len(ms) and exact[ms[j + 1]] == "GEMV":
                j += 1
            hi = min(4, ms[j + 1] - 1) if j + 1 < len(ms) else 4
            detail = ", ".join(f"M={m}: GEMV {pts[m]['GEMV'] * 1e3:.1f} us vs MMQ {pts[m]['MMQ'] * 1e3:.1f} us"
                               for m in ms[i:j + 1])
            lines.append(f"# {N}x{K}: {detail}")
            lines.append(f"band GEMV {ms[i]} {hi} {N} {K}")
            i = j + 1
        # the fused path from the smallest M after which it beats the others
        # that meet the bound
        lo = None
        for m in reversed(ms):
            cand = {p: t for p, t in pts[m].items() if p in ("GEMV", "MMQ", "BF16X3")}
            if "BF16X3" in cand and min(cand, key=cand.get) == "BF16X3":
                lo = m
            else:
                break
        if lo is not None:
            lines.append(f"# {N}x{K}: BF16X3 fastest exact-bound path from M={lo} "
                         f"({pts[lo]['BF16X3'] * 1e3:.1f} us vs MMQ {pts[lo]['MMQ'] * 1e3:.1f} us)")
            lines.append(f"band BF16X3 {lo} {BIG} {N} {K}")
        # bf16 from the smallest M after which it always wins
        lo = None
        for m in reversed(ms):
            if "DEQ_BF16" in pts[m] and min(pts[m], key=pts[m].get) == "DEQ_BF16":
                lo = m
            else:
                break
        if lo is not None:
            lines.append(f"# {N}x{K}: DEQ_BF16 fastest from M={lo} "
                         f"({pts[lo]['DEQ_BF16'] * 1e3:.1f} us vs MMQ {pts[lo]['MMQ'] * 1e3:.1f} us)")
            lines.append(f"band DEQ_BF16 {lo} {BIG} {N} {K}")
    if gemv_ok_n:
        n_hi = max(gemv_ok_n)
        if gemv_lost_n and min(gemv_lost_n) <= n_hi:
            n_hi = min(gemv_lost_n) - 1
        lines.append(f"# other shapes: GEMV at M <= 4 up to N={n_hi} (largest N where it won every measured M <= 4)")
        lines.append(f"band GEMV 1 4 1-{n_hi} *")
    elif gemv_lost_n:
        lines.append("# GEMV measured at M <= 4 for N in {" + ", ".join(map(str, sorted(set(gemv_lost_n))))
                     + "}: the streaming MMQ kernel was faster at every point")
    lines.append("band MMQ 1 1000000000 * *")
    return "\n".join(lines) + "\n"


def main(argv=None):
    argv = sys.argv[1:] if argv is None else argv
    if not argv:
        print(__doc__)
        sys.exit(2)
    best, cus = load(argv[0])
    text = table(best, cus=cus)
    if len(argv) > 1:
        with open(argv[1], "w") as f:
            f.write(text)
    else:
        sys.stdout.write(text)


if __name__ == "__main__":
    main()
