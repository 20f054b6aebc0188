"""Build libiq4xs.so (HIP kernels for gfx950 + the C ABI) in-tree.

    python -m iq4_xs_q8_amd.build      # or iq4_xs_q8_amd.build.build()

Every HIP source is compiled with hipcc for gfx950 only, with packed-FP32
instructions disabled (-packed-fp32-ops) and without fast-math; the object
files go to iq4_xs_q8_amd/_build/ and are linked into
iq4_xs_q8_amd/libiq4xs.so.  The dispatch table text
(csrc/dispatch_gfx950.txt) is embedded as a string literal.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libiq4xs.so")

HIP_SOURCES = ("quantize.hip", "gemv.hip", "mmq.hip", "mmv.hip", "mmqt.hip", "deq.hip", "fused.hip", "abi.hip",
               "probe.hip")
CXX_SOURCES = ("dispatch.cpp",)
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIPFLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra",
            "-Wno-unused-parameter", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", BUILD]
CXXFLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", BUILD]


def _embed_table() -> None:
    with open(os.path.join(CSRC, f"dispatch_{ARCH}.txt")) as f:
        text = f.read()
    lines = ['"' + line.replace("\\", "\\\\").replace('"', '\\"') + '\\n"' for line in text.splitlines()]
    out = os.path.join(BUILD, "dispatch_table.inc")
    body = "\n".join(lines) + "\n"
    if not os.path.exists(out) or open(out).read() != body:
        with open(out, "w") as f:
            f.write(body)


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # the host pass of hipcc does not know the packed-fp32 feature: drop that note
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if msg.strip() and verbose:
        print(msg, file=sys.stderr)


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    _embed_table()
    cmds, objs = [], []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append([HIPCC, *HIPFLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append(["g++", *CXXFLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
