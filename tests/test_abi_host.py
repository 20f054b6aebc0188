"""Host-side tests of the C ABI (no GPU needed).

The library must load, export every function include/iq4xs.h declares, and
validate its arguments on the host before any HIP call: argument errors come
back as EINVAL / EALIGN even where no GPU exists, and well-formed calls on a
machine without a gfx950 device come back as EDEVICE.
"""
import ctypes
import json
import os
import re
import subprocess
import sys

import pytest

import iq4_xs_q8_amd as iq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "iq4xs.h")
L = iq.lib
A = 1 << 20          # a 16-byte aligned fake address (never dereferenced)


def _has_gpu():
    import torch
    return torch.cuda.is_available()


def test_header_declarations_are_exported():
    """Every function of every header under include/ is exported by the
    library and bound by the Python package."""
    out = subprocess.run(["nm", "-D", "--defined-only", iq.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (iq4xs_\w+)$", out, flags=re.M))
    for header, names in ((HEADER, iq.EXPORTS), (os.path.join(ROOT, "include", "iq4xs_probe.h"), iq.PROBE_EXPORTS)):
        text = open(header).read()
        declared = set(re.findall(r"^\w[\w\s\*]*?\b(iq4xs_\w+)\s*\(", text, flags=re.M))
        assert declared == set(names), (header, declared ^ set(names))
        assert declared <= exported, declared - exported
    headers = sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))
    assert headers == ["iq4xs.h", "iq4xs_probe.h"], headers


def test_probe_arguments_checked_on_the_host():
    assert L.iq4xs_probe_read(None, 16, A, 1, None) == -1
    assert L.iq4xs_probe_read(A, 15, A, 1, None) == -1
    assert L.iq4xs_probe_read(A + 4, 16, A, 1, None) == -1
    assert L.iq4xs_probe_write(A, 0, 1, 1, None) == -1
    assert L.iq4xs_probe_mfma(7, 1, A, 1, None) == -1
    assert L.iq4xs_probe_mfma(0, 0, A, 1, None) == -1
    assert L.iq4xs_probe_mix(4, 1, A, 1, None) == -1
    assert L.iq4xs_probe_mix(-1, 1, A, 1, None) == -1
    assert L.iq4xs_probe_mix(0, 0, A, 1, None) == -1
    assert L.iq4xs_probe_mix(0, 1, None, 1, None) == -1
    assert L.iq4xs_probe_mix(0, 1, A, 0, None) == -1


def test_probe_constants_match_binding():
    text = open(os.path.join(ROOT, "include", "iq4xs_probe.h")).read()
    consts = dict((k, int(v)) for k, v in re.findall(r"#define (IQ4XS_PROBE_\w+) (\d+)", text))
    assert consts["IQ4XS_PROBE_MFMA_I8"] == iq.PROBE_MFMA_I8 and consts["IQ4XS_PROBE_MFMA_BF16"] == iq.PROBE_MFMA_BF16
    assert [consts[f"IQ4XS_PROBE_MIX_{n}"] for n in ("MFMA", "VALU", "SAME", "SPLIT")] == \
        [iq.PROBE_MIX_MFMA, iq.PROBE_MIX_VALU, iq.PROBE_MIX_SAME, iq.PROBE_MIX_SPLIT]


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict((k, int(v)) for k, v in re.findall(r"#define (IQ4XS_\w+) \(?(-?\d+)\)?", text))
    assert consts["IQ4XS_OK"] == iq.OK and consts["IQ4XS_EINVAL"] == iq.EINVAL
    assert consts["IQ4XS_EALIGN"] == iq.EALIGN and consts["IQ4XS_EDEVICE"] == iq.EDEVICE
    assert consts["IQ4XS_ETABLE"] == iq.ETABLE and consts["IQ4XS_ELAUNCH"] == iq.ELAUNCH
    assert consts["IQ4XS_ENOMEM"] == iq.ENOMEM and consts["IQ4XS_EPATH"] == iq.EPATH
    for name, v in iq.PATHS.items():
        assert consts["IQ4XS_PATH_" + name] == v
        assert iq.path_name(v) == name


def test_sizes():
    assert iq.weight_bytes(10240, 5120) == 10240 * 20 * 136
    assert iq.q8_1_bytes(16, 5120) == 16 * 160 * 36
    out = ctypes.c_size_t()
    for N, K in ((0, 256), (1, 0), (1, 128), (1, 300), (-1, 256)):
        assert L.iq4xs_weight_bytes(N, K, ctypes.byref(out)) == iq.EINVAL
    for M, K in ((0, 32), (1, 16), (1, 33)):
        assert L.iq4xs_q8_1_bytes(M, K, ctypes.byref(out)) == iq.EINVAL
    assert L.iq4xs_weight_bytes(1, 256, None) == iq.EINVAL


@pytest.mark.parametrize("M,N,K", [(0, 8, 256), (4, 0, 256), (4, 8, 0), (4, 8, 128), (4, 8, 300),
                                   (1 << 40, 8, 256), (4, 1 << 40, 256), (70000, 8, 32768)])
def test_gemm_bad_sizes(M, N, K):
    assert L.iq4xs_gemm(A, A * 2, A * 4, M, N, K, None) == iq.EINVAL
    assert L.iq4xs_gemm_q8_1(A, A * 2, A * 4, M, N, K, 0, None) == iq.EINVAL


def test_gemm_null_and_alignment():
    assert L.iq4xs_gemm(None, A, A * 4, 4, 8, 256, None) == iq.EINVAL
    assert L.iq4xs_gemm(A, None, A * 4, 4, 8, 256, None) == iq.EINVAL
    assert L.iq4xs_gemm(A, A * 2, None, 4, 8, 256, None) == iq.EINVAL
    assert L.iq4xs_gemm(A + 8, A * 2, A * 4, 4, 8, 256, None) == iq.EALIGN
    assert L.iq4xs_gemm(A, A * 2 + 4, A * 4, 4, 8, 256, None) == iq.EALIGN
    assert L.iq4xs_gemm(A, A * 2, A * 4 + 4, 4, 8, 256, None) == iq.EALIGN
    assert L.iq4xs_gemm_q8_1(A, A * 2 + 2, A * 4, 4, 8, 256, 0, None) == iq.EALIGN
    assert L.iq4xs_gemm_q8_1(A, A * 2 + 4, A * 4, 4, 8, 256, 0, None) != iq.EALIGN
    assert L.iq4xs_quantize_q8_1(A + 4, A * 2, 4, 256, None) == iq.EALIGN
    assert L.iq4xs_dequantize_bf16(A, A * 2 + 8, 8, 256, None) == iq.EALIGN


def test_overlap_rejected():
    # Y inside W, Y inside X
    assert L.iq4xs_gemm(A, A * 4, A + 256, 4, 8, 256, None) == iq.EINVAL
    assert L.iq4xs_gemm(A * 4, A, A + 256, 4, 8, 256, None) == iq.EINVAL
    assert L.iq4xs_gemm_q8_1(A * 4, A, A + 64, 4, 8, 256, 0, None) == iq.EINVAL
    assert L.iq4xs_quantize_q8_1(A, A + 16, 4, 256, None) == iq.EINVAL


def test_unknown_path_and_gemv_limit():
    assert L.iq4xs_gemm_path(A, A * 2, A * 4, 4, 8, 256, 9, None) == iq.EINVAL
    assert L.iq4xs_gemm_path(A, A * 2, A * 4, 4, 8, 256, -1, None) == iq.EINVAL
    assert L.iq4xs_gemm_path(A, A * 2, A * 4, 5, 8, 256, iq.PATH_GEMV, None) == iq.EPATH


def test_fused_path_on_the_host():
    """The fused compensated path (BF16X3): its name, its scratch (the hi/lo
    activation planes, 4 bytes per element of M rounded up to 256 rows), its
    band in a table, and the prepared-activation entry point refusing it."""
    assert iq.path_name(iq.PATH_BF16X3) == "BF16X3" and iq.PATHS["BF16X3"] == iq.PATH_BF16X3
    size = ctypes.c_size_t()
    for M, K in ((1, 256), (256, 5120), (257, 5120), (512, 17408)):
        assert L.iq4xs_gemm_workspace_bytes(M, 4096, K, iq.PATH_BF16X3, ctypes.byref(size)) == iq.OK
        assert size.value == (K // 32) * (-(-M // 256) * 256) * 128, (M, K)
    assert L.iq4xs_gemm_workspace_bytes(4, 1024, 300, iq.PATH_BF16X3, ctypes.byref(size)) == iq.EINVAL
    # prepared activations feed the integer kernels only
    ab = ctypes.c_size_t()
    assert L.iq4xs_act_bytes(256, 512, ctypes.byref(ab)) == iq.OK
    assert L.iq4xs_gemm_act(A, 1 << 44, 2 << 44, 256, 512, 512, iq.PATH_BF16X3, None) == iq.EPATH


def test_workspace_query_and_checks():
    size = ctypes.c_size_t()
    ref = {}
    for path in (iq.PATH_GEMV, iq.PATH_MMQ, iq.PATH_DEQ_BF16):
        assert L.iq4xs_gemm_workspace_bytes(4, 1024, 2048, path, ctypes.byref(size)) == iq.OK
        ref[path] = size.value
        assert size.value > 0
    # the bf16 path holds the hi/lo bf16 activation planes of 256 padded rows (no
    # weight copy: it dequantizes inside the GEMM); the integer paths the Q8_1 planes
    assert ref[iq.PATH_DEQ_BF16] == (2048 // 32) * 256 * 128
    assert ref[iq.PATH_GEMV] >= 4 * 2048 * 1.125
    assert L.iq4xs_gemm_workspace_bytes(4, 1024, 2048, iq.PATH_AUTO, ctypes.byref(size)) == iq.OK
    assert size.value == ref[iq.dispatch(4, 1024, 2048)]
    assert L.iq4xs_gemm_workspace_bytes(5, 1024, 2048, iq.PATH_GEMV, ctypes.byref(size)) == iq.EPATH
    assert L.iq4xs_gemm_workspace_bytes(4, 1024, 300, iq.PATH_MMQ, ctypes.byref(size)) == iq.EINVAL
    assert L.iq4xs_gemm_workspace_bytes(4, 1024, 2048, iq.PATH_MMQ, None) == iq.EINVAL
    assert iq.workspace_bytes(4, 1024, 2048, iq.PATH_MMQ) == ref[iq.PATH_MMQ]

    need = iq.workspace_bytes(4, 8, 256, iq.PATH_MMQ)
    WS = 1 << 30
    assert L.iq4xs_gemm_ws(A, A * 2, A * 4, 4, 8, 256, iq.PATH_MMQ, None, need, None) == iq.EINVAL
    assert L.iq4xs_gemm_ws(A, A * 2, A * 4, 4, 8, 256, iq.PATH_MMQ, WS, need - 1, None) == iq.EINVAL
    assert L.iq4xs_gemm_ws(A, A * 2, A * 4, 4, 8, 256, iq.PATH_MMQ, WS + 16, need, None) == iq.EALIGN
    assert L.iq4xs_gemm_ws(A, A * 2, A * 4, 4, 8, 256, iq.PATH_MMQ, A * 4 - 256, need, None) == iq.EINVAL
    # the workspace must not overlap X either (the quantizer reads X while it
    # writes the activation planes into the workspace)
    assert L.iq4xs_gemm_ws(A, A * 2, A * 4, 4, 8, 256, iq.PATH_MMQ, A * 2 + 256, need, None) == iq.EINVAL
    assert "workspace overlaps" in L.iq4xs_last_error().decode()
    assert L.iq4xs_gemm_ws(A, A * 2, A * 4, 5, 8, 256, iq.PATH_GEMV, WS, need, None) == iq.EPATH
    assert L.iq4xs_gemm_ws(A, A * 2, A * 4 + 4, 4, 8, 256, iq.PATH_MMQ, WS, need, None) == iq.EALIGN


def test_act_workspace_query_and_checks():
    """The prepared-activation matmul's own scratch: exactly the partial-tile
    part of iq4xs_gemm_ws's scratch (which also holds the activation planes),
    0 where no tile has more than two owners; the caller-workspace entry point
    checks it before anything runs."""
    size = ctypes.c_size_t()
    for M, N, K in ((64, 5120, 1024), (128, 5120, 17408), (100, 200, 4096), (512, 248320, 5120), (8, 300, 1024)):
        assert L.iq4xs_gemm_act_workspace_bytes(M, N, K, iq.PATH_MMQ, ctypes.byref(size)) == iq.OK
        planes = -(-iq.act_bytes(M, K) // 256) * 256
        assert size.value == iq.workspace_bytes(M, N, K, iq.PATH_MMQ) - planes, (M, N, K)
        assert iq.act_workspace_bytes(M, N, K, iq.PATH_MMQ | iq.Y_ZEROED) == size.value
    assert iq.act_workspace_bytes(64, 5120, 1024, iq.PATH_MMQ) > 0
    assert iq.act_workspace_bytes(512, 248320, 5120, iq.PATH_MMQ) == 0
    assert iq.act_workspace_bytes(4, 1024, 2048, iq.PATH_GEMV) == 0
    assert L.iq4xs_gemm_act_workspace_bytes(4, 1024, 2048, iq.PATH_MMQ, None) == iq.EINVAL
    assert L.iq4xs_gemm_act_workspace_bytes(4, 1024, 300, iq.PATH_MMQ, ctypes.byref(size)) == iq.EINVAL
    assert L.iq4xs_gemm_act_workspace_bytes(5, 1024, 2048, iq.PATH_GEMV, ctypes.byref(size)) == iq.EPATH
    assert L.iq4xs_gemm_act_workspace_bytes(4, 1024, 2048, iq.PATH_DEQ_BF16, ctypes.byref(size)) == iq.EPATH
    assert L.iq4xs_gemm_act_workspace_bytes(4, 1024, 2048, iq.PATH_BF16X3, ctypes.byref(size)) == iq.EPATH

    M, N, K = 64, 5120, 1024
    need = iq.act_workspace_bytes(M, N, K, iq.PATH_MMQ)
    W, ACT, Y, WS = A, A * 2, A * 4, A * 8
    f = L.iq4xs_gemm_act_ws
    assert f(None, ACT, Y, M, N, K, iq.PATH_MMQ, WS, need, None) == iq.EINVAL
    assert f(W, ACT, Y, M, N, K, iq.PATH_MMQ, None, need, None) == iq.EINVAL
    assert "null workspace" in L.iq4xs_last_error().decode()
    assert f(W, ACT, Y, M, N, K, iq.PATH_MMQ, WS, need - 1, None) == iq.EINVAL
    assert f(W, ACT, Y, M, N, K, iq.PATH_MMQ, WS + 16, need, None) == iq.EALIGN
    assert f(W, ACT + 16, Y, M, N, K, iq.PATH_MMQ, WS, need, None) == iq.EALIGN
    for ws in (Y + 256, W + 256, ACT + 256, Y - 256):
        assert f(W, ACT, Y, M, N, K, iq.PATH_MMQ, ws, need, None) == iq.EINVAL, hex(ws)
        assert "workspace overlaps" in L.iq4xs_last_error().decode()
    assert f(W, ACT, Y, M, N, K, iq.PATH_DEQ_BF16, WS, need, None) == iq.EPATH


@pytest.mark.skipif(_has_gpu(), reason="checks the no-device error")
def test_no_device_reports_edevice():
    assert L.iq4xs_gemm(A, A * 2, A * 4, 4, 8, 256, None) == iq.EDEVICE
    ws = iq.workspace_bytes(4, 8, 256, iq.PATH_MMQ)
    assert L.iq4xs_gemm_ws(A, A * 2, A * 4, 4, 8, 256, iq.PATH_MMQ, 1 << 30, ws, None) == iq.EDEVICE
    assert "device" in L.iq4xs_last_error().decode()
    assert L.iq4xs_quantize_q8_1(A, A * 2, 4, 256, None) == iq.EDEVICE
    assert L.iq4xs_dequantize_bf16(A, A * 2, 8, 256, None) == iq.EDEVICE
    # with nothing to check in the workspace (a shape that needs none), a NULL one
    # passes the argument checks and the call stops at the device
    assert iq.act_workspace_bytes(512, 248320, 5120, iq.PATH_MMQ) == 0
    assert L.iq4xs_gemm_act_ws(1 << 40, 2 << 40, 3 << 40, 512, 248320, 5120, iq.PATH_MMQ, None, 0, None) == iq.EDEVICE


def _group_args(ws, ys, ns):
    G = max(len(ws), 1)
    return ((ctypes.c_void_p * G)(*ws), (ctypes.c_void_p * G)(*ys), (ctypes.c_int64 * G)(*ns))


def test_gemm_group_validation():
    g = L.iq4xs_gemm_group
    w, y, n = _group_args([A, A * 2], [A * 4, A * 8], [8, 16])
    assert g(None, y, n, 2, A * 16, 4, 256, None, 0, None) == iq.EINVAL
    assert g(w, y, n, 2, None, 4, 256, None, 0, None) == iq.EINVAL
    assert g(w, y, n, 0, A * 16, 4, 256, None, 0, None) == iq.EINVAL
    w5, y5, n5 = _group_args([A] * 5, [A * 4] * 5, [8] * 5)
    assert g(w5, y5, n5, 5, A * 16, 4, 256, None, 0, None) == iq.EINVAL
    assert g(w, y, n, 2, A * 16 + 4, 4, 256, None, 0, None) == iq.EALIGN
    wa, ya, na = _group_args([A, A * 2 + 8], [A * 4, A * 8], [8, 16])
    assert g(wa, ya, na, 2, A * 16, 4, 256, None, 0, None) == iq.EALIGN
    wz, yz, nz = _group_args([A, None], [A * 4, A * 8], [8, 16])
    assert g(wz, yz, nz, 2, A * 16, 4, 256, None, 0, None) == iq.EINVAL
    wb, yb, nb = _group_args([A, A * 2], [A * 4, A * 8], [8, 0])
    assert g(wb, yb, nb, 2, A * 16, 4, 256, None, 0, None) == iq.EINVAL
    assert g(w, y, n, 2, A * 16, 4, 300, None, 0, None) == iq.EINVAL
    # an output overlapping another output, a weight matrix or X
    wo, yo, no = _group_args([A, A * 2], [A * 4, A * 4 + 64], [8, 16])
    assert g(wo, yo, no, 2, A * 16, 4, 256, None, 0, None) == iq.EINVAL
    wo, yo, no = _group_args([A, A * 2], [A * 4, A * 2], [8, 16])
    assert g(wo, yo, no, 2, A * 16, 4, 256, None, 0, None) == iq.EINVAL
    assert g(w, y, n, 2, A * 8, 4, 256, None, 0, None) == iq.EINVAL
    assert "overlap" in L.iq4xs_last_error().decode()
    # caller workspace: aligned, and overlapping nothing
    assert g(w, y, n, 2, A * 16, 4, 256, A * 64 + 16, 1 << 20, None) == iq.EALIGN
    assert g(w, y, n, 2, A * 16, 4, 256, A * 4, 1 << 20, None) == iq.EINVAL
    size = ctypes.c_size_t()
    assert L.iq4xs_gemm_group_workspace_bytes(n, 0, 4, 256, ctypes.byref(size)) == iq.EINVAL
    assert L.iq4xs_gemm_group_workspace_bytes(n, 2, 4, 300, ctypes.byref(size)) == iq.EINVAL
    assert L.iq4xs_gemm_group_workspace_bytes(n, 2, 4, 256, None) == iq.EINVAL


@pytest.mark.skipif(_has_gpu(), reason="checks the no-device error")
def test_gemm_group_no_device():
    w, y, n = _group_args([A, A * 2], [A * 4, A * 8], [8, 16])
    assert L.iq4xs_gemm_group(w, y, n, 2, A * 16, 4, 256, None, 0, None) == iq.EDEVICE


def test_default_dispatch_table():
    iq.load_dispatch_table(None)
    seen = set()
    for M in list(range(1, 130)) + [192, 256, 384, 512, 1000]:
        for (N, K) in ((10240, 5120), (5120, 17408), (2048, 2048), (248320, 5120)):
            p = iq.dispatch(M, N, K)
            seen.add(p)
            assert p in (iq.PATH_GEMV, iq.PATH_MMQ), (M, N, K, p)
            if p == iq.PATH_GEMV:
                assert M <= 4
    assert iq.PATH_MMQ in seen


def test_table_loading(tmp_path):
    good = tmp_path / "t.txt"
    good.write_text("arch gfx950\nband GEMV 4 4 1024 *\nband MMQ 1 7 * *\nband MMQ 8 100000 * *\n")
    bad_gemv = tmp_path / "g.txt"
    bad_gemv.write_text("arch gfx950\nband GEMV 1 9 * *\n")
    garbled = tmp_path / "b.txt"
    garbled.write_text("arch gfx950\nband MMQ one 7 * *\n")
    noarch = tmp_path / "n.txt"
    noarch.write_text("band MMQ 1 7 * *\n")
    ranged = tmp_path / "r.txt"
    ranged.write_text("arch gfx950\nband GEMV 1 4 1-4096 256-512\nband MMQ 1 100000 * *\n")
    bad_ranges = []
    for i, rng in enumerate(("5-3", "0-9", "1-", "-4", "1-2-3", "a-b")):
        f = tmp_path / f"br{i}.txt"
        f.write_text(f"arch gfx950\nband MMQ 1 7 {rng} *\n")
        bad_ranges.append(f)
    try:
        iq.load_dispatch_table(str(ranged))
        assert iq.dispatch(4, 4096, 256) == iq.PATH_GEMV
        assert iq.dispatch(1, 1, 512) == iq.PATH_GEMV
        assert iq.dispatch(4, 4097, 256) == iq.PATH_MMQ
        assert iq.dispatch(4, 4096, 768) == iq.PATH_MMQ
        assert iq.dispatch(5, 4096, 256) == iq.PATH_MMQ
        iq.load_dispatch_table(str(good))
        assert iq.dispatch(3, 4096, 256) == iq.PATH_MMQ
        assert iq.dispatch(4, 1024, 256) == iq.PATH_GEMV
        assert iq.dispatch(4, 2048, 256) == iq.PATH_MMQ
        for f in (bad_gemv, garbled, noarch, tmp_path / "missing.txt", *bad_ranges):
            assert L.iq4xs_load_dispatch_table(str(f).encode()) == iq.ETABLE
            # previous table still in force
            assert iq.dispatch(3, 4096, 256) == iq.PATH_MMQ
        # M outside every band
        short = tmp_path / "s.txt"
        short.write_text("arch gfx950\nband MMQ 1 7 * *\n")
        iq.load_dispatch_table(str(short))
        p = ctypes.c_int()
        assert L.iq4xs_dispatch(8, 4096, 256, ctypes.byref(p)) == iq.EPATH
    finally:
        iq.load_dispatch_table(None)


def test_bf16_bands_need_opt_in(tmp_path):
    t = tmp_path / "t.txt"
    t.write_text("arch gfx950\nband DEQ_BF16 64 100000 * *\nband MMQ 1 100000 * *\n")
    code = ("import iq4_xs_q8_amd as iq, sys; iq.load_dispatch_table(sys.argv[1]); "
            "print(iq.dispatch(128, 4096, 4096))")
    env = dict(os.environ, PYTHONPATH=ROOT)
    env.pop("IQ4XS_ALLOW_BF16", None)
    off = subprocess.run([sys.executable, "-c", code, str(t)], env=env, capture_output=True,
                         text=True, check=True).stdout.strip()
    env["IQ4XS_ALLOW_BF16"] = "1"
    on = subprocess.run([sys.executable, "-c", code, str(t)], env=env, capture_output=True,
                        text=True, check=True).stdout.strip()
    assert int(off) == iq.PATH_MMQ and int(on) == iq.PATH_DEQ_BF16


def test_env_table_read_once_and_fail_closed(tmp_path):
    bad = tmp_path / "bad.txt"
    bad.write_text("garbage\n")
    code = ("import ctypes, iq4_xs_q8_amd as iq; p = ctypes.c_int(); "
            "print(iq.lib.iq4xs_init(), iq.lib.iq4xs_dispatch(8, 4096, 4096, ctypes.byref(p)))")
    env = dict(os.environ, PYTHONPATH=ROOT, IQ4XS_DISPATCH_TABLE=str(bad))
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                         check=True).stdout.split()
    assert [int(v) for v in out] == [iq.ETABLE, iq.ETABLE]


def test_calibrate_writes_a_loadable_table(tmp_path):
    """The sweep -> table step: bands follow the measured winners."""
    from iq4_xs_q8_amd import calibrate
    recs = []
    def rec(N, K, M, path, ms):
        recs.append({"N": N, "K": K, "M": M, "path": path, "ms": ms})
    for M, g, q in ((1, 0.010, 0.012), (2, 0.011, 0.012), (4, 0.013, 0.012)):
        rec(4096, 1024, M, "GEMV", g)
        rec(4096, 1024, M, "MMQ", q)
    rec(8192, 1024, 1, "GEMV", 0.02)
    rec(8192, 1024, 1, "MMQ", 0.01)
    for M, q, b in ((128, 0.1, 0.2), (256, 0.3, 0.2), (512, 0.6, 0.4)):
        rec(4096, 4096, M, "MMQ", q)
        rec(4096, 4096, M, "DEQ_BF16", b)
    for M, q, x in ((64, 0.1, 0.2), (128, 0.2, 0.15), (256, 0.3, 0.35), (512, 0.6, 0.5)):
        rec(8192, 4096, M, "MMQ", q)
        rec(8192, 4096, M, "BF16X3", x)
    sweep = tmp_path / "sweep.jsonl"
    sweep.write_text("\n".join(json.dumps(r) for r in recs) + "\n")
    out = tmp_path / "table.txt"
    calibrate.main([str(sweep), str(out)])
    text = out.read_text()
    assert "band GEMV 1 3 4096 1024" in text and "band DEQ_BF16 256 1000000000 4096 4096" in text
    # the fused path wins at 128 but not at 256, so only from 512 on
    assert "band BF16X3 512 1000000000 8192 4096" in text
    try:
        iq.load_dispatch_table(str(out))
        assert iq.dispatch(2, 4096, 1024) == iq.PATH_GEMV
        assert iq.dispatch(4, 4096, 1024) == iq.PATH_MMQ
        assert iq.dispatch(1, 8192, 1024) == iq.PATH_MMQ
        assert iq.dispatch(300, 4096, 4096) == iq.PATH_MMQ      # bf16 bands need the opt-in
        assert iq.dispatch(600, 8192, 4096) == iq.PATH_BF16X3    # within the bound: no opt-in
        assert iq.dispatch(300, 8192, 4096) == iq.PATH_MMQ
    finally:
        iq.load_dispatch_table(None)


def test_table_compute_unit_key(tmp_path):
    """The table may name the compute-unit count its bands were measured on;
    a malformed count is refused as a whole, a valid one loads (the count is
    compared with the device's only when an AUTO call runs on a device, which
    the GPU tests check), and the built-in table names 256."""
    ok = tmp_path / "ok.txt"
    ok.write_text("arch gfx950\ncus 128\nband MMQ 1 1000000000 * *\n")
    try:
        iq.load_dispatch_table(str(ok))
        assert iq.dispatch(8, 4096, 4096) == iq.PATH_MMQ      # host-only query: no device check
        for i, bad in enumerate(("cus 0", "cus x", "cus -4", "cus 1 2", "cus 99999999")):
            f = tmp_path / f"bad{i}.txt"
            f.write_text(f"arch gfx950\n{bad}\nband GEMV 1 4 * *\n")
            assert L.iq4xs_load_dispatch_table(str(f).encode()) == iq.ETABLE, bad
            assert iq.dispatch(2, 4096, 4096) == iq.PATH_MMQ  # the previous table stays
    finally:
        iq.load_dispatch_table(None)
    builtin = open(os.path.join(ROOT, "iq4_xs_q8_amd", "csrc", "dispatch_gfx950.txt")).read()
    assert re.search(r"^cus 256$", builtin, flags=re.M)


def test_calibrate_carries_the_compute_unit_count(tmp_path):
    from iq4_xs_q8_amd import calibrate
    recs = [{"N": 4096, "K": 1024, "M": 1, "path": p, "ms": t, "cus": 256}
            for p, t in (("GEMV", 0.01), ("MMQ", 0.02))]
    sweep = tmp_path / "sweep.jsonl"
    sweep.write_text("\n".join(json.dumps(r) for r in recs) + "\n")
    out = tmp_path / "table.txt"
    calibrate.main([str(sweep), str(out)])
    assert "\ncus 256\n" in out.read_text()
    recs.append(dict(recs[0], cus=128))
    sweep.write_text("\n".join(json.dumps(r) for r in recs) + "\n")
    with pytest.raises(SystemExit):
        calibrate.main([str(sweep), str(out)])


def test_noalloc_rejects_shapes_beyond_the_static_scratch():
    """The allocation-free entry point refuses, on the host and before any
    HIP call, a shape whose scratch would not fit the static array."""
    assert iq.STATIC_SCRATCH_BYTES == 128 << 20
    text = open(HEADER).read()
    assert re.search(r"#define IQ4XS_STATIC_SCRATCH_BYTES \(128u << 20\)", text)
    # activation planes of 8192 x 17408 alone are 160 MB
    far = 1 << 44                     # fake addresses far apart: no overlap
    assert L.iq4xs_gemm_noalloc(A, far, 2 * far, 8192, 8, 17408, iq.PATH_MMQ, None) == iq.EINVAL
    assert b"static scratch" in L.iq4xs_last_error()
    # the bf16 paths' activation planes at 8192 x 17408: 570 MB
    for p in (iq.PATH_DEQ_BF16, iq.PATH_BF16X3):
        assert L.iq4xs_gemm_noalloc(A, far, 2 * far, 8192, 8, 17408, p, None) == iq.EINVAL
    assert b"static scratch" in L.iq4xs_last_error()
    # argument checks as iq4xs_gemm_path
    assert L.iq4xs_gemm_noalloc(None, A * 2, A * 4, 4, 8, 256, 0, None) == iq.EINVAL
    assert L.iq4xs_gemm_noalloc(A + 8, A * 2, A * 4, 4, 8, 256, 0, None) == iq.EALIGN
    assert L.iq4xs_gemm_noalloc(A, A * 2, A * 4, 4, 8, 300, 0, None) == iq.EINVAL
    if not _has_gpu():
        assert L.iq4xs_gemm_noalloc(A, A * 2, A * 4, 4, 8, 256, 0, None) == iq.EDEVICE


def test_format_entry_points_validate_on_the_host():
    out = ctypes.c_size_t()
    assert L.iq4xs_weight_bytes_fmt(iq.FMT_IQ4_XS, 10, 512, ctypes.byref(out)) == iq.OK and out.value == 10 * 2 * 136
    assert L.iq4xs_weight_bytes_fmt(iq.FMT_IQ4_NL, 10, 512, ctypes.byref(out)) == iq.OK and out.value == 10 * 16 * 18
    assert L.iq4xs_weight_bytes_fmt(iq.FMT_Q4_0, 10, 512, ctypes.byref(out)) == iq.OK and out.value == 10 * 16 * 18
    assert iq.weight_bytes_fmt(iq.FMT_Q4_0, 5120, 17408) == 5120 * 544 * 18
    assert L.iq4xs_weight_bytes_fmt(3, 10, 512, ctypes.byref(out)) == iq.EINVAL
    assert L.iq4xs_weight_bytes_fmt(-1, 10, 512, ctypes.byref(out)) == iq.EINVAL
    assert L.iq4xs_weight_bytes_fmt(iq.FMT_IQ4_NL, 10, 480, ctypes.byref(out)) == iq.EINVAL   # K % 256
    far = 1 << 44
    for bad_fmt in (3, 7, -2):
        assert L.iq4xs_gemm_fmt(bad_fmt, A, far, 2 * far, 4, 8, 256, 0, None, 0, None) == iq.EINVAL
    for fmt in (iq.FMT_IQ4_NL, iq.FMT_Q4_0):
        # the bf16 paths read IQ4_XS only
        for p in (iq.PATH_DEQ_BF16, iq.PATH_BF16X3):
            assert L.iq4xs_gemm_fmt(fmt, A, far, 2 * far, 64, 8, 256, p, None, 0, None) == iq.EPATH
            assert L.iq4xs_gemm_fmt_workspace_bytes(fmt, 64, 8, 256, p, ctypes.byref(out)) == iq.EPATH
        assert L.iq4xs_gemm_fmt(fmt, A, far, 2 * far, 4, 8, 300, 0, None, 0, None) == iq.EINVAL
        assert L.iq4xs_gemm_fmt(fmt, A + 8, far, 2 * far, 4, 8, 256, 0, None, 0, None) == iq.EALIGN
        assert L.iq4xs_gemm_fmt(fmt, A, far, 2 * far, 5, 8, 256, iq.PATH_GEMV, None, 0, None) == iq.EPATH
        # Y overlapping W (18-byte blocks: 8 x 256 weights = 1152 bytes)
        assert L.iq4xs_gemm_fmt(fmt, A, far, A + 1024, 4, 8, 256, 0, None, 0, None) == iq.EINVAL
        if not _has_gpu():
            assert L.iq4xs_gemm_fmt(fmt, A, far, 2 * far, 4, 8, 256, 0, None, 0, None) == iq.EDEVICE
        assert iq.fmt_workspace_bytes(fmt, 16, 1024, 512, iq.PATH_MMQ) > 0


def test_format_binding_shapes():
    import torch
    X = torch.zeros((4, 512))
    with pytest.raises(ValueError, match="W must have shape"):
        iq.gemm_fmt(torch.zeros((8, 512 // 256 * 136), dtype=torch.uint8), X, iq.FMT_IQ4_NL)
    with pytest.raises(ValueError, match="unknown weight format"):
        iq.gemm_fmt(torch.zeros((8, 288), dtype=torch.uint8), X, 5)
    with pytest.raises(TypeError, match="CUDA"):
        iq.gemm_fmt(torch.zeros((8, 288), dtype=torch.uint8), X, iq.FMT_Q4_0)


def test_calibrate_reads_the_text_summary(tmp_path):
    """The committed sweep summary reproduces the table calibrate.py writes
    from the JSONL it was made from."""
    from iq4_xs_q8_amd import calibrate
    recs = []
    for M, g, q in ((1, 0.010, 0.012), (2, 0.011, 0.012), (4, 0.013, 0.012)):
        recs += [{"N": 4096, "K": 1024, "M": M, "path": "GEMV", "ms": g, "cus": 256},
                 {"N": 4096, "K": 1024, "M": M, "path": "MMQ", "ms": q, "cus": 256, "kernel_ms": q * 0.8}]
    sweep = tmp_path / "sweep.jsonl"
    sweep.write_text("\n".join(json.dumps(r) for r in recs) + "\n")
    text = tmp_path / "sweep.txt"
    subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-sweep", str(sweep), "--out",
                    str(text), "--cmd", "test"], check=True, capture_output=True, env=dict(os.environ, PYTHONPATH=ROOT))
    a, b = tmp_path / "a.txt", tmp_path / "b.txt"
    calibrate.main([str(sweep), str(a)])
    calibrate.main([str(text), str(b)])
    assert a.read_text() == b.read_text() and "cus 256" in a.read_text()
    # the committed summary reproduces the built-in table
    committed = os.path.join(ROOT, "profiles", "dispatch_sweep_gfx950.txt")
    if os.path.exists(committed):
        c = tmp_path / "c.txt"
        calibrate.main([committed, str(c)])
        builtin = open(os.path.join(ROOT, "iq4_xs_q8_amd", "csrc", "dispatch_gfx950.txt")).read()
        assert c.read_text() == builtin
