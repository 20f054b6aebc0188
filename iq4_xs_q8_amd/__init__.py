"""iq4_xs_q8_amd -- IQ4_XS x Q8_1 quantized matmul for AMD MI355X (gfx950).

Thin ctypes binding over libiq4xs.so (C ABI in include/iq4xs.h).  This
module only marshals arguments: tensors become device pointers, the current
torch stream becomes the hipStream_t, and non-zero status codes become
Iq4xsError.  Every step of the computation runs in the library's HIP
kernels; there is no CPU or PyTorch fallback, and importing the package
fails loudly when the library has not been built
(``python -m iq4_xs_q8_amd.build``).

Layouts (see the header): W is uint8 [N, K/256*136] (GGUF IQ4_XS super-blocks,
row n = output row n), X fp32 [M, K], Xq uint8 [M, K/32*36] (Q8_1 blocks),
Y fp32 [M, N].
"""

from __future__ import annotations

import contextlib
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libiq4xs.so")

OK, EINVAL, EALIGN, EDEVICE, ETABLE, ELAUNCH, ENOMEM, EPATH = 0, -1, -2, -3, -4, -5, -6, -7
PATH_AUTO, PATH_GEMV, PATH_MMQ, PATH_DEQ_BF16, PATH_BF16X3 = 0, 1, 2, 3, 4
PATHS = {"AUTO": PATH_AUTO, "GEMV": PATH_GEMV, "MMQ": PATH_MMQ, "DEQ_BF16": PATH_DEQ_BF16,
         "BF16X3": PATH_BF16X3}
FMT_IQ4_XS, FMT_IQ4_NL, FMT_Q4_0 = 0, 1, 2
FMTS = {"IQ4_XS": FMT_IQ4_XS, "IQ4_NL": FMT_IQ4_NL, "Q4_0": FMT_Q4_0}
_UNIT_BYTES = {FMT_IQ4_XS: 136, FMT_IQ4_NL: 144, FMT_Q4_0: 144}    # bytes per 256 weights
Y_ZEROED = 0x100     # gemm_act hint: Y already holds zeros

EXPORTS = ("iq4xs_weight_bytes", "iq4xs_q8_1_bytes", "iq4xs_init", "iq4xs_quantize_q8_1",
           "iq4xs_gemm", "iq4xs_gemm_path", "iq4xs_gemm_workspace_bytes", "iq4xs_gemm_ws",
           "iq4xs_gemm_noalloc", "iq4xs_weight_bytes_fmt", "iq4xs_gemm_fmt_workspace_bytes",
           "iq4xs_gemm_fmt", "iq4xs_gemm_q8_1", "iq4xs_act_bytes",
           "iq4xs_prepare_act", "iq4xs_gemm_act", "iq4xs_gemm_act_workspace_bytes", "iq4xs_gemm_act_ws",
           "iq4xs_gemm_group_workspace_bytes", "iq4xs_gemm_group",
           "iq4xs_dequantize_bf16",
           "iq4xs_dispatch", "iq4xs_load_dispatch_table", "iq4xs_path_name", "iq4xs_last_error")


# measurement kernels (include/iq4xs_probe.h)
PROBE_EXPORTS = ("iq4xs_probe_read", "iq4xs_probe_write", "iq4xs_probe_mfma", "iq4xs_probe_mix")
PROBE_MFMA_I8, PROBE_MFMA_BF16 = 0, 1
PROBE_MIX_MFMA, PROBE_MIX_VALU, PROBE_MIX_SAME, PROBE_MIX_SPLIT = 0, 1, 2, 3


class Iq4xsError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"iq4xs error {code}: {message}")
        self.code = code


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m iq4_xs_q8_amd.build`")
    lib = ctypes.CDLL(path)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    sz = ctypes.POINTER(ctypes.c_size_t)
    sig = {
        "iq4xs_weight_bytes": [i64, i64, sz],
        "iq4xs_q8_1_bytes": [i64, i64, sz],
        "iq4xs_init": [],
        "iq4xs_quantize_q8_1": [p, p, i64, i64, p],
        "iq4xs_gemm": [p, p, p, i64, i64, i64, p],
        "iq4xs_gemm_path": [p, p, p, i64, i64, i64, i32, p],
        "iq4xs_gemm_workspace_bytes": [i64, i64, i64, i32, sz],
        "iq4xs_gemm_ws": [p, p, p, i64, i64, i64, i32, p, ctypes.c_size_t, p],
        "iq4xs_gemm_noalloc": [p, p, p, i64, i64, i64, i32, p],
        "iq4xs_weight_bytes_fmt": [i32, i64, i64, sz],
        "iq4xs_gemm_fmt_workspace_bytes": [i32, i64, i64, i64, i32, sz],
        "iq4xs_gemm_fmt": [i32, p, p, p, i64, i64, i64, i32, p, ctypes.c_size_t, p],
        "iq4xs_gemm_q8_1": [p, p, p, i64, i64, i64, i32, p],
        "iq4xs_act_bytes": [i64, i64, sz],
        "iq4xs_prepare_act": [p, p, i64, i64, p],
        "iq4xs_gemm_act": [p, p, p, i64, i64, i64, i32, p],
        "iq4xs_gemm_act_workspace_bytes": [i64, i64, i64, i32, sz],
        "iq4xs_gemm_act_ws": [p, p, p, i64, i64, i64, i32, p, ctypes.c_size_t, p],
        "iq4xs_gemm_group_workspace_bytes": [ctypes.POINTER(i64), i32, i64, i64, sz],
        "iq4xs_gemm_group": [ctypes.POINTER(p), ctypes.POINTER(p), ctypes.POINTER(i64), i32, p, i64, i64, p,
                             ctypes.c_size_t, p],
        "iq4xs_dequantize_bf16": [p, p, i64, i64, p],
        "iq4xs_dispatch": [i64, i64, i64, ctypes.POINTER(ctypes.c_int)],
        "iq4xs_load_dispatch_table": [ctypes.c_char_p],
    }
    sig.update({
        "iq4xs_probe_read": [p, ctypes.c_size_t, p, i32, p],
        "iq4xs_probe_write": [p, ctypes.c_size_t, ctypes.c_uint32, i32, p],
        "iq4xs_probe_mfma": [i32, i32, p, i32, p],
        "iq4xs_probe_mix": [i32, i32, p, i32, p],
    })
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.iq4xs_path_name.argtypes = [ctypes.c_int]
    lib.iq4xs_path_name.restype = ctypes.c_char_p
    lib.iq4xs_last_error.argtypes = []
    lib.iq4xs_last_error.restype = ctypes.c_char_p
    return lib


_lib = None


def _L() -> ctypes.CDLL:
    """The loaded library; raises if libiq4xs.so has not been built."""
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


def __getattr__(name):          # ``iq4_xs_q8_amd.lib`` loads on first access
    if name == "lib":
        return _L()
    raise AttributeError(name)


def check(rc: int) -> None:
    if rc != OK:
        raise Iq4xsError(rc, _L().iq4xs_last_error().decode())


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _on(t: torch.Tensor):
    """Make t's device current for the call (a no-op when it already is)."""
    if not t.is_cuda or t.device.index == torch.cuda.current_device():
        return contextlib.nullcontext()      # (a non-GPU tensor is rejected inside)
    return torch.cuda.device(t.device)


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _shape(t, name: str, shape) -> None:
    """t must be a tensor of exactly `shape` (checked before anything reaches
    the library, which only sees raw pointers)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _at_least(t, name: str, nbytes: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, {nbytes} needed")


def _one_device(*ts) -> None:
    devs = {t.device for t in ts if isinstance(t, torch.Tensor)}
    if len(devs) > 1:
        raise ValueError(f"tensors on different devices: {sorted(str(d) for d in devs)}")


def _mk(t, name: str) -> tuple:
    """(M, K) of a 2-D activation tensor."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D [M, K], got shape {tuple(t.shape)}")
    return int(t.shape[0]), int(t.shape[1])


def _wrows(W, K: int, fmt: int = FMT_IQ4_XS) -> int:
    """N of a weight tensor [N, K/256 * unit bytes] (K a multiple of 256; a
    unit of 256 weights is 136 bytes in IQ4_XS, 144 in IQ4_NL and Q4_0)."""
    if K % 256:
        raise ValueError(f"K must be a multiple of 256, got {K}")
    if fmt not in _UNIT_BYTES:
        raise ValueError(f"unknown weight format {fmt}")
    if not isinstance(W, torch.Tensor) or W.dim() != 2:
        raise ValueError(f"W must be a 2-D tensor [N, {K // 256 * _UNIT_BYTES[fmt]}]")
    _shape(W, "W", (W.shape[0], K // 256 * _UNIT_BYTES[fmt]))
    return int(W.shape[0])


def weight_bytes(N: int, K: int) -> int:
    out = ctypes.c_size_t()
    check(_L().iq4xs_weight_bytes(N, K, ctypes.byref(out)))
    return out.value


def q8_1_bytes(M: int, K: int) -> int:
    out = ctypes.c_size_t()
    check(_L().iq4xs_q8_1_bytes(M, K, ctypes.byref(out)))
    return out.value


def quantize_q8_1(X: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """fp32 [M, K] -> Q8_1 uint8 [M, K/32*36]."""
    M, K = _mk(X, "X")
    if out is None:
        out = torch.empty((M, (K // 32) * 36), dtype=torch.uint8, device=X.device)
    _shape(out, "Xq", (M, (K // 32) * 36))
    _one_device(X, out)
    with _on(X):
        check(_L().iq4xs_quantize_q8_1(_dev(X, torch.float32, "X"), _dev(out, torch.uint8, "Xq"),
                                      M, K, _stream(X)))
    return out


def workspace_bytes(M: int, N: int, K: int, path: int = PATH_AUTO) -> int:
    out = ctypes.c_size_t()
    check(_L().iq4xs_gemm_workspace_bytes(M, N, K, path, ctypes.byref(out)))
    return out.value


def gemm(W: torch.Tensor, X: torch.Tensor, path: int = PATH_AUTO,
         out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Y[M, N] = X[M, K] * W[N, K]^T with X quantized to Q8_1 on the device.

    With `workspace` (uint8, workspace_bytes(M, N, K, path) bytes) nothing is
    allocated inside the call, so it can be captured in a graph."""
    M, K = _mk(X, "X")
    N = _wrows(W, K)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=X.device)
    _shape(out, "Y", (M, N))
    _one_device(W, X, out, workspace)
    with _on(X):
        if workspace is None:
            check(_L().iq4xs_gemm_path(_dev(W, torch.uint8, "W"), _dev(X, torch.float32, "X"),
                                      _dev(out, torch.float32, "Y"), M, N, K, path, _stream(X)))
        else:
            check(_L().iq4xs_gemm_ws(_dev(W, torch.uint8, "W"), _dev(X, torch.float32, "X"),
                                    _dev(out, torch.float32, "Y"), M, N, K, path,
                                    _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
                                    _stream(X)))
    return out


STATIC_SCRATCH_BYTES = 128 << 20    # IQ4XS_STATIC_SCRATCH_BYTES


def gemm_noalloc(W: torch.Tensor, X: torch.Tensor, out: torch.Tensor, path: int = PATH_AUTO) -> torch.Tensor:
    """gemm() with the library's static per-device scratch: nothing is
    allocated (the output must be given).  Calls that overlap on one device
    race on that scratch."""
    M, K = _mk(X, "X")
    N = _wrows(W, K)
    _shape(out, "Y", (M, N))
    _one_device(W, X, out)
    with _on(X):
        check(_L().iq4xs_gemm_noalloc(_dev(W, torch.uint8, "W"), _dev(X, torch.float32, "X"),
                                     _dev(out, torch.float32, "Y"), M, N, K, path, _stream(X)))
    return out


def weight_bytes_fmt(fmt: int, N: int, K: int) -> int:
    out = ctypes.c_size_t()
    check(_L().iq4xs_weight_bytes_fmt(fmt, N, K, ctypes.byref(out)))
    return out.value


def fmt_workspace_bytes(fmt: int, M: int, N: int, K: int, path: int = PATH_AUTO) -> int:
    out = ctypes.c_size_t()
    check(_L().iq4xs_gemm_fmt_workspace_bytes(fmt, M, N, K, path, ctypes.byref(out)))
    return out.value


def gemm_fmt(W: torch.Tensor, X: torch.Tensor, fmt: int, path: int = PATH_AUTO,
             out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Y[M, N] = X[M, K] * W[N, K]^T for W in IQ4_XS, IQ4_NL or Q4_0 (uint8
    [N, K/256 * 136] or [N, K/32 * 18]); X quantized to Q8_1 on the device."""
    M, K = _mk(X, "X")
    N = _wrows(W, K, fmt)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=X.device)
    _shape(out, "Y", (M, N))
    _one_device(W, X, out, workspace)
    with _on(X):
        ws = _dev(workspace, torch.uint8, "workspace") if workspace is not None else None
        wsb = workspace.numel() if workspace is not None else 0
        check(_L().iq4xs_gemm_fmt(fmt, _dev(W, torch.uint8, "W"), _dev(X, torch.float32, "X"),
                                 _dev(out, torch.float32, "Y"), M, N, K, path, ws, wsb, _stream(X)))
    return out


def gemm_q8_1(W: torch.Tensor, Xq: torch.Tensor, K: int, path: int = PATH_AUTO,
              out: torch.Tensor | None = None) -> torch.Tensor:
    """Y[M, N] from already-quantized Q8_1 activations Xq [M, K/32*36]."""
    N = _wrows(W, K)
    if not isinstance(Xq, torch.Tensor) or Xq.dim() != 2:
        raise ValueError("Xq must be a 2-D tensor [M, K/32*36]")
    M = int(Xq.shape[0])
    _shape(Xq, "Xq", (M, K // 32 * 36))
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=Xq.device)
    _shape(out, "Y", (M, N))
    _one_device(W, Xq, out)
    with _on(Xq):
        check(_L().iq4xs_gemm_q8_1(_dev(W, torch.uint8, "W"), _dev(Xq, torch.uint8, "Xq"),
                                  _dev(out, torch.float32, "Y"), M, N, K, path, _stream(Xq)))
    return out


def act_bytes(M: int, K: int) -> int:
    out = ctypes.c_size_t()
    check(_L().iq4xs_act_bytes(M, K, ctypes.byref(out)))
    return out.value


def prepare_act(X: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Quantize fp32 X [M, K] into the kernels' activation layout (opaque uint8)."""
    M, K = _mk(X, "X")
    need = act_bytes(M, K)
    if out is None:
        out = torch.empty(need, dtype=torch.uint8, device=X.device)
    _at_least(out, "act", need)
    _one_device(X, out)
    with _on(X):
        check(_L().iq4xs_prepare_act(_dev(X, torch.float32, "X"), _dev(out, torch.uint8, "act"),
                                    M, K, _stream(X)))
    return out


def act_workspace_bytes(M: int, N: int, K: int, path: int = PATH_AUTO) -> int:
    """Bytes of partial-result scratch gemm_act needs for this shape (often 0)."""
    out = ctypes.c_size_t()
    check(_L().iq4xs_gemm_act_workspace_bytes(M, N, K, path, ctypes.byref(out)))
    return out.value


def gemm_act(W: torch.Tensor, act: torch.Tensor, M: int, K: int, path: int = PATH_AUTO,
             out: torch.Tensor | None = None, y_zeroed: bool = False,
             workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Y[M, N] from prepared activations (the matmul kernel; y_zeroed: `out`
    already holds zeros, so no zeroing kernel runs before it).  With
    `workspace` (uint8, act_workspace_bytes(M, N, K, path) bytes) nothing is
    allocated inside the call, so it can be captured in a graph."""
    N = _wrows(W, K)
    _at_least(act, "act", act_bytes(M, K))
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=act.device)
    _shape(out, "Y", (M, N))
    _one_device(W, act, out, workspace)
    flag = path | (Y_ZEROED if y_zeroed else 0)
    with _on(act):
        if workspace is None:
            check(_L().iq4xs_gemm_act(_dev(W, torch.uint8, "W"), _dev(act, torch.uint8, "act"),
                                     _dev(out, torch.float32, "Y"), M, N, K, flag, _stream(act)))
        else:
            wp = _dev(workspace, torch.uint8, "workspace")
            ws = wp if workspace.numel() else None          # an empty tensor may have no address
            check(_L().iq4xs_gemm_act_ws(_dev(W, torch.uint8, "W"), _dev(act, torch.uint8, "act"),
                                        _dev(out, torch.float32, "Y"), M, N, K, flag, ws,
                                        workspace.numel(), _stream(act)))
    return out


MAX_GROUP = 4     # IQ4XS_MAX_GROUP


def group_workspace_bytes(Ns: list, M: int, K: int) -> int:
    n = (ctypes.c_int64 * max(len(Ns), 1))(*Ns)
    out = ctypes.c_size_t()
    check(_L().iq4xs_gemm_group_workspace_bytes(n, len(Ns), M, K, ctypes.byref(out)))
    return out.value


def gemm_group(Ws: list, X: torch.Tensor, outs: list | None = None,
               workspace: torch.Tensor | None = None) -> list:
    """Y[g] = X * Ws[g]^T for every weight matrix of the group (same K): X is
    quantized once and, where the shapes allow, one matmul launch covers all
    of them.  With `workspace` (uint8, group_workspace_bytes(...) bytes)
    nothing is allocated inside the call."""
    M, K = _mk(X, "X")
    G = len(Ws)
    Ns = [_wrows(W, K) for W in Ws]
    if outs is None:
        outs = [torch.empty((M, N), dtype=torch.float32, device=X.device) for N in Ns]
    if len(outs) != G:
        raise ValueError("one output per weight matrix")
    for g, (o, N) in enumerate(zip(outs, Ns)):
        _shape(o, f"Y[{g}]", (M, N))
    _one_device(X, workspace, *Ws, *outs)
    w = (ctypes.c_void_p * max(G, 1))(*[_dev(W, torch.uint8, "W") for W in Ws])
    y = (ctypes.c_void_p * max(G, 1))(*[_dev(o, torch.float32, "Y") for o in outs])
    n = (ctypes.c_int64 * max(G, 1))(*[W.shape[0] for W in Ws])
    with _on(X):
        ws = _dev(workspace, torch.uint8, "workspace") if workspace is not None else None
        wsb = workspace.numel() if workspace is not None else 0
        check(_L().iq4xs_gemm_group(w, y, n, G, _dev(X, torch.float32, "X"), M, K, ws, wsb, _stream(X)))
    return outs


def dequantize_bf16(W: torch.Tensor, K: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """IQ4_XS [N, K/256*136] -> bf16 [N, K]."""
    N = _wrows(W, K)
    if out is None:
        out = torch.empty((N, K), dtype=torch.bfloat16, device=W.device)
    _shape(out, "Wb", (N, K))
    _one_device(W, out)
    with _on(W):
        check(_L().iq4xs_dequantize_bf16(_dev(W, torch.uint8, "W"), _dev(out, torch.bfloat16, "Wb"),
                                        N, K, _stream(W)))
    return out


def dispatch(M: int, N: int, K: int) -> int:
    p = ctypes.c_int()
    check(_L().iq4xs_dispatch(M, N, K, ctypes.byref(p)))
    return p.value


def load_dispatch_table(path: str | None = None) -> None:
    check(_L().iq4xs_load_dispatch_table(path.encode() if path else None))


def path_name(p: int) -> str:
    return _L().iq4xs_path_name(p).decode()


# ---------------------------------------------------------------- probes
def _probe_check(rc: int, what: str) -> None:
    if rc != 0:
        raise Iq4xsError(rc, f"{what} failed")


def probe_read(buf: torch.Tensor, sink: torch.Tensor, grid: int = 4096) -> None:
    """Stream-read all of buf (uint8, 16-byte multiple) with the library's read probe."""
    _at_least(sink, "sink", 4 * grid)
    with _on(buf):
        _probe_check(_L().iq4xs_probe_read(_dev(buf, torch.uint8, "buf"), buf.numel(),
                                          _dev(sink, torch.int32, "sink"), grid, _stream(buf)), "probe_read")


def probe_write(buf: torch.Tensor, value: int = 0x3F800000, grid: int = 4096) -> None:
    with _on(buf):
        _probe_check(_L().iq4xs_probe_write(_dev(buf, torch.uint8, "buf"), buf.numel(), value, grid,
                                           _stream(buf)), "probe_write")


def probe_mfma(kind: int, iters: int, out: torch.Tensor, grid: int) -> None:
    """out: int32 (int8 probe) or float32 (bf16 probe), grid * 256 elements."""
    _at_least(out, "out", 4 * 256 * grid)
    dt = torch.int32 if kind == PROBE_MFMA_I8 else torch.float32
    with _on(out):
        _probe_check(_L().iq4xs_probe_mfma(kind, iters, _dev(out, dt, "out"), grid, _stream(out)), "probe_mfma")


def probe_mix(mode: int, iters: int, out: torch.Tensor, grid: int) -> None:
    """Matrix-core beside vector-ALU work (PROBE_MIX_*); out: int32, grid * 512 elements."""
    _at_least(out, "out", 4 * 512 * grid)
    with _on(out):
        _probe_check(_L().iq4xs_probe_mix(mode, iters, _dev(out, torch.int32, "out"), grid, _stream(out)),
                     "probe_mix")
