"""Binding of libqgceil.so (include/qgceil.h): the measurement kernels and
host loops that the benchmark reports next to the GEMM kernels -- the
sustained MFMA rate and shader clock, the sustained streaming read rate, how
far vector work overlaps MFMAs on one SIMD, and the host cost of a launch and
of a qg_run call. Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

from . import Layout, Operation, Workspace, _current_stream, _ptr
from . import lib as _qglib

CEIL_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqgceil.so")
EXPORTS = ["qgc_mfma_loop", "qgc_stream_read", "qgc_issue_mix", "qgc_empty", "qgc_host_us_per_call",
           "qgc_host_us_per_empty"]

MFMA_THREADS = 512
MFMA_FLOPS_PER_ROUND = 4 * 32768  # four 32x32x16 MFMAs per wave and round
ISSUE_MFMA_PER_ROUND, ISSUE_VALU_PER_ROUND = 4, 16  # per wave and round of qgc_issue_mix
ISSUE_KINDS = {0: "fma_f32", 1: "bitwise", 2: "fma_mix"}
STREAM_THREADS = 256
STREAM_BLOCK_BYTES = 256 * 8 * 16


def _load():
    if not os.path.exists(CEIL_PATH):
        raise ImportError(f"{CEIL_PATH} is not built; run `python quantized_gemm_bf16_amd/build.py`")
    L = ctypes.CDLL(CEIL_PATH)
    vp, i32, sz, P = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.POINTER
    L.qgc_mfma_loop.argtypes = [i32, i32, vp, vp, vp]
    L.qgc_stream_read.argtypes = [vp, sz, i32, vp, vp]
    L.qgc_issue_mix.argtypes = [i32, i32, i32, i32, vp, vp, vp]
    L.qgc_empty.argtypes = [vp]
    L.qgc_host_us_per_call.argtypes = [vp, i32, vp, P(Operation), ctypes.c_float, vp, P(Layout), vp, P(Layout), vp,
                                       P(Layout), vp, P(Layout), ctypes.c_float, vp, P(Layout), vp, P(Layout),
                                       P(Workspace), vp, P(ctypes.c_double)]
    L.qgc_host_us_per_empty.argtypes = [i32, i32, vp, P(ctypes.c_double)]
    for n in EXPORTS:
        getattr(L, n).restype = i32
    return L


lib = _load()


def _ok(st, what):
    if st != 0:
        raise RuntimeError(f"{what} failed with status {st}")


def mfma_loop(grid, iters, sink, clk, stream=None):
    _ok(lib.qgc_mfma_loop(grid, iters, _ptr(sink), _ptr(clk), stream or _current_stream()), "qgc_mfma_loop")


def stream_read(src, nbytes, grid, sink, stream=None):
    _ok(lib.qgc_stream_read(_ptr(src), nbytes, grid, _ptr(sink), stream or _current_stream()), "qgc_stream_read")


def issue_mix(mode, kind, grid, iters, sink, clk, stream=None):
    _ok(lib.qgc_issue_mix(mode, kind, grid, iters, _ptr(sink), _ptr(clk), stream or _current_stream()),
        "qgc_issue_mix")


def empty(stream=None):
    _ok(lib.qgc_empty(stream or _current_stream()), "qgc_empty")


def host_us_per_run(n, gemm, op, alpha, A, Ad, U, Ud, B, Bd, V, Vd, beta, C, Cd, D, Dd, ws, stream=None):
    """Host microseconds per qg_run call over n back-to-back calls (C loop)."""
    out = ctypes.c_double()
    r = lambda x: ctypes.byref(x) if x is not None else None  # noqa: E731
    fn = ctypes.cast(_qglib.qg_run, ctypes.c_void_p)
    _ok(lib.qgc_host_us_per_call(fn, n, gemm.h, ctypes.byref(op), alpha, _ptr(A), r(Ad), _ptr(U), r(Ud), _ptr(B),
                                 r(Bd), _ptr(V), r(Vd), beta, _ptr(C), r(Cd), _ptr(D), r(Dd), r(ws),
                                 stream or _current_stream(), ctypes.byref(out)), "qgc_host_us_per_call")
    return out.value


def host_us_per_empty(n, arg_bytes=0, stream=None):
    """Host microseconds per launch of an empty kernel (arg_bytes 0 or 256)."""
    out = ctypes.c_double()
    _ok(lib.qgc_host_us_per_empty(n, arg_bytes, stream or _current_stream(), ctypes.byref(out)),
        "qgc_host_us_per_empty")
    return out.value
