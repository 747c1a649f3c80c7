"""Python binding of libqgemm.so (argument marshalling only).

Every name mirrors an entry point of include/qgemm.h; the functions build the
descriptor structs, pass raw device pointers and the current HIP stream, and
turn negative status codes into `QGemmError`. All arithmetic runs in the
library's gfx950 kernels. PyTorch supplies device memory and streams.

The library must have been built (`python quantized_gemm_bf16_amd/build.py`);
importing this package without it raises immediately -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgemm.so")

# ---- enums (include/qgemm.h) -------------------------------------------------
F32, F16, BF16, E4M3, I8, I32, U4 = 0, 1, 2, 3, 4, 5, 6
ROW_MAJOR, COL_MAJOR = 0, 1
POLICY_DEFAULT, POLICY_MEASURE, POLICY_REUSE, POLICY_FORCE = 0, 1, 2, 3
EPI_ALPHA_BETA, EPI_BIAS, EPI_RELU, EPI_GELU, EPI_QUANT_I8 = 0, 1, 2, 4, 8
QUANT_NONE, QUANT_INT4_ZP, QUANT_BLOCK_F32 = 0, 1, 2
SCHED_AUTO, SCHED_DP, SCHED_SPLITK, SCHED_STREAMK = 0, 1, 2, 3

OK = 0
ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_ALIGNMENT, ERR_WORKSPACE = -1, -2, -3, -4
ERR_NO_KERNEL, ERR_HIP, ERR_FORMAT, ERR_BUFFER_SMALL = -5, -6, -7, -8

DTYPE_CODES = {"f32": F32, "f16": F16, "bf16": BF16, "e4m3": E4M3, "i8": I8, "i32": I32, "u4": U4}

EXPORTS = ["qg_create", "qg_destroy", "qg_barriers_size", "qg_partials_size", "qg_run", "qg_plan",
           "qg_export", "qg_import", "qg_get_tuning_seq", "qg_cache_size", "qg_kernel_count",
           "qg_kernel_name", "qg_status_str", "qg_version", "qg_streamk_units", "qg_streamk_fixup",
           "qg_run_noalloc", "qg_noalloc_barriers_size", "qg_noalloc_partials_size", "qg_run_timed"]


class Layout(ctypes.Structure):
    _fields_ = [("type", ctypes.c_int32), ("order", ctypes.c_int32), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("ld", ctypes.c_int64), ("num", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("offsets", ctypes.c_void_p), ("stride", ctypes.c_int64)]


class Quant(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("group_k", ctypes.c_int32), ("group_mn", ctypes.c_int32),
                ("zero_point", ctypes.c_int32)]


class EpilogueArgs(ctypes.Structure):
    _fields_ = [("bias", ctypes.c_void_p), ("bias_type", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("row_scale", ctypes.c_void_p), ("zero_point", ctypes.c_float), ("reserved1", ctypes.c_int32)]


class Operation(ctypes.Structure):
    _fields_ = [("policy", ctypes.c_int32), ("epilogue", ctypes.c_int32), ("quant_a", Quant),
                ("quant_b", Quant), ("schedule", ctypes.c_int32), ("split_k", ctypes.c_int32),
                ("programs", ctypes.c_int32), ("kernel", ctypes.c_int32), ("epi", EpilogueArgs)]


class Workspace(ctypes.Structure):
    _fields_ = [("barriers", ctypes.c_void_p), ("barriers_size", ctypes.c_size_t),
                ("partials", ctypes.c_void_p), ("partials_size", ctypes.c_size_t)]


class QGemmError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} ({status})")


def _load(path=LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python quantized_gemm_bf16_amd/build.py`")
    # PyTorch ships its own HIP runtime, asked for by file name (libamdhip64.so)
    # but carrying the soname libamdhip64.so.7 that libqgemm.so asks for. Loaded
    # first, it satisfies both; if libqgemm.so came first, torch would load a
    # second HIP runtime into the process and the two would not share devices.
    import torch  # noqa: F401
    L = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    P = ctypes.POINTER
    L.qg_create.argtypes = [P(vp)]
    L.qg_destroy.argtypes = [vp]
    L.qg_barriers_size.restype = sz
    L.qg_partials_size.restype = sz
    L.qg_run.argtypes = [vp, P(Operation), ctypes.c_float, vp, P(Layout), vp, P(Layout), vp, P(Layout), vp,
                         P(Layout), ctypes.c_float, vp, P(Layout), vp, P(Layout), P(Workspace), vp]
    L.qg_run_noalloc.argtypes = [vp, P(Operation), ctypes.c_float, vp, P(Layout), vp, P(Layout), vp, P(Layout),
                                 vp, P(Layout), ctypes.c_float, vp, P(Layout), vp, P(Layout), vp]
    L.qg_run_timed.argtypes = [vp, P(Operation), ctypes.c_float, vp, P(Layout), vp, P(Layout), vp, P(Layout), vp,
                               P(Layout), ctypes.c_float, vp, P(Layout), vp, P(Layout), P(Workspace), vp,
                               vp, ctypes.c_int64, P(ctypes.c_int64)]
    L.qg_noalloc_barriers_size.restype = sz
    L.qg_noalloc_partials_size.restype = sz
    L.qg_plan.argtypes = [vp, P(Operation), P(Layout), P(Layout), P(Layout), P(Layout), P(Layout), P(Layout),
                          ctypes.c_float, ctypes.c_float, P(Workspace), ctypes.c_char_p, sz]
    L.qg_export.argtypes = [vp, ctypes.c_char_p, sz, P(sz)]
    L.qg_import.argtypes = [vp, ctypes.c_char_p, sz]
    L.qg_get_tuning_seq.argtypes = [vp, P(i32), i32, P(i32)]
    L.qg_cache_size.argtypes = [vp, P(i32)]
    L.qg_kernel_count.restype = i32
    L.qg_kernel_name.argtypes = [i32]
    L.qg_kernel_name.restype = ctypes.c_char_p
    L.qg_status_str.argtypes = [i32]
    L.qg_status_str.restype = ctypes.c_char_p
    L.qg_version.restype = ctypes.c_char_p
    L.qg_streamk_units.argtypes = [i32, i32, i32, P(ctypes.c_int32), i32, P(i32)]
    L.qg_streamk_fixup.argtypes = [i32, i32, i32, i32, P(ctypes.c_int32), i32, P(i32)]
    for name in ("qg_create", "qg_destroy", "qg_run", "qg_run_noalloc", "qg_run_timed", "qg_plan", "qg_export",
                 "qg_import",
                 "qg_get_tuning_seq", "qg_cache_size", "qg_streamk_units", "qg_streamk_fixup"):
        getattr(L, name).restype = i32
    return L


lib = _load()


def status_str(status: int) -> str:
    return lib.qg_status_str(int(status)).decode()


def version() -> str:
    return lib.qg_version().decode()


def barriers_size() -> int:
    return int(lib.qg_barriers_size())


def partials_size() -> int:
    return int(lib.qg_partials_size())


def noalloc_barriers_size() -> int:
    return int(lib.qg_noalloc_barriers_size())


def noalloc_partials_size() -> int:
    return int(lib.qg_noalloc_partials_size())


def kernel_names():
    return [lib.qg_kernel_name(i).decode() for i in range(lib.qg_kernel_count())]


def streamk_units(tiles, iters, programs):
    """qg_streamk_units: [(program, tile, k_begin, k_end, slot), ...]."""
    n = ctypes.c_int()
    st = lib.qg_streamk_units(int(tiles), int(iters), int(programs), None, 0, ctypes.byref(n))
    if st not in (OK, ERR_BUFFER_SMALL):
        raise QGemmError(st, "qg_streamk_units")
    buf = (ctypes.c_int32 * (5 * max(n.value, 1)))()
    _check(lib.qg_streamk_units(int(tiles), int(iters), int(programs), buf, n.value, ctypes.byref(n)),
           "qg_streamk_units")
    return [tuple(buf[5 * i:5 * i + 5]) for i in range(n.value)]


def streamk_fixup(tiles, iters, programs, tile):
    """qg_streamk_fixup: partial-piece slots of a shared tile in k order."""
    buf = (ctypes.c_int32 * (programs + 1))()
    n = ctypes.c_int()
    _check(lib.qg_streamk_fixup(int(tiles), int(iters), int(programs), int(tile), buf, programs + 1,
                                ctypes.byref(n)), "qg_streamk_fixup")
    return list(buf[:n.value])


def layout(dtype, rows, cols, ld=None, num=0, offsets=0, stride=0, order=ROW_MAJOR) -> Layout:
    t = DTYPE_CODES[dtype] if isinstance(dtype, str) else int(dtype)
    if ld is None:
        ld = cols // 8 if t == U4 else cols
    return Layout(t, order, int(rows), int(cols), int(ld), int(num), 0, int(offsets or 0), int(stride))


def operation(policy=POLICY_DEFAULT, schedule=SCHED_AUTO, split_k=0, programs=0, kernel=-1,
              quant_a=(QUANT_NONE, 0, 0, 0), quant_b=(QUANT_NONE, 0, 0, 0), epilogue=EPI_ALPHA_BETA,
              bias=None, bias_type="f32", row_scale=None, zero_point=0.0) -> Operation:
    """bias / row_scale: device tensors or raw pointers (kept alive by the caller)."""
    bt = DTYPE_CODES[bias_type] if isinstance(bias_type, str) else int(bias_type)
    epi = EpilogueArgs(_ptr(bias), bt, 0, _ptr(row_scale), float(zero_point), 0)
    return Operation(policy, int(epilogue), Quant(*quant_a), Quant(*quant_b), schedule, split_k, programs, kernel,
                     epi)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _check(st, what):
    if st != OK:
        raise QGemmError(st, what)


class Gemm:
    """One handle per device (qg_create / qg_destroy)."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check(lib.qg_create(ctypes.byref(h)), "qg_create")
        self.h = h

    def close(self):
        if self.h:
            lib.qg_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def run_raw(self, op, alpha, A, Ad, U, Ud, B, Bd, V, Vd, beta, C, Cd, D, Dd, ws, stream=None) -> int:
        """qg_run with explicit descriptors; returns the status code."""
        def r(x):
            return None if x is None else ctypes.byref(x)
        return lib.qg_run(self.h, ctypes.byref(op), float(alpha), _ptr(A), r(Ad), _ptr(U), r(Ud), _ptr(B), r(Bd),
                          _ptr(V), r(Vd), float(beta), _ptr(C), r(Cd), _ptr(D), r(Dd), r(ws),
                          stream if stream is not None else _current_stream())

    def run(self, *args, **kw):
        _check(self.run_raw(*args, **kw), "qg_run")

    def run_noalloc_raw(self, op, alpha, A, Ad, U, Ud, B, Bd, V, Vd, beta, C, Cd, D, Dd, stream=None) -> int:
        """qg_run_noalloc (workspace from the library's own device array); returns the status code."""
        def r(x):
            return None if x is None else ctypes.byref(x)
        return lib.qg_run_noalloc(self.h, ctypes.byref(op), float(alpha), _ptr(A), r(Ad), _ptr(U), r(Ud), _ptr(B),
                                  r(Bd), _ptr(V), r(Vd), float(beta), _ptr(C), r(Cd), _ptr(D), r(Dd),
                                  stream if stream is not None else _current_stream())

    def run_timed_raw(self, op, alpha, A, Ad, U, Ud, B, Bd, V, Vd, beta, C, Cd, D, Dd, ws, stamps, units_cap,
                      stream=None):
        """qg_run_timed: a split-K run that writes 8 timestamps per split-K unit to
        the device buffer `stamps` (units_cap units). Returns (status, units)."""
        def r(x):
            return None if x is None else ctypes.byref(x)
        n = ctypes.c_int64()
        st = lib.qg_run_timed(self.h, ctypes.byref(op), float(alpha), _ptr(A), r(Ad), _ptr(U), r(Ud), _ptr(B),
                              r(Bd), _ptr(V), r(Vd), float(beta), _ptr(C), r(Cd), _ptr(D), r(Dd), r(ws),
                              stream if stream is not None else _current_stream(), _ptr(stamps), int(units_cap),
                              ctypes.byref(n))
        return st, n.value

    def plan(self, op, Ad, Ud, Bd, Vd, Cd, Dd, alpha, beta, ws=None) -> str:
        buf = ctypes.create_string_buffer(512)
        def r(x):
            return None if x is None else ctypes.byref(x)
        _check(lib.qg_plan(self.h, ctypes.byref(op), r(Ad), r(Ud), r(Bd), r(Vd), r(Cd), r(Dd), float(alpha),
                           float(beta), r(ws), buf, 512), "qg_plan")
        return buf.value.decode()

    def export(self) -> str:
        n = ctypes.c_size_t()
        _check(lib.qg_export(self.h, None, 0, ctypes.byref(n)), "qg_export")
        buf = ctypes.create_string_buffer(n.value)
        _check(lib.qg_export(self.h, buf, n.value, ctypes.byref(n)), "qg_export")
        return buf.value.decode()

    def import_(self, text: str) -> int:
        b = text.encode()
        return lib.qg_import(self.h, b, len(b))

    def tuning_seq(self):
        cnt = ctypes.c_int()
        _check(lib.qg_get_tuning_seq(self.h, None, 0, ctypes.byref(cnt)), "qg_get_tuning_seq")
        arr = (ctypes.c_int * cnt.value)()
        _check(lib.qg_get_tuning_seq(self.h, arr, cnt.value, ctypes.byref(cnt)), "qg_get_tuning_seq")
        return list(arr)

    def cache_size(self) -> int:
        n = ctypes.c_int()
        _check(lib.qg_cache_size(self.h, ctypes.byref(n)), "qg_cache_size")
        return n.value


def _current_stream():
    import torch
    if torch.cuda.is_available():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return None


def workspace(device="cuda", barriers=None, partials=None):
    """Allocates a zeroed workspace (torch tensors kept alive by the returned object)."""
    import torch

    class _WS:
        pass

    w = _WS()
    w.barriers = torch.zeros((barriers or barriers_size()) // 4, dtype=torch.int32, device=device)
    w.partials = torch.empty((partials or partials_size()) // 4, dtype=torch.float32, device=device)
    w.desc = Workspace(w.barriers.data_ptr(), w.barriers.numel() * 4, w.partials.data_ptr(), w.partials.numel() * 4)
    return w
