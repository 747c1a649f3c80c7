"""CPU oracle for the GEMM engine -- TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of
`bench.py` may import this package. The product path never does, and this
package imports nothing from the product: it shares no code with the GPU
path. It holds

  * `gemm(problem, rows=None, splits=1)`: the fp64 triple-loop reference in
    `oracle.c` (D = alpha*(A@B) + beta*C, the operation of the page
    "InternLM Lmdeploy Gemm Interface", Description / Run signature),
    returning (ref, absdot) for every requested output;
  * the scalar decoders of that library (bf16, fp16, OCP E4M3).

How work is divided among workgroups (split-K, stream-K) does not change
what is computed, so the oracle has no notion of it beyond the `splits`
self-check (contiguous K chunks summed in fp64, then in order).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")

_DT = {"f32": 0, "f16": 1, "bf16": 2, "e4m3": 3, "i8": 4, "i32": 5, "u4": 6}
Q_NONE, Q_INT4, Q_BLOCK = 0, 1, 2


class _Problem(ctypes.Structure):
    _fields_ = [
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("ta", ctypes.c_int32), ("tb", ctypes.c_int32), ("tc", ctypes.c_int32),
        ("qa", ctypes.c_int32), ("qb", ctypes.c_int32),
        ("A", ctypes.c_void_p), ("lda", ctypes.c_int64),
        ("B", ctypes.c_void_p), ("ldb", ctypes.c_int64),
        ("C", ctypes.c_void_p), ("ldc", ctypes.c_int64),
        ("U", ctypes.c_void_p), ("ldu", ctypes.c_int64),
        ("V", ctypes.c_void_p), ("ldv", ctypes.c_int64),
        ("gm_a", ctypes.c_int32), ("gk_a", ctypes.c_int32),
        ("gn_b", ctypes.c_int32), ("gk_b", ctypes.c_int32),
        ("zero_point", ctypes.c_int32),
        ("alpha", ctypes.c_double), ("beta", ctypes.c_double),
        ("E", ctypes.c_int32), ("offsets", ctypes.c_void_p),
        ("b_batch", ctypes.c_int64), ("v_batch", ctypes.c_int64),
        ("splits", ctypes.c_int32),
        ("epi", ctypes.c_int32), ("bias_type", ctypes.c_int32),
        ("bias", ctypes.c_void_p), ("row_scale", ctypes.c_void_p),
        ("out_zero_point", ctypes.c_double),
    ]


def build(force: bool = False) -> str:
    """Compile oracle.c (plain C, -O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(os.path.join(_HERE, "oracle.c")):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               os.path.join(_HERE, "oracle.c"), "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_SO)
        L.or_gemm.argtypes = [ctypes.POINTER(_Problem), ctypes.c_void_p, ctypes.c_int64,
                              ctypes.c_void_p, ctypes.c_void_p]
        L.or_gemm.restype = ctypes.c_int
        for name, at in (("or_dec_bf16", ctypes.c_uint16), ("or_dec_f16", ctypes.c_uint16),
                         ("or_dec_e4m3", ctypes.c_uint8)):
            f = getattr(L, name)
            f.argtypes = [at]
            f.restype = ctypes.c_double
        L.or_num_threads.restype = ctypes.c_int
        L.or_set_num_threads.argtypes = [ctypes.c_int]
        L.or_set_num_threads.restype = None
        L.or_quant_codes.argtypes = [ctypes.POINTER(_Problem), ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.or_quant_codes.restype = ctypes.c_int
        _lib = L
    return _lib


def num_threads() -> int:
    return int(lib().or_num_threads())


def set_num_threads(n: int) -> None:
    """OpenMP threads of later oracle calls from this thread."""
    lib().or_set_num_threads(int(n))


def dec_bf16(bits: int) -> float:
    return lib().or_dec_bf16(int(bits))


def dec_f16(bits: int) -> float:
    return lib().or_dec_f16(int(bits))


def dec_e4m3(code: int) -> float:
    return lib().or_dec_e4m3(int(code))


def _ptr(a):
    return None if a is None else a.ctypes.data


def _problem(p: dict, splits: int, alpha, beta, keep):
    """Marshals a problem dict into the C struct (arrays appended to `keep`,
    which the caller holds while the struct is in use)."""

    def c(a):
        a = np.ascontiguousarray(a)
        keep.append(a)
        return a

    M, N, K = p["M"], p["N"], p["K"]
    st = _Problem()
    st.M, st.N, st.K = M, N, K
    kind = p["kind"]
    st.ta = _DT[p["in_dtype"]]
    A = c(p["A"])
    st.A, st.lda = _ptr(A), K
    st.alpha = p["alpha"] if alpha is None else alpha
    st.beta = p["beta"] if beta is None else beta
    st.tc = -1
    if p.get("C") is not None:
        C = c(p["C"])
        st.tc = _DT[p["c_dtype"]]
        st.C, st.ldc = _ptr(C), N
    st.splits = max(1, int(splits))
    if kind == "w4a16":
        B, V = c(p["B"]), c(p["V"])
        st.tb, st.qb = _DT["u4"], Q_INT4
        st.B, st.ldb = _ptr(B), K // 8
        st.V, st.ldv = _ptr(V), V.shape[1]
        st.gk_b, st.zero_point = p["group"], p["zero_point"]
        if p.get("Z") is not None:  # per-group zero points
            Z = c(np.asarray(p["Z"], dtype=np.int8))
            st.U, st.ldu = _ptr(Z), Z.shape[1]
    elif kind == "grouped":
        B = c(p["B"])
        off = c(np.asarray(p["offsets"], dtype=np.int32))
        st.E, st.offsets = p["E"], _ptr(off)
        st.tb = _DT[p["in_dtype"]]
        st.B, st.ldb, st.b_batch = _ptr(B), K, N * K
        if p["in_dtype"] == "e4m3":
            U, V = c(p["U"]), c(p["V"])
            st.qa = st.qb = Q_BLOCK
            st.U, st.ldu, st.gm_a, st.gk_a = _ptr(U), U.shape[1], 1, p["group_k"]
            st.V, st.ldv, st.gn_b, st.gk_b = _ptr(V), V.shape[2], p["group_n"], p["group_k"]
            st.v_batch = V.shape[1] * V.shape[2]
    else:
        B = c(p["B"])
        st.tb = _DT[p["in_dtype"]]
        st.B, st.ldb = _ptr(B), K
        if p["in_dtype"] == "e4m3":
            U, V = c(p["U"]), c(p["V"])
            st.qa = st.qb = Q_BLOCK
            st.U, st.ldu, st.gm_a, st.gk_a = _ptr(U), U.shape[1], 1, p["group_k"]
            st.V, st.ldv, st.gn_b, st.gk_b = _ptr(V), V.shape[1], p["group_n"], p["group_k"]
        elif p.get("w8a8"):
            # one scale per row of A and per row of B: 1 x K blocks
            U, V = c(p["U"]), c(p["V"])
            st.qa = st.qb = Q_BLOCK
            st.U, st.ldu, st.gm_a, st.gk_a = _ptr(U), U.shape[1], 1, max(K, 1)
            st.V, st.ldv, st.gn_b, st.gk_b = _ptr(V), V.shape[1], 1, max(K, 1)
    ep = p.get("epilogue")
    if ep:
        st.epi = int(ep["flags"])
        if ep.get("bias") is not None:
            b = c(ep["bias"])
            st.bias, st.bias_type = _ptr(b), _DT[ep["bias_type"]]
        if ep.get("row_scale") is not None:
            rs = c(np.asarray(ep["row_scale"], dtype=np.float32))
            st.row_scale = _ptr(rs)
        st.out_zero_point = float(ep.get("zero_point", 0.0))
    return st


def gemm(p: dict, rows=None, splits: int = 1, alpha=None, beta=None):
    """fp64 reference for a problem dict built by `synth` (epilogue steps
    included when p["epilogue"] is set; quantisation is quant_codes).

    Returns (ref, absdot), float64 arrays of shape [len(rows) or M, N].
    `alpha` / `beta` override the problem's own values."""
    keep = []

    def c(a):
        a = np.ascontiguousarray(a)
        keep.append(a)
        return a

    M, N = p["M"], p["N"]
    st = _problem(p, splits, alpha, beta, keep)
    if rows is None:
        n = M
        rp = None
    else:
        r = c(np.asarray(rows, dtype=np.int64))
        n = len(r)
        rp = _ptr(r)
    ref = np.empty((n, N), dtype=np.float64)
    absdot = np.empty((n, N), dtype=np.float64)
    rc = lib().or_gemm(ctypes.byref(st), rp, n, ref.ctypes.data, absdot.ctypes.data)
    if rc != 0:
        raise ValueError("oracle rejected the problem")
    return ref, absdot


def quant_codes(p: dict, ref, rows=None):
    """Output quantisation of oracle outputs `ref` (rows as passed to gemm):
    returns (pre, code) with pre = ref * row_scale + zero_point (fp64) and code
    its saturated round-half-even int8 value."""
    keep = []
    st = _problem(p, 1, None, None, keep)
    ref = np.ascontiguousarray(ref, dtype=np.float64)
    if rows is None:
        rp, n = None, p["M"]
    else:
        r = np.asarray(rows, dtype=np.int64)
        keep.append(r)
        rp, n = _ptr(r), len(r)
    pre = np.empty_like(ref)
    code = np.empty(ref.shape, dtype=np.int32)
    if lib().or_quant_codes(ctypes.byref(st), rp, n, ref.ctypes.data, pre.ctypes.data, code.ctypes.data) != 0:
        raise ValueError("oracle rejected the problem")
    return pre, code

