"""Pass rule for float paths of the GEMM engine.

|D - ref| <= 2^-10 * |alpha| * absdot + 2^-8 * |beta * c| + ulp_out(max(|ref|, |D|))

ref and absdot = sum_k |a_ik * b_kj| come from the fp64 oracle; ulp_out is the
spacing of the output format at the larger of |ref| and |D| (p = 8 bf16,
11 fp16, 24 fp32; e_min = -126 bf16 / fp32, -14 fp16). The int8 -> int32
path must be bit-exact instead.
"""
import numpy as np

_FMT = {"bf16": (8, -126), "f16": (11, -14), "f32": (24, -126)}


def ulp_out(m, dtype):
    p, emin = _FMT[dtype]
    m = np.asarray(m, dtype=np.float64)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(m > 0, m, 1.0)))
    e = np.where(m > 0, np.maximum(e, emin), emin)
    return np.ldexp(1.0, (e - p + 1).astype(np.int64))


def bound(ref, absdot, D, alpha, beta, c, dtype):
    cterm = 0.0 if (beta == 0 or c is None) else np.abs(beta * np.asarray(c, dtype=np.float64))
    m = np.maximum(np.abs(ref), np.abs(D))
    return 2.0 ** -10 * abs(alpha) * absdot + 2.0 ** -8 * cterm + ulp_out(m, dtype)


def check(D, ref, absdot, alpha, beta, c, dtype, what=""):
    """Raise AssertionError naming the worst element when the bound fails."""
    D = np.asarray(D, dtype=np.float64)
    b = bound(ref, absdot, D, alpha, beta, c, dtype)
    err = np.abs(D - ref)
    bad = ~(err <= b)
    if bad.any():
        idx = np.unravel_index(np.argmax(np.where(bad, err / np.where(b > 0, b, 1e-300), -1)), D.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {D.size} outside tolerance; worst at {idx}: "
            f"D={D[idx]!r} ref={ref[idx]!r} err={err[idx]:.3e} bound={b[idx]:.3e}")
    return float((err / b).max()) if D.size else 0.0


# ---------------------------------------------------------------- fused epilogue
# Bias and ReLU are 1-Lipschitz and GELU (x * Phi(x)) is at most 1.13-Lipschitz,
# so the pre-activation bound carries over scaled by L; the fp32 bias add and
# the fp32 erf add a few ulps of the value itself (2^-20 relative margin).
GELU_LIPSCHITZ = 1.13


def bound_epilogue(ref, absdot, D, alpha, beta, c, bias_row, flags, dtype):
    L = GELU_LIPSCHITZ if flags & 4 else 1.0
    cterm = 0.0 if (beta == 0 or c is None) else np.abs(beta * np.asarray(c, dtype=np.float64))
    bterm = 0.0 if bias_row is None else np.abs(bias_row)[None, :]
    m = np.maximum(np.abs(ref), np.abs(D))
    pre = 2.0 ** -10 * abs(alpha) * absdot + 2.0 ** -8 * cterm
    return L * pre + 2.0 ** -20 * (m + bterm) + ulp_out(m, dtype)


def check_epilogue(D, ref, absdot, alpha, beta, c, bias_row, flags, dtype, what=""):
    D = np.asarray(D, dtype=np.float64)
    b = bound_epilogue(ref, absdot, D, alpha, beta, c, bias_row, flags, dtype)
    err = np.abs(D - ref)
    bad = ~(err <= b)
    if bad.any():
        idx = np.unravel_index(np.argmax(np.where(bad, err / np.where(b > 0, b, 1e-300), -1)), D.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {D.size} outside tolerance; worst at {idx}: "
            f"D={D[idx]!r} ref={ref[idx]!r} err={err[idx]:.3e} bound={b[idx]:.3e}")


def check_codes(code_gpu, pre, code_ref, xtol, scale_rows, what=""):
    """int8 output codes: equal to the oracle's code, except where the oracle's
    unrounded value pre = x * s + zp lies within the kernel's possible error
    (xtol * |s| on x, plus fp32 rounding of the fma) of a rounding boundary;
    there either neighbouring (saturated) code is accepted."""
    code_gpu = np.asarray(code_gpu).astype(np.int64)
    code_ref = np.asarray(code_ref).astype(np.int64)
    margin = xtol * np.abs(scale_rows)[:, None] + 2.0 ** -22 * np.abs(pre) + 1e-6
    lo = np.clip(np.rint(pre - margin), -128, 127)
    hi = np.clip(np.rint(pre + margin), -128, 127)
    ok = (code_gpu == code_ref) | ((code_gpu >= lo) & (code_gpu <= hi))
    if not ok.all():
        idx = np.unravel_index(np.argmin(ok), ok.shape)
        raise AssertionError(f"{what}: {int((~ok).sum())} codes differ; at {idx}: gpu={code_gpu[idx]} "
                             f"ref={code_ref[idx]} pre={pre[idx]!r} margin={margin[idx]:.3e}")
    return int((code_gpu != code_ref).sum())
