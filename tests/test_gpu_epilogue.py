"""GPU parity of the fused epilogue (bias, ReLU / GELU, per-row int8 output
quantisation) against the fp64 oracle, through the C ABI, on every kernel
family and schedule that ends in the shared epilogue."""
import numpy as np
import pytest
import torch

import oracle
import quantized_gemm_bf16_amd as qg
import synth
from tests import tolerance
from tests.gpu_util import Run, decode_c, dev

pytestmark = pytest.mark.gpu

BIAS, RELU, GELU, QUANT = qg.EPI_BIAS, qg.EPI_RELU, qg.EPI_GELU, qg.EPI_QUANT_I8


@pytest.fixture(scope="module")
def g():
    assert torch.cuda.is_available()
    return qg.Gemm()


@pytest.fixture(scope="module")
def ws():
    return qg.workspace()


def kidx(name):
    return qg.kernel_names().index(name)


def bias_values(N, bias_type, seed):
    b = synth.uniform((N,), -1.5, 1.5, seed)
    if bias_type == "f32":
        return b.astype(np.float32), b.astype(np.float64)
    bits = synth.to_storage(b, bias_type)
    return bits, oracle_decode(bits, bias_type)


def oracle_decode(bits, t):
    if t == "bf16":
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    return bits.view(np.float16).astype(np.float64)


def run_epilogue(g, ws, p, flags, bias_type="f32", sched=None, kname=None, rows=None, seed=3):
    N, M = p["N"], p["M"]
    bias_store, bias_f64 = bias_values(N, bias_type, seed) if flags & BIAS else (None, None)
    row_scale = synth.uniform((M,), 0.5, 4.0, seed + 1).astype(np.float32) if flags & QUANT else None
    zp = 3.0 if flags & QUANT else 0.0
    p = dict(p, epilogue=dict(flags=flags, bias=bias_store, bias_type=bias_type, row_scale=row_scale,
                              zero_point=zp))
    out = "i8" if flags & QUANT else p["out_dtype"]
    r = Run(g, p, ws, out_dtype=out)
    bias_dev = dev(bias_store) if bias_store is not None else None
    rs_dev = dev(row_scale) if row_scale is not None else None
    kw = dict(epilogue=flags, bias=bias_dev, bias_type=bias_type, row_scale=rs_dev, zero_point=zp)
    if kname is not None:
        kw.update(policy=qg.POLICY_FORCE, kernel=kidx(kname))
    if sched == "split3":
        kw.update(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=3)
    elif sched == "streamk":
        kw.update(policy=qg.POLICY_FORCE, schedule=qg.SCHED_STREAMK, programs=19)
    op = r.op(**kw)
    print(p["M"], p["N"], p["K"], flags, r.plan(op), flush=True)
    D = r.run(op)
    ref, absdot = oracle.gemm(p, rows=rows)
    Dsel = D if rows is None else D[np.asarray(rows)]
    c = decode_c(p)
    if c is not None and rows is not None:
        c = c[np.asarray(rows)]
    if flags & QUANT:
        pre, code = oracle.quant_codes(p, ref, rows=rows)
        xtol = tolerance.bound_epilogue(ref, absdot, ref, p["alpha"], p["beta"], c, bias_f64, flags, "f32")
        scales = row_scale if rows is None else row_scale[np.asarray(rows)]
        ndiff = tolerance.check_codes(Dsel, pre, code, xtol, scales, what=f"codes flags={flags}")
        print("codes differing at a rounding boundary:", ndiff, flush=True)
    else:
        tolerance.check_epilogue(Dsel, ref, absdot, p["alpha"], p["beta"], c, bias_f64, flags, out,
                                 what=f"flags={flags}")
    return D


@pytest.mark.parametrize("flags", [BIAS, RELU, GELU, BIAS | RELU, BIAS | GELU, QUANT, BIAS | GELU | QUANT])
@pytest.mark.parametrize("kname", ["tile_BF16_256x256x128b_w2x4_s2", "tile_BF16_128x128x128b_w2x2_s4"])
def test_tile_kernels(g, ws, flags, kname):
    p = synth.dense_problem(300, 264, 200, "bf16", "bf16", c_dtype="bf16", alpha=0.5, beta=1.0, seed=41)
    run_epilogue(g, ws, p, flags, kname=kname)


@pytest.mark.parametrize("sched", ["split3", "streamk"])
@pytest.mark.parametrize("flags", [BIAS | GELU, BIAS | RELU | QUANT])
def test_split_schedules_apply_epilogue_once(g, ws, sched, flags):
    p = synth.dense_problem(160, 384, 1536, "f16", "f32", c_dtype="f32", alpha=1.0, beta=-0.5, seed=43)
    run_epilogue(g, ws, p, flags, bias_type="f16", sched=sched)


@pytest.mark.parametrize("flags", [BIAS | GELU, BIAS | QUANT])
def test_decode_skinny(g, ws, flags):
    p = synth.config_decode(M=16, N=1024, K=4096)
    run_epilogue(g, ws, p, flags, bias_type="bf16", sched="split3")


@pytest.mark.parametrize("flags", [BIAS | RELU, GELU | QUANT])
def test_w4a16_and_fp8(g, ws, flags):
    p = synth.w4a16_problem(32, 512, 1024, seed=45)
    run_epilogue(g, ws, p, flags)
    q = synth.dense_fp8_problem(96, 384, 640, seed=46)
    run_epilogue(g, ws, q, flags)


def test_grouped_moe_rows(g, ws):
    counts = np.array([5, 0, 300, 1, 129], dtype=np.int32)
    p = synth.grouped_problem(counts, 256, 384, seed=47)
    run_epilogue(g, ws, p, BIAS | GELU)
    run_epilogue(g, ws, p, BIAS | QUANT)


def test_invalid_epilogues(g, ws):
    p = synth.dense_problem(64, 64, 64, "bf16", "bf16", seed=48)
    r = Run(g, p, ws)
    bias = torch.zeros(64, device="cuda")
    assert r.launch(r.op(epilogue=RELU | GELU)) == qg.ERR_INVALID_ARG
    assert r.launch(r.op(epilogue=BIAS)) == qg.ERR_INVALID_ARG                       # no bias pointer
    assert r.launch(r.op(epilogue=BIAS, bias=bias, bias_type="i8")) == qg.ERR_UNSUPPORTED
    assert r.launch(r.op(epilogue=QUANT)) == qg.ERR_INVALID_ARG                      # no row scales
    # quantised codes need an int8 D, and an int8 D needs quantisation
    assert r.launch(r.op(epilogue=QUANT, row_scale=bias)) == qg.ERR_UNSUPPORTED
    assert r.launch(r.op(epilogue=1 << 6)) == qg.ERR_INVALID_ARG
