"""GPU parity of the int8 w8a8 path (int8 A and B with one fp32 scale per row of
A and per row of B; exact int32 sums, then the float epilogue) against the fp64
oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import quantized_gemm_bf16_amd as qg
import synth
from tests.gpu_util import Run, check_against_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    assert torch.cuda.is_available()
    return qg.Gemm()


@pytest.fixture(scope="module")
def ws():
    return qg.workspace()


def kidx(name):
    return qg.kernel_names().index(name)


@pytest.mark.parametrize("kname", [None, "tile_I8_256x256x128b_w2x4_s2", "tile_I8_128x128x128b_w2x2_s4",
                                   "skinny_I8_1x16x32x256b_w4_d3_n0"])
@pytest.mark.parametrize("sched", ["dp", "split3", "streamk"])
def test_kernels_and_schedules(g, ws, kname, sched):
    M = 16 if kname and kname.startswith("skinny") else 200
    p = synth.w8a8_problem(M, 300, 528, out_dtype="bf16", c_dtype="bf16", alpha=0.5, beta=1.0, seed=M + 1)
    r = Run(g, p, ws)
    kw = {} if kname is None else dict(policy=qg.POLICY_FORCE, kernel=kidx(kname))
    if sched == "split3":
        kw.update(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=3)
    elif sched == "streamk":
        kw.update(policy=qg.POLICY_FORCE, schedule=qg.SCHED_STREAMK, programs=23)
    op = r.op(**kw)
    print(kname, sched, r.plan(op), flush=True)
    D = r.run(op)
    check_against_oracle(p, D, what=f"w8a8 {kname} {sched}")
    assert int(ws.barriers.abs().sum().item()) == 0
    assert np.array_equal(D, r.run(op))


@pytest.mark.parametrize("out", ["f32", "f16"])
def test_output_types_and_square(g, ws, out):
    p = synth.w8a8_problem(1024, 1024, 2048, out_dtype=out, c_dtype="f32", beta=-1.0, seed=5)
    r = Run(g, p, ws)
    print(r.plan(), flush=True)
    check_against_oracle(p, r.run(), what=f"w8a8 1024^2x2048 -> {out}")


def test_with_fused_epilogue(g, ws):
    p = synth.w8a8_problem(64, 256, 512, out_dtype="bf16", seed=6)
    bias = torch.linspace(-1, 1, 256, device="cuda")
    p_ref = dict(p, epilogue=dict(flags=qg.EPI_BIAS | qg.EPI_RELU, bias=bias.cpu().numpy(), bias_type="f32"))
    r = Run(g, p, ws)
    D = r.run(r.op(epilogue=qg.EPI_BIAS | qg.EPI_RELU, bias=bias, bias_type="f32"))
    check_against_oracle(p_ref, D, what="w8a8 + bias + relu")
