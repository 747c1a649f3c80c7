"""GPU parity of the weight-only int4 path (A bf16, B u4 + fp16 group scales)
against the fp64 oracle, through the C ABI."""
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


def test_config_full_size_every_output(g, ws):
    p = synth.config_w4a16()
    r = Run(g, p, ws)
    print(r.plan(), flush=True)
    D = r.run()
    check_against_oracle(p, D, what="W4A16 64x8192x8192")


@pytest.mark.parametrize("kname", ["w4_BF16_64x256_w8_s4", "w4_BF16_32x256_w8_s4"])
@pytest.mark.parametrize("shape", [(1, 256, 128), (5, 300, 384), (33, 520, 1024), (64, 256, 2048), (100, 264, 640)])
@pytest.mark.parametrize("sched", ["dp", "split3", "streamk"])
def test_ragged(g, ws, kname, shape, sched):
    M, N, K = shape
    p = synth.w4a16_problem(M, N, K, seed=M + N + K)
    r = Run(g, p, ws)
    if sched == "dp":
        op = r.op(policy=qg.POLICY_FORCE, schedule=qg.SCHED_DP, kernel=kidx(kname))
    elif sched == "split3":
        op = r.op(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=3, kernel=kidx(kname))
    else:
        op = r.op(policy=qg.POLICY_FORCE, schedule=qg.SCHED_STREAMK, programs=11, kernel=kidx(kname))
    print(kname, shape, sched, r.plan(op), flush=True)
    D1 = r.run(op)
    check_against_oracle(p, D1, what=f"{kname} {shape} {sched}")
    assert int(ws.barriers.abs().sum().item()) == 0
    assert np.array_equal(D1, r.run(op))


@pytest.mark.parametrize("zp", [0, 15])
def test_zero_points_and_beta(g, ws, zp):
    p = synth.w4a16_problem(48, 512, 768, seed=9, zero_point=zp)
    p["C"] = synth.to_bf16_bits(synth.uniform((48, 512), -1, 1, 10))
    p["c_dtype"], p["beta"], p["alpha"] = "bf16", 0.5, 2.0
    p["out_dtype"] = "f32"
    check_against_oracle(p, Run(g, p, ws).run(), what=f"W4A16 zp={zp}")


@pytest.mark.parametrize("kname", ["w4_BF16_64x256_w8_s4", "w4_BF16_32x256_w8_s4"])
@pytest.mark.parametrize("sched", ["dp", "split3"])
def test_asymmetric_per_group_zero_points(g, ws, kname, sched):
    p = synth.w4a16_problem(40, 520, 1024, seed=31, asym=True)
    r = Run(g, p, ws)
    if sched == "dp":
        op = r.op(policy=qg.POLICY_FORCE, schedule=qg.SCHED_DP, kernel=kidx(kname))
    else:
        op = r.op(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=3, kernel=kidx(kname))
    print(kname, sched, r.plan(op), flush=True)
    check_against_oracle(p, r.run(op), what=f"asym int4 {kname} {sched}")


def test_asymmetric_full_size_every_output(g, ws):
    p = synth.w4a16_problem(64, 8192, 8192, asym=True)
    r = Run(g, p, ws)
    check_against_oracle(p, r.run(), what="asym W4A16 64x8192x8192")
