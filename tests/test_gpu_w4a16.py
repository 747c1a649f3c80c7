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


W4_KERNELS = [n for n in qg.kernel_names() if n.startswith("w4_BF16_")]


def test_config_full_size_every_output(g, ws):
    p = synth.config_w4a16()
    r = Run(g, p, ws)
    print(r.plan(), flush=True)
    D = r.run()
    check_against_oracle(p, D, what="W4A16 64x8192x8192")


@pytest.mark.parametrize("kname", W4_KERNELS)
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


@pytest.mark.parametrize("kname", W4_KERNELS)
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


@pytest.mark.parametrize("asym", [False, True], ids=["sym", "asym"])
@pytest.mark.parametrize("sched", ["dp", "split3"])
def test_zero_point_columns_are_exact(g, ws, asym, sched):
    # columns whose nibbles all equal their zero point dequantise to zero
    # weights: the result must be exactly 0 there (the oracle's ref is 0 and
    # absdot is 0, so the bound leaves one ulp of |D| only); columns with
    # single such groups stay within the bound
    M, N, K = 40, 300, 1280
    cols = [0, 17, 128, 255, 299]
    groups = [(5, 0), (5, 9), (40, 3), (130, 7), (200, 1), (201, 2), (202, 3)]
    p = synth.w4a16_problem(M, N, K, seed=61, asym=asym, zp_cols=cols, zp_groups=groups)
    p["out_dtype"] = "f32"
    r = Run(g, p, ws)
    for kname in W4_KERNELS:
        if sched == "dp":
            op = r.op(policy=qg.POLICY_FORCE, schedule=qg.SCHED_DP, kernel=kidx(kname))
        else:
            op = r.op(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=3, kernel=kidx(kname))
        D = r.run(op)
        assert np.all(D[:, cols] == 0.0), f"{kname}: zero-point columns not exactly 0"
        check_against_oracle(p, D, what=f"{kname} zero-point groups {sched}")


@pytest.mark.parametrize("asym", [False, True], ids=["sym", "asym"])
@pytest.mark.parametrize("K", [128, 384, 1152])
def test_odd_group_count_ignores_scale_padding(g, ws, K, asym):
    # an odd number of 128-deep groups leaves the second group of the last
    # k-tile past K; its scale slot holds the row padding, poisoned here with
    # fp16 NaN, which must not reach the result (nor may the zero-point
    # padding, poisoned with 0x7F bytes, in the asymmetric case)
    p = synth.w4a16_problem(33, 264, K, seed=K + 7, asym=asym)
    r = Run(g, p, ws)
    G = K // 128
    assert r.ldv > G
    r.V[:, G:] = 0x7E00  # fp16 quiet NaN bit pattern (the device tensor holds int16 bits)
    if asym:
        assert r.U.shape[1] > G
        r.U[:, G:] = 0x7F
    for kname in W4_KERNELS:
        for op in (r.op(policy=qg.POLICY_FORCE, schedule=qg.SCHED_DP, kernel=kidx(kname)),
                   r.op(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=3, kernel=kidx(kname)),
                   r.op(policy=qg.POLICY_FORCE, schedule=qg.SCHED_STREAMK, programs=5, kernel=kidx(kname))):
            check_against_oracle(p, r.run(op), what=f"{kname} K={K} asym={asym} {r.plan(op)}")
