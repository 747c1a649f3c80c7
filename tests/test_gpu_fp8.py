"""GPU parity of the block-scaled fp8 path (e4m3 A and B; fp32 scales per
1 x 128 block of A and per 128 x 128 block of B) against the fp64 oracle,
through the C ABI."""
import numpy as np
import pytest
import torch

import quantized_gemm_bf16_amd as qg
import synth
from tests.gpu_util import Run, check_against_oracle

pytestmark = pytest.mark.gpu

F8 = ["f8_E4M3_128x256_w2x4_s3", "f8_E4M3_256x128_w4x2_s3", "f8_E4M3_64x256_w1x4_s3"]


@pytest.fixture(scope="module")
def g():
    assert torch.cuda.is_available()
    return qg.Gemm()


@pytest.fixture(scope="module")
def ws():
    return qg.workspace()


def kidx(name):
    return qg.kernel_names().index(name)


def forced(r, kname, sched):
    if sched == "dp":
        return r.op(policy=qg.POLICY_FORCE, schedule=qg.SCHED_DP, kernel=kidx(kname))
    if sched == "split3":
        return r.op(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=3, kernel=kidx(kname))
    return r.op(policy=qg.POLICY_FORCE, schedule=qg.SCHED_STREAMK, programs=13, kernel=kidx(kname))


@pytest.mark.parametrize("kname", F8)
@pytest.mark.parametrize("shape", [(1, 128, 128), (70, 300, 400), (130, 520, 1040), (256, 256, 2048), (300, 136, 272)])
@pytest.mark.parametrize("sched", ["dp", "split3", "streamk"])
def test_dense_ragged(g, ws, kname, shape, sched):
    M, N, K = shape
    p = synth.dense_fp8_problem(M, N, K, seed=M + 3 * N + K)
    r = Run(g, p, ws)
    op = forced(r, kname, sched)
    print(kname, shape, sched, r.plan(op), flush=True)
    D1 = r.run(op)
    check_against_oracle(p, D1, what=f"{kname} {shape} {sched}")
    assert int(ws.barriers.abs().sum().item()) == 0
    assert np.array_equal(D1, r.run(op))


@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
def test_alpha_beta_and_output_types(g, ws, out):
    p = synth.dense_fp8_problem(96, 384, 640, out_dtype=out, c_dtype="f32", alpha=0.75, beta=-1.25, seed=5)
    r = Run(g, p, ws)
    print(r.plan(), flush=True)
    check_against_oracle(p, r.run(), what=f"fp8 alpha/beta -> {out}")


def test_default_dispatch_square(g, ws):
    p = synth.dense_fp8_problem(512, 512, 1024, seed=6)
    r = Run(g, p, ws)
    desc = r.plan()
    print(desc, flush=True)
    assert desc.startswith("kernel=f8_E4M3_")
    check_against_oracle(p, r.run(), what="fp8 512x512x1024 default")


def test_zero_scales_and_extreme_codes(g, ws):
    # codes at +-448 (0x7E / 0xFE), the smallest subnormal (0x01), zero scales in some blocks
    M, N, K = 64, 256, 384
    p = synth.dense_fp8_problem(M, N, K, seed=8)
    A, B = p["A"].copy(), p["B"].copy()
    A[:, ::7] = 0x7E
    A[:, 3::11] = 0x01
    B[:, ::5] = 0xFE
    B[:, 2::13] = 0x81
    U, V = p["U"].copy(), p["V"].copy()
    U[5, 1] = 0.0
    V[1, 2] = 0.0
    p.update(A=A, B=B, U=U, V=V)
    r = Run(g, p, ws)
    for kname in F8:
        check_against_oracle(p, r.run(r.op(policy=qg.POLICY_FORCE, kernel=kidx(kname))), what=f"fp8 extremes {kname}")


@pytest.mark.parametrize("kname", F8)
def test_grouped_small_with_empty_experts(g, ws, kname):
    counts = np.array([5, 0, 300, 1, 0, 129, 256, 0], dtype=np.int32)
    p = synth.grouped_problem(counts, 384, 256, fp8=True, seed=19)
    r = Run(g, p, ws)
    op = r.op(policy=qg.POLICY_FORCE, kernel=kidx(kname))
    print(kname, r.plan(op), flush=True)
    check_against_oracle(p, r.run(op), what=f"grouped fp8 {kname}")


def test_grouped_ragged_k_and_n(g, ws):
    counts = np.array([0, 77, 1, 200, 0, 64], dtype=np.int32)
    p = synth.grouped_problem(counts, 200, 400, fp8=True, seed=23)
    r = Run(g, p, ws)
    print(r.plan(), flush=True)
    check_against_oracle(p, r.run(), what="grouped fp8 N=200 K=400")
