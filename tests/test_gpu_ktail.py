"""GPU parity when K * element size is not a multiple of 16 bytes: the last
16-byte chunk of every A and B row is only partly inside K. The rows are
stored with a pitch ld > K whose padding holds NaN codes (bf16 / fp16 / e4m3)
or extreme int8 values, so a padding byte that reached an MFMA would show in
the result. Every kernel family and schedule is run against the fp64 oracle,
with the straddling chunk in the first k-tile, in a middle one and in the
last k-tile of a split."""
import numpy as np
import pytest
import torch

import quantized_gemm_bf16_amd as qg
import synth
from tests.gpu_util import Run, check_against_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return qg.Gemm()


@pytest.fixture(scope="module")
def ws():
    return qg.workspace()


def kidx(name):
    return qg.kernel_names().index(name)


def ops_for(r, kname, scheds):
    out = []
    for s in scheds:
        if s == "dp":
            out.append((s, r.op(policy=qg.POLICY_FORCE, schedule=qg.SCHED_DP, kernel=kidx(kname))))
        elif s == "split3":
            out.append((s, r.op(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=3, kernel=kidx(kname))))
        else:
            out.append((s, r.op(policy=qg.POLICY_FORCE, schedule=qg.SCHED_STREAMK, programs=37, kernel=kidx(kname))))
    return out


def check_runs(g, ws, p, ldk, kname, scheds):
    r = Run(g, p, ws, ldk=ldk)
    first = None
    for s, op in ops_for(r, kname, scheds):
        print(kname, p["M"], p["N"], p["K"], ldk, s, r.plan(op), flush=True)
        D = r.run(op)
        check_against_oracle(p, D, what=f"{kname} K={p['K']} ld={ldk} {s}")
        assert int(ws.barriers.abs().sum().item()) == 0
        if first is None:
            first = D
    return first


_TILE16 = [n for n in qg.kernel_names() if n.startswith(("tile_BF16_", "tile_F16_"))]
_TILE8 = [n for n in qg.kernel_names() if n.startswith("tile_I8_")]
_SKINNY16 = [n for n in qg.kernel_names() if n.startswith(("skinny_BF16_", "skinny_F16_"))]
_SKINNY8 = [n for n in qg.kernel_names() if n.startswith("skinny_I8_")]
_F8 = [n for n in qg.kernel_names() if n.startswith("f8_")]


# (M, N, K, ld): K = 6 lies inside the first chunk of the first k-tile;
# K = 100 ends in the second k-tile of 64 elements; K = 1002 in a late one
@pytest.mark.parametrize("kname", _TILE16)
@pytest.mark.parametrize("shape", [(70, 130, 6, 8), (200, 300, 100, 104), (257, 129, 1002, 1008)])
def test_tile_16bit(g, ws, kname, shape):
    M, N, K, ld = shape
    ind = "f16" if kname.startswith("tile_F16_") else "bf16"
    p = synth.dense_problem(M, N, K, ind, "bf16", c_dtype="f32", alpha=0.75, beta=-0.5, dist="uniform", seed=K + M)
    scheds = ["dp", "split3", "streamk"] if K > 512 else ["dp"]
    check_runs(g, ws, p, ld, kname, scheds)


@pytest.mark.parametrize("kname", _TILE8)
@pytest.mark.parametrize("shape", [(65, 70, 1, 16), (200, 300, 40, 48), (130, 257, 1001, 1008)])
def test_tile_int8_exact(g, ws, kname, shape):
    M, N, K, ld = shape
    p = synth.dense_problem(M, N, K, "i8", "i32", c_dtype="i32", alpha=1.0, beta=1.0, seed=K + N)
    scheds = ["dp", "split3", "streamk"] if K > 512 else ["dp"]
    check_runs(g, ws, p, ld, kname, scheds)


def test_w8a8(g, ws):
    p = synth.w8a8_problem(150, 260, 1001, out_dtype="bf16", c_dtype="bf16", alpha=1.0, beta=0.5, seed=5)
    for kname in ("tile_I8_128x128x128b_w2x2_s4", "tile_I8_32x128x128b_w1x4_s4"):
        check_runs(g, ws, p, 1008, kname, ["dp", "split3"])


@pytest.mark.parametrize("kname", _SKINNY16)
@pytest.mark.parametrize("shape", [(1, 130, 6, 8), (5, 200, 1002, 1008), (16, 1000, 4100, 4104)])
def test_skinny_16bit(g, ws, kname, shape):
    M, N, K, ld = shape
    if "_2x16x" in kname:
        M += 16
    ind = "f16" if kname.startswith("skinny_F16_") else "bf16"
    p = synth.dense_problem(M, N, K, ind, ind, c_dtype=ind, alpha=1.0, beta=1.0, a_std=0.02, b_std=0.02, seed=N + K)
    scheds = ["dp", "split3", "streamk"] if K > 512 else ["dp"]
    D = check_runs(g, ws, p, ld, kname, scheds)
    assert not np.isnan(D).any()


@pytest.mark.parametrize("kname", _SKINNY8)
@pytest.mark.parametrize("shape", [(3, 100, 1, 16), (16, 700, 1001, 1008)])
def test_skinny_int8_exact(g, ws, kname, shape):
    M, N, K, ld = shape
    p = synth.dense_problem(M, N, K, "i8", "i32", c_dtype="i32", alpha=1.0, beta=1.0, seed=M + K)
    scheds = ["dp", "split3", "streamk"] if K > 512 else ["dp"]
    check_runs(g, ws, p, ld, kname, scheds)


@pytest.mark.parametrize("kname", _F8)
@pytest.mark.parametrize("shape", [(70, 260, 40, 48), (200, 300, 1001, 1008)])
def test_fp8(g, ws, kname, shape):
    M, N, K, ld = shape
    p = synth.dense_fp8_problem(M, N, K, out_dtype="bf16", c_dtype="bf16", alpha=1.0, beta=0.5, seed=K)
    scheds = ["dp", "split3", "streamk"] if K > 512 else ["dp"]
    check_runs(g, ws, p, ld, kname, scheds)


@pytest.mark.parametrize("fp8", [False, True])
def test_grouped(g, ws, fp8):
    counts = [0, 37, 300, 1, 0, 129]
    p = synth.grouped_problem(counts, 264, 1001 if fp8 else 1002, fp8=fp8, seed=17)
    r = Run(g, p, ws, ldk=1008)
    print("grouped fp8" if fp8 else "grouped bf16", r.plan(), flush=True)
    check_against_oracle(p, r.run(), what=f"grouped K={p['K']} ld=1008 fp8={fp8}")


@pytest.mark.parametrize("M, sched", [(16, "split8"), (1, "streamk256")])
def test_decode_shape_default_kernel(g, ws, M, sched):
    # the decode shape with K = 14330: the last chunk of a bf16 row holds 4
    # bytes of K and 12 of padding; default kernel choice, every output
    p = synth.dense_problem(M, 4096, 14330, "bf16", "bf16", c_dtype="bf16", alpha=1.0, beta=1.0, a_std=0.02,
                            b_std=0.02, seed=23)
    r = Run(g, p, ws, ldk=14336)
    if sched == "split8":
        op = r.op(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=8)
    else:
        op = r.op(policy=qg.POLICY_FORCE, schedule=qg.SCHED_STREAMK, programs=256)
    print(M, sched, r.plan(op), flush=True)
    check_against_oracle(p, r.run(op), what=f"decode M={M} K=14330 {sched}")
    assert int(ws.barriers.abs().sum().item()) == 0
