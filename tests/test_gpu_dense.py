"""GPU parity of the dense paths (bf16 / fp16 / int8) against the fp64 oracle,
called through the C ABI. Sizes span several tiles with ragged tails; the
full-size dense workloads are checked on every output."""
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


def test_tiny_config(g, ws):
    p = synth.config_tiny()
    r = Run(g, p, ws)
    print("plan:", r.plan(), flush=True)
    D = r.run()
    check_against_oracle(p, D, what="256^3 bf16 alpha 1.5 beta 0.5 fp32 out")


@pytest.mark.parametrize("kname", ["tile_BF16_256x256x128b_w2x4_s2", "tile_BF16_128x128x128b_w2x2_s4",
                                   "tile_BF16_32x128x128b_w1x4_s4", "tile_BF16_32x64x128b_w1x2_s6"])
@pytest.mark.parametrize("shape", [(300, 200, 136), (257, 513, 264), (64, 64, 64), (33, 1000, 72), (1, 130, 8)])
def test_ragged_each_kernel(g, ws, kname, shape):
    M, N, K = shape
    p = synth.dense_problem(M, N, K, "bf16", "bf16", c_dtype="f32", alpha=0.75, beta=-1.25, dist="uniform", seed=M + N + K)
    r = Run(g, p, ws)
    op = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_DP, kernel=kidx(kname))
    print(kname, shape, r.plan(op), flush=True)
    check_against_oracle(p, r.run(op), what=f"{kname} {shape}")


_TILES_16 = [n for n in qg.kernel_names() if n.startswith(("tile_BF16_", "tile_F16_"))]


@pytest.mark.parametrize("kname", _TILES_16)
@pytest.mark.parametrize("shape", [(300, 200, 136), (257, 517, 264), (33, 1001, 72), (1, 130, 8)])
@pytest.mark.parametrize("out", ["bf16", "f16"])
def test_staged_epilogue_ragged(g, ws, kname, shape, out):
    # 16-bit D with no C and no fused steps leaves through the LDS-staged
    # row-segment store: ragged M and N tails (N % 8 != 0 takes the per-element
    # end of a row), and nothing written past column N (checked by Run.run)
    M, N, K = shape
    ind = "f16" if kname.startswith("tile_F16_") else "bf16"
    p = synth.dense_problem(M, N, K, ind, out, c_dtype=None, alpha=0.75, beta=0.0, dist="uniform", seed=M + 2 * N + K)
    r = Run(g, p, ws)
    op = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_DP, kernel=kidx(kname))
    print(kname, shape, out, r.plan(op), flush=True)
    check_against_oracle(p, r.run(op), what=f"{kname} {shape} {out}")


@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("cdt", [None, "f32", "bf16", "f16"])
def test_output_and_c_types(g, ws, out, cdt):
    p = synth.dense_problem(96, 80, 192, "bf16", out, c_dtype=cdt, alpha=1.0, beta=0.5 if cdt else 0.0, dist="uniform", seed=7)
    check_against_oracle(p, Run(g, p, ws).run(), what=f"out {out} C {cdt}")


@pytest.mark.parametrize("nk", [1, 2, 3, 5, 7, 8])
def test_odd_and_even_k_tile_counts(g, ws, nk):
    # 64 bf16 per k-tile: an odd k-tile count changes which ring stage the last tile uses
    p = synth.dense_problem(256, 256, 64 * nk, "bf16", "f32", dist="normal", seed=nk)
    for kname in ["tile_BF16_256x256x128b_w2x4_s2", "tile_BF16_128x128x128b_w2x2_s4", "tile_BF16_32x64x128b_w1x2_s6"]:
        op = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_DP, kernel=kidx(kname))
        check_against_oracle(p, Run(g, p, ws).run(op), what=f"{kname} k-tiles {nk}")


def test_fp16_ragged(g, ws):
    p = synth.dense_problem(200, 328, 456, "f16", "f16", c_dtype="f16", alpha=1.0, beta=1.0, dist="uniform", seed=9)
    for kname in ["tile_F16_256x256x128b_w2x4_s2", "tile_F16_128x128x128b_w2x2_s4", "tile_F16_32x128x128b_w1x4_s4"]:
        op = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_DP, kernel=kidx(kname))
        check_against_oracle(p, Run(g, p, ws).run(op), what=kname)


@pytest.mark.parametrize("split", [1, 2, 3, 8])
def test_splitk_matches_oracle_and_leaves_barriers_zero(g, ws, split):
    p = synth.dense_problem(48, 520, 2056, "bf16", "bf16", c_dtype="bf16", alpha=1.0, beta=1.0, a_std=0.02, b_std=0.02, seed=11)
    r = Run(g, p, ws)
    for kname in ["tile_BF16_32x128x128b_w1x4_s4", "tile_BF16_128x128x128b_w2x2_s4"]:
        op = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=split, kernel=kidx(kname))
        print(kname, r.plan(op), flush=True)
        D1 = r.run(op)
        check_against_oracle(p, D1, what=f"{kname} split {split}")
        assert int(ws.barriers.abs().sum().item()) == 0
        D2 = r.run(op)
        assert np.array_equal(D1, D2), "split-K result must not depend on arrival order"


@pytest.mark.parametrize("programs", [256, 7, 100])
def test_streamk(g, ws, programs):
    p = synth.dense_problem(200, 700, 1000, "bf16", "f32", c_dtype="f32", alpha=1.0, beta=0.5, dist="uniform", seed=13)
    r = Run(g, p, ws)
    for kname in ["tile_BF16_128x128x128b_w2x2_s4", "tile_BF16_32x128x128b_w1x4_s4"]:
        op = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_STREAMK, programs=programs, kernel=kidx(kname))
        print(kname, r.plan(op), flush=True)
        D1 = r.run(op)
        check_against_oracle(p, D1, what=f"{kname} stream-K {programs}")
        assert int(ws.barriers.abs().sum().item()) == 0
        assert np.array_equal(D1, r.run(op))


@pytest.mark.parametrize("M", [1, 16])
@pytest.mark.parametrize("sched", ["splitk8", "streamk"])
def test_decode_config_full_size(g, ws, M, sched):
    p = synth.config_decode(M=M)
    r = Run(g, p, ws)
    if sched == "splitk8":
        op = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=8)
    else:
        op = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_STREAMK, programs=256)
    print(r.plan(op), flush=True)
    check_against_oracle(p, r.run(op), what=f"decode M={M} {sched}")
    assert int(ws.barriers.abs().sum().item()) == 0


@pytest.mark.timeout(300)
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_square_4096_every_output(g, ws, dtype):
    # the headline configuration as the benchmark runs it (DEFAULT plan), all
    # 16.8 M outputs against the oracle (about 137 GFLOP of fp64 on the host)
    p = synth.config_square(dtype)
    r = Run(g, p, ws)
    print(r.plan(), flush=True)
    D = r.run()
    check_against_oracle(p, D, what=f"4096^3 {dtype}")


# ---------------------------------------------------------------- int8 -> int32, bit-exact
@pytest.mark.parametrize("shape", [(256, 256, 256), (300, 200, 144), (1, 77, 528)])
def test_int8_exact(g, ws, shape):
    M, N, K = shape
    p = synth.dense_problem(M, N, K, "i8", "i32", c_dtype="i32", alpha=1.0, beta=1.0, seed=M * 3 + K)
    r = Run(g, p, ws)
    for kname in ["tile_I8_256x256x128b_w2x4_s2", "tile_I8_128x128x128b_w2x2_s4", "tile_I8_32x128x128b_w1x4_s4"]:
        op = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_DP, kernel=kidx(kname))
        check_against_oracle(p, r.run(op), what=f"{kname} {shape}")


def test_int8_decode_split8_exact(g, ws):
    p = synth.dense_problem(16, 4096, 14336, "i8", "i32", c_dtype=None, alpha=1.0, beta=0.0, seed=5)
    r = Run(g, p, ws)
    op = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=8)
    check_against_oracle(p, r.run(op), what="int8 decode split 8")
    op = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_STREAMK, programs=256)
    check_against_oracle(p, r.run(op), what="int8 decode stream-K")


@pytest.mark.timeout(300)
def test_int8_square_4096_every_output(g, ws):
    p = synth.dense_problem(4096, 4096, 4096, "i8", "i32", seed=3)
    D = Run(g, p, ws).run()
    check_against_oracle(p, D, what="int8 4096^3")


# ---------------------------------------------------------------- grouped
def test_grouped_small_with_empty_experts(g, ws):
    counts = np.array([5, 0, 300, 1, 0, 129, 256, 0], dtype=np.int32)
    p = synth.grouped_problem(counts, 384, 256, seed=17)
    r = Run(g, p, ws)
    for kname in ["tile_BF16_256x256x128b_w2x4_s2", "tile_BF16_128x128x128b_w2x2_s4"]:
        op = qg.operation(policy=qg.POLICY_FORCE, kernel=kidx(kname))
        print(kname, r.plan(op), flush=True)
        check_against_oracle(p, r.run(op), what=f"grouped {kname}")


@pytest.mark.parametrize("E", [1, 16, 17, 1023])
def test_grouped_expert_counts(g, ws, E):
    # the per-expert m-tile prefix is built by one wave, 16 experts a lane:
    # 16 and 17 experts end on and just past a lane's share, 1023 is the most
    # the engine takes (64 lanes x 16); every third expert is empty
    rng = np.random.default_rng(E)
    counts = rng.integers(1, 70, size=E).astype(np.int32)
    counts[::3] = 0
    if counts.sum() == 0:
        counts[-1] = 5
    p = synth.grouped_problem(counts, 72, 64, seed=E)
    r = Run(g, p, ws)
    for kname in ["tile_BF16_32x128x128b_w1x4_s4", "tile_BF16_128x128x128b_w2x2_s4"]:
        op = qg.operation(policy=qg.POLICY_FORCE, kernel=kidx(kname))
        print(E, kname, r.plan(op), flush=True)
        check_against_oracle(p, r.run(op), what=f"grouped E={E} {kname}")


def test_tiny_config_plan_is_logged(g, ws):
    p = synth.config_tiny()
    desc = Run(g, p, ws).plan()
    assert desc.startswith("kernel=tile_BF16_")


# ---------------------------------------------------------------- skinny-M streaming kernels
SKINNY = ["skinny_BF16_1x16x16x256b_w4_d4_n0", "skinny_BF16_1x16x128x256b_w8_d2_n1", "skinny_BF16_1x16x64x256b_w2_d2_n0",
          "skinny_BF16_2x16x32x256b_w4_d2_n0", "skinny_BF16_1x16x64x256b_w4_d3_n1", "skinny_BF16_1x16x128x256b_w8_d3_n2"]


@pytest.mark.parametrize("kname", SKINNY)
@pytest.mark.parametrize("shape", [(1, 130, 520), (16, 4096, 1032), (5, 77, 8), (13, 200, 4104)])
@pytest.mark.parametrize("sched", ["dp", "split3", "streamk"])
def test_skinny_kernels(g, ws, kname, shape, sched):
    M, N, K = shape
    if kname.startswith("skinny_BF16_2x"):
        M = M + 16  # exercise the second 16-row tile
    p = synth.dense_problem(M, N, K, "bf16", "bf16", c_dtype="bf16", alpha=1.0, beta=1.0, a_std=0.02, b_std=0.02, seed=N + K)
    r = Run(g, p, ws)
    if sched == "dp":
        op = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_DP, kernel=kidx(kname))
    elif sched == "split3":
        op = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=3, kernel=kidx(kname))
    else:
        op = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_STREAMK, programs=37, kernel=kidx(kname))
    print(kname, shape, r.plan(op), flush=True)
    D1 = r.run(op)
    check_against_oracle(p, D1, what=f"{kname} {shape} {sched}")
    assert int(ws.barriers.abs().sum().item()) == 0
    assert np.array_equal(D1, r.run(op))


@pytest.mark.parametrize("M", [1, 16])
def test_skinny_decode_full_size_split8(g, ws, M):
    p = synth.config_decode(M=M)
    r = Run(g, p, ws)
    op = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=8, kernel=kidx("skinny_BF16_1x16x32x256b_w4_d3_n0"))
    print(r.plan(op), flush=True)
    check_against_oracle(p, r.run(op), what=f"skinny decode M={M}")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_skinny_shared_a_ring_matches_per_wave_a(g, ws, dt):
    # the shared-A N-split kernel sums every output in the same order as the
    # per-wave-A one: bit-identical results, at the decode shape with split-K 8
    p = synth.dense_problem(16, 4096, 14336, dt, dt, c_dtype=dt, alpha=1.0, beta=1.0, a_std=0.02, b_std=0.02, seed=21)
    r = Run(g, p, ws)
    E = "BF16" if dt == "bf16" else "F16"
    out = {}
    for kn in (f"skinny_{E}_1x16x128x256b_w8_d3_n2", f"skinny_{E}_1x16x128x256b_w8_d2_n1"):
        op = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=8, kernel=kidx(kn))
        print(kn, r.plan(op), flush=True)
        out[kn] = r.run(op)
    a, b = out.values()
    check_against_oracle(p, a, what=f"shared-A decode {dt}")
    assert np.array_equal(a, b)
    assert int(ws.barriers.abs().sum().item()) == 0


@pytest.mark.parametrize("M", [1, 16])
@pytest.mark.parametrize("sched", ["split8", "streamk256"])
def test_decode_full_size_default_kernels(g, ws, M, sched):
    # the decode configuration exactly as the benchmark runs it (kernel left to
    # the heuristic), every output against the oracle
    p = synth.config_decode(M=M)
    r = Run(g, p, ws)
    if sched == "split8":
        op = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=8)
    else:
        op = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_STREAMK, programs=256)
    print(M, sched, r.plan(op), flush=True)
    check_against_oracle(p, r.run(op), what=f"decode M={M} {sched}")
    assert int(ws.barriers.abs().sum().item()) == 0


def test_decode_default_plan_uses_shared_a(g, ws):
    p = synth.config_decode(M=16)
    r = Run(g, p, ws)
    op = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=8)
    assert "kernel=skinny_BF16_1x16x128x256b_w8_d3_n2" in r.plan(op)


def test_skinny_fp16_and_int8(g, ws):
    p = synth.dense_problem(9, 300, 2056, "f16", "f16", c_dtype="f32", alpha=0.5, beta=2.0, dist="uniform", seed=3)
    op = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=4, kernel=kidx("skinny_F16_1x16x32x256b_w4_d3_n0"))
    check_against_oracle(p, Run(g, p, ws).run(op), what="skinny f16")
    p = synth.dense_problem(16, 4096, 14336, "i8", "i32", c_dtype="i32", alpha=1.0, beta=1.0, seed=8)
    for sched in (qg.SCHED_SPLITK, qg.SCHED_STREAMK):
        for kn in ("skinny_I8_1x16x32x256b_w4_d3_n0", "skinny_I8_1x16x128x256b_w8_d2_n1"):
            op = qg.operation(policy=qg.POLICY_FORCE, schedule=sched, split_k=8, programs=256, kernel=kidx(kn))
            check_against_oracle(p, Run(g, p, ws).run(op), what=f"skinny int8 decode {kn}")


# ---------------------------------------------------------------- degenerate shapes
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_k_zero_gives_beta_c(g, ws, out):
    # K = 0: the sum is empty, D = beta * C (alpha times an empty sum is 0)
    M, N = 70, 136
    C = synth.uniform((M, N), -2, 2, 3)
    A = torch.empty(M, 0, device="cuda", dtype=torch.bfloat16)
    B = torch.empty(N, 0, device="cuda", dtype=torch.bfloat16)
    Cd_t = torch.from_numpy(C).cuda()
    D = torch.full((M, N), float("nan"), device="cuda", dtype=torch.float32 if out == "f32" else torch.bfloat16)
    L = qg.layout
    # a 16-byte-aligned dummy for the empty operands (never read)
    dummy = torch.zeros(16, device="cuda", dtype=torch.bfloat16)
    st = g.run_raw(qg.operation(), 2.0, dummy, L("bf16", M, 0, ld=8), None, None, dummy, L("bf16", N, 0, ld=8),
                   None, None, -0.5, Cd_t, L("f32", M, N), D, L(out, M, N), ws.desc)
    assert st == qg.OK
    torch.cuda.synchronize()
    want = torch.from_numpy(-0.5 * C.astype(np.float64))
    got = D.double().cpu()
    tol = 2.0 ** -8 * want.abs() + 1e-30 if out == "bf16" else 2.0 ** -23 * want.abs() + 1e-30
    assert ((got - want).abs() <= tol).all()


@pytest.mark.parametrize("shape", [(1, 1, 16), (1, 8, 8), (3, 1, 64)])
def test_tiny_edges(g, ws, shape):
    M, N, K = shape
    p = synth.dense_problem(M, N, K, "bf16", "f32", c_dtype="f32", alpha=1.0, beta=1.0, dist="uniform", seed=M + N + K)
    r = Run(g, p, ws)
    print(shape, r.plan(), flush=True)
    check_against_oracle(p, r.run(), what=f"tiny {shape}")
