"""GPU parity of batched GEMM (batches of one M x N x K shape, no offsets
array; the batched variant of the TileLang tutorial "gemm_variants.py") against
the fp64 oracle, through the C ABI."""
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


@pytest.mark.parametrize("kname", [None, "tile_BF16_256x256x128b_w2x4_s2", "tile_BF16_128x128x128b_w2x2_s4",
                                   "tile_BF16_32x128x128b_w1x4_s4", "skinny_BF16_1x16x16x256b_w8_d2_n0"])
@pytest.mark.parametrize("shape", [(3, 100, 200, 136), (2, 256, 256, 512), (5, 17, 300, 1040), (1, 64, 72, 64)])
def test_bf16_shapes(g, ws, kname, shape):
    batch, M, N, K = shape
    p = synth.batched_problem(batch, M, N, K, c_dtype="bf16", alpha=1.25, beta=-0.5, seed=batch * 1000 + M)
    r = Run(g, p, ws)
    op = r.op() if kname is None else r.op(policy=qg.POLICY_FORCE, kernel=kidx(kname))
    if batch == 1 and kname and kname.startswith("skinny_") and M > 16:
        # one batch is a plain GEMM, where a skinny kernel must cover all M rows
        with pytest.raises(qg.QGemmError) as e:
            r.plan(op)
        assert e.value.status == qg.ERR_NO_KERNEL
        return
    desc = r.plan(op)
    print(shape, desc, flush=True)
    assert ("schedule=batched" in desc) == (batch > 1)  # one batch is a plain GEMM
    D = r.run(op)
    check_against_oracle(p, D, what=f"batched {shape} {kname}")
    assert np.array_equal(D, r.run(op))


def test_shared_b_and_output_types(g, ws):
    for out in ("f32", "f16"):
        p = synth.batched_problem(4, 48, 256, 320, in_dtype="f16", out_dtype=out, c_dtype="f32", beta=1.0,
                                  seed=7, share_b=True)
        r = Run(g, p, ws)
        print(r.plan(), flush=True)
        check_against_oracle(p, r.run(), what=f"batched shared B -> {out}")


def test_decode_shaped_batches(g, ws):
    # many skinny products: the heuristic picks a skinny kernel for the batch
    p = synth.batched_problem(8, 16, 1024, 2048, c_dtype="bf16", beta=1.0, seed=9, a_std=0.02)
    r = Run(g, p, ws)
    desc = r.plan()
    print(desc, flush=True)
    assert "kernel=skinny_" in desc
    check_against_oracle(p, r.run(), what="batched decode")


def test_int8_exact(g, ws):
    p = synth.batched_problem(3, 96, 160, 256, in_dtype="i8", c_dtype="i32", beta=1.0, seed=11)
    r = Run(g, p, ws)
    print(r.plan(), flush=True)
    check_against_oracle(p, r.run(), what="batched int8")


@pytest.mark.parametrize("share_b", [False, True])
def test_fp8_block_scaled(g, ws, share_b):
    p = synth.batched_problem(3, 70, 256, 384, fp8=True, seed=13, share_b=share_b)
    r = Run(g, p, ws)
    print(r.plan(), flush=True)
    check_against_oracle(p, r.run(), what=f"batched fp8 shared={share_b}")
