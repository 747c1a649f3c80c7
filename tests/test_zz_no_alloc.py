"""qg_run_noalloc (workspace from the library's per-GPU device array) against
qg_run with a caller-owned workspace of the same size: same plans, so the
results must be bit-identical, and both within the oracle's bound. Two calls
in a row, the second on a smaller problem, so the second run starts from the
array as the first left it (counters back at zero, stale partials)."""
import numpy as np
import pytest
import torch

import quantized_gemm_bf16_amd as qg
import synth
from tests.gpu_util import Run, check_against_oracle

pytestmark = pytest.mark.gpu


def _noalloc(g, r, op):
    p = r.p
    r.D.fill_(float("nan"))
    st = g.run_noalloc_raw(op, p["alpha"], r.A, r.Ad, r.U, r.Ud, r.B, r.Bd, r.V, r.Vd, p["beta"], r.C, r.Cd, r.D,
                           r.Dd)
    assert st == qg.OK, qg.status_str(st)
    torch.cuda.synchronize()
    D = r.D.double().cpu().numpy()
    assert np.isnan(D[:, p["N"]:]).all(), "write past column N"
    return np.ascontiguousarray(D[:, :p["N"]])


def _same_size_workspace():
    return qg.workspace(barriers=qg.noalloc_barriers_size(), partials=qg.noalloc_partials_size())


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_qg_run_on_two_calls(order):
    assert torch.cuda.is_available()
    g = qg.Gemm()
    ws = _same_size_workspace()
    cases = [
        # the decode configuration with split-K 8 (2 MiB of partials)
        (synth.config_decode(M=16),
         dict(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=8)),
        # a smaller, ragged problem with stream-K over 37 programs
        (synth.dense_problem(5, 1000, 3000, "bf16", "bf16", c_dtype="f32", alpha=0.5, beta=2.0,
                             a_std=0.02, b_std=0.02, seed=44),
         dict(policy=qg.POLICY_FORCE, schedule=qg.SCHED_STREAMK, programs=37)),
    ]
    for i, (p, kw) in enumerate(cases):
        r = Run(g, p, ws)
        op = r.op(**kw)
        print("case", i, p["M"], p["N"], p["K"], r.plan(op), flush=True)
        want = r.run(op)
        check_against_oracle(p, want, what=f"qg_run case {i}")
        got = _noalloc(g, r, op)
        assert np.array_equal(got, want), f"case {i}: qg_run_noalloc differs from qg_run"
        # and once more: the counters must have come back to zero
        assert np.array_equal(_noalloc(g, r, op), want), f"case {i}: second no-alloc run differs"


def test_noalloc_default_policy_and_w4a16():
    g = qg.Gemm()
    ws = _same_size_workspace()
    for p in (synth.dense_problem(16, 2048, 8192, "bf16", "bf16", c_dtype="bf16", alpha=1.0, beta=1.0,
                                  a_std=0.02, b_std=0.02, seed=45),
              synth.w4a16_problem(16, 512, 1024, seed=46)):
        r = Run(g, p, ws)
        op = r.op()
        print(r.plan(op), flush=True)
        want = r.run(op)
        got = _noalloc(g, r, op)
        assert np.array_equal(got, want)
        check_against_oracle(p, got, what="no-alloc default plan")


def test_noalloc_refusals():
    g = qg.Gemm()
    p = synth.dense_problem(16, 1024, 2048, "bf16", "bf16", seed=47)
    r = Run(g, p, None)
    # measuring needs events and synchronisation
    st = g.run_noalloc_raw(r.op(policy=qg.POLICY_MEASURE), 1.0, r.A, r.Ad, None, None, r.B, r.Bd, None, None, 0.0,
                           None, None, r.D, r.Dd)
    assert st == qg.ERR_UNSUPPORTED
    # a plan whose partials exceed the array: 16 tiles of 256 x 256 split 16 ways
    # need 64 MiB
    q = synth.dense_problem(1024, 1024, 8192, "bf16", "bf16", seed=48)
    rq = Run(g, q, None)
    op = rq.op(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=16,
               kernel=qg.kernel_names().index("tile_BF16_256x256x128b_w2x4_s2"))
    st = g.run_noalloc_raw(op, 1.0, rq.A, rq.Ad, None, None, rq.B, rq.Bd, None, None, 0.0, None, None, rq.D, rq.Dd)
    assert st == qg.ERR_WORKSPACE
