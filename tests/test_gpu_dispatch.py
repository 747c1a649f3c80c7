"""GPU tests of the dispatch layer: the measuring policy fills the cache, the
cache answers later calls (exact key and tuning-sequence bucket), and an
exported cache imported into a fresh handle reproduces the same launches."""
import numpy as np
import pytest
import torch

import quantized_gemm_bf16_amd as qg
import synth
from tests.gpu_util import Run, check_against_oracle

pytestmark = pytest.mark.gpu


def kname(desc):
    return dict(kv.split("=") for kv in desc.split())["kernel"]


def test_measure_fills_cache_and_is_reused():
    ws = qg.workspace()
    g = qg.Gemm()
    p = synth.dense_problem(16, 1024, 2048, "bf16", "bf16", c_dtype="bf16", alpha=1.0, beta=1.0,
                            a_std=0.02, b_std=0.02, seed=3)
    r = Run(g, p, ws)
    assert g.cache_size() == 0
    D = r.run(r.op(policy=qg.POLICY_MEASURE))
    check_against_oracle(p, D, what="measured run")
    assert g.cache_size() == 1
    assert int(ws.barriers.abs().sum().item()) == 0
    chosen = r.plan(r.op(policy=qg.POLICY_REUSE))
    print("measured choice:", chosen, flush=True)
    # a second MEASURE call on the same key hits the cache (no new entry)
    D2 = r.run(r.op(policy=qg.POLICY_MEASURE))
    assert g.cache_size() == 1
    assert np.array_equal(D, D2)
    # DEFAULT now follows the cache; a smaller M in the same tuning bucket too
    assert r.plan(r.op(policy=qg.POLICY_DEFAULT)) == chosen
    p12 = synth.dense_problem(12, 1024, 2048, "bf16", "bf16", c_dtype="bf16", alpha=1.0, beta=1.0,
                              a_std=0.02, b_std=0.02, seed=4)
    r12 = Run(g, p12, ws)
    assert kname(r12.plan(r12.op(policy=qg.POLICY_REUSE))) == kname(chosen)
    check_against_oracle(p12, r12.run(r12.op(policy=qg.POLICY_REUSE)), what="bucket reuse M=12")


def test_export_import_roundtrip_on_device():
    ws = qg.workspace()
    g = qg.Gemm()
    p = synth.dense_problem(32, 768, 1536, "bf16", "f32", c_dtype="f32", alpha=0.5, beta=2.0, seed=5)
    r = Run(g, p, ws)
    D = r.run(r.op(policy=qg.POLICY_MEASURE))
    text = g.export()
    g2 = qg.Gemm()
    r2 = Run(g2, p, ws)
    with pytest.raises(qg.QGemmError) as e:
        r2.run(r2.op(policy=qg.POLICY_REUSE))
    assert e.value.status == qg.ERR_NO_KERNEL
    g2.import_(text)
    assert g2.cache_size() == g.cache_size()
    assert r2.plan(r2.op(policy=qg.POLICY_REUSE)) == r.plan(r.op(policy=qg.POLICY_REUSE))
    D2 = r2.run(r2.op(policy=qg.POLICY_REUSE))
    assert np.array_equal(D, D2)
    check_against_oracle(p, D2, what="imported choice")


def test_measure_refuses_aliased_c_and_d():
    ws = qg.workspace()
    g = qg.Gemm()
    M, N, K = 16, 256, 512
    p = synth.dense_problem(M, N, K, "bf16", "bf16", c_dtype="bf16", alpha=1.0, beta=1.0,
                            a_std=0.02, b_std=0.02, seed=12)
    r = Run(g, p, ws)
    CD = r.C.clone()  # D aliases C: D = A @ B + D
    Cd = qg.layout("bf16", M, N, ld=r.ldn)
    st = g.run_raw(qg.operation(policy=qg.POLICY_MEASURE), 1.0, r.A, r.Ad, None, None, r.B, r.Bd,
                   None, None, 1.0, CD, Cd, CD, Cd, ws.desc)
    assert st == qg.ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.equal(CD, r.C), "a refused call must not have touched D"
    # DEFAULT accepts the in-place update; every output against the oracle
    st = g.run_raw(qg.operation(), 1.0, r.A, r.Ad, None, None, r.B, r.Bd, None, None, 1.0, CD, Cd, CD, Cd, ws.desc)
    assert st == qg.OK
    torch.cuda.synchronize()
    D = CD.view(torch.bfloat16).double().cpu().numpy()[:, :N]  # C was uploaded as bf16 bit patterns
    check_against_oracle(p, D, what="in-place D = A @ B + D")


def test_measure_policy_under_graph_capture_does_not_measure():
    # measuring synchronises the stream; under capture the engine resolves
    # like DEFAULT instead and leaves the cache empty
    ws = qg.workspace()
    g = qg.Gemm()
    p = synth.dense_problem(16, 1024, 2048, "bf16", "bf16", c_dtype="bf16", alpha=1.0, beta=1.0,
                            a_std=0.02, b_std=0.02, seed=6)
    r = Run(g, p, ws)
    op = r.op(policy=qg.POLICY_MEASURE)
    eager_default = r.run(r.op())
    ws.partials.fill_(float("nan"))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        assert r.launch(op) == qg.OK
    assert g.cache_size() == 0
    for rep in range(3):
        r.D.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = r.D.double().cpu().numpy()[:, :p["N"]]
        assert np.array_equal(got, eager_default), f"replay {rep}"
    check_against_oracle(p, eager_default, what="MEASURE under capture")
    # outside capture the same call measures and fills the cache
    r.run(op)
    assert g.cache_size() == 1
