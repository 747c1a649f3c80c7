"""qg_run inside a captured HIP graph: several replays, with eager work and
synchronisations between them, must each reproduce the eager result bit for
bit (DP and split-K plans; split-K relies on the arrival counters returning to
zero at the end of every run)."""
import numpy as np
import pytest
import torch

import quantized_gemm_bf16_amd as qg
import synth
from tests.gpu_util import Run, check_against_oracle

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("case", ["dp", "splitk", "streamk"])
def test_graph_replays_match_eager(case):
    g = qg.Gemm()
    ws = qg.workspace()
    if case == "dp":
        p = synth.dense_problem(512, 384, 1024, "bf16", "bf16", c_dtype="f32", alpha=1.0, beta=0.5, dist="uniform", seed=2)
        op = qg.operation()
    else:
        p = synth.dense_problem(16, 1024, 4096, "bf16", "bf16", c_dtype="bf16", alpha=1.0, beta=1.0,
                                a_std=0.02, b_std=0.02, seed=4)
        op = qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK if case == "splitk" else qg.SCHED_STREAMK,
                          split_k=4, programs=64)
    r = Run(g, p, ws)
    eager = r.run(op)
    check_against_oracle(p, eager, what=f"eager {case}")
    r.D.fill_(float("nan"))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        assert r.launch(op) == qg.OK
    scratch = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        r.D.fill_(float("nan"))
        scratch.mul_(1.0001)  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = r.D.double().cpu().numpy()[:, :p["N"]]
        assert np.array_equal(got, eager), f"replay {rep} differs from eager"
        assert int(ws.barriers.abs().sum().item()) == 0
