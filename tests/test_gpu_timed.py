"""GPU tests of qg_run_timed: a split-K or data-parallel launch that records
where its time goes. The result must be the very bits of qg_run's, the
arrival counters must be left zero, and every unit must leave eight ordered
timestamps."""
import numpy as np
import pytest
import torch

import quantized_gemm_bf16_amd as qg
import synth
from tests.gpu_util import Run, check_against_oracle

pytestmark = pytest.mark.gpu


def kname(desc):
    return dict(kv.split("=") for kv in desc.split())["kernel"]


CASES = {
    "decode_bf16_split8": (lambda: synth.dense_problem(16, 4096, 14336, "bf16", "bf16", c_dtype="bf16", alpha=1.0,
                                                       beta=1.0, a_std=0.02, b_std=0.02, seed=71), 8),
    "w4a16_split4": (lambda: synth.w4a16_problem(64, 1024, 2048, seed=72), 4),
    "int8_split3": (lambda: synth.dense_problem(16, 512, 1024, "i8", "i32", seed=73), 3),
    "ragged_bf16_split3": (lambda: synth.dense_problem(5, 300, 1000, "bf16", "f32", seed=74), 3),
    "tile_bf16_split2": (lambda: synth.dense_problem(256, 384, 1024, "bf16", "f32", seed=76), 2),
    # data-parallel (split 1): every unit completes its tile
    "tile_bf16_dp": (lambda: synth.dense_problem(512, 768, 1024, "bf16", "bf16", seed=77), 1),
    "decode_bf16_dp": (lambda: synth.dense_problem(16, 1024, 4096, "bf16", "bf16", c_dtype="bf16", alpha=1.0,
                                                   beta=1.0, a_std=0.02, b_std=0.02, seed=78), 1),
    "w4a16_dp": (lambda: synth.w4a16_problem(64, 1024, 2048, seed=79), 1),
}


@pytest.mark.parametrize("case", list(CASES))
def test_timed_run_matches_and_records(case):
    make, split = CASES[case]
    p = make()
    ws = qg.workspace()
    g = qg.Gemm()
    r = Run(g, p, ws)
    op = r.op(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=split) if split > 1 else \
        r.op(policy=qg.POLICY_FORCE, schedule=qg.SCHED_DP)
    desc = r.plan(op)
    print(case, desc, flush=True)
    D1 = r.run(op)
    check_against_oracle(p, D1, what=f"{case} qg_run")

    d = dict(kv.split("=") for kv in desc.split())
    assert d["schedule"] == ("splitk" if split > 1 else "dp"), desc
    units = int(d["tiles"]) * int(d["split"])
    stamps = torch.full((units * 8,), -1, dtype=torch.int64, device="cuda")
    ws.partials.fill_(float("nan"))
    r.reset_output()
    st, n = r.launch_timed(op, stamps)
    assert st == qg.OK and n == units
    torch.cuda.synchronize()
    D2 = r.run_result()
    assert np.array_equal(D1, D2), f"{case}: timed run differs from qg_run"
    assert int(ws.barriers.abs().sum().item()) == 0, "arrival counters not left zero"

    s = stamps.view(units, 8).cpu().numpy().astype(np.int64)
    assert (s != -1).all(), "a unit left a timestamp unwritten"
    last = s[:, 5]
    assert set(np.unique(last)) <= {0, 1}
    assert int(last.sum()) == int(d["tiles"]), "one completing unit per tile"
    assert (s[:, 0] <= s[:, 1]).all() and (s[:, 1] <= s[:, 2]).all() and (s[:, 2] <= s[:, 4]).all()
    done = last == 1
    assert (s[done, 2] <= s[done, 3]).all() and (s[done, 3] <= s[done, 4]).all()
    assert (s[~done, 3] == 0).all() and (s[~done, 4] == s[~done, 2]).all()
    assert (s[:, 6] <= s[:, 7]).all()
    if split == 1:
        # data-parallel: nothing published or read back
        assert (s[:, 2] == s[:, 1]).all() and (s[:, 3] == s[:, 1]).all()
    span_us = (s[:, 4].max() - s[:, 0].min()) / 100.0
    print(f"{case}: {units} units, span {span_us:.2f} us", flush=True)
    assert 0 < span_us < 1e5


def test_timed_run_refuses_other_schedules():
    ws = qg.workspace()
    g = qg.Gemm()
    stamps = torch.zeros(8 << 10, dtype=torch.int64, device="cuda")
    r = Run(g, synth.dense_problem(64, 256, 256, "bf16", "bf16", seed=75), ws)
    st, _ = r.launch_timed(r.op(policy=qg.POLICY_FORCE, schedule=qg.SCHED_STREAMK, programs=7), stamps)
    assert st == qg.ERR_UNSUPPORTED
    rg = Run(g, synth.grouped_problem(np.array([40, 0, 70]), 256, 256, seed=80), ws)
    st, _ = rg.launch_timed(rg.op(), stamps)
    assert st == qg.ERR_UNSUPPORTED
    assert int(stamps.abs().sum().item()) == 0
