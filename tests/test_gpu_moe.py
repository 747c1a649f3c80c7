"""GPU parity of the grouped MoE GEMM at its full size (64 experts, Zipf(1.1)
row counts summing to 65536, N = 2048, K = 7168), bf16 and block-scaled fp8,
on sampled rows: the first and last row of every non-empty expert, and two
seeded rows inside every BM-row m-tile of every expert (BM from the plan), so
that every tile the grouped schedule runs is compared."""
import numpy as np
import pytest
import torch

import quantized_gemm_bf16_amd as qg
import synth
from tests.gpu_util import Run, check_against_oracle

pytestmark = pytest.mark.gpu


def moe_rows(p, bm, per_tile=2, seed=77):
    off = np.asarray(p["offsets"])
    g = np.random.default_rng(seed)
    rows = set()
    for e in range(p["E"]):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        rows |= {lo, hi - 1}
        for t0 in range(lo, hi, bm):
            t1 = min(hi, t0 + bm)
            rows |= set(g.integers(t0, t1, size=per_tile).tolist())
    return sorted(rows)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_moe_config_sampled_rows(fp8):
    assert torch.cuda.is_available()
    g = qg.Gemm()
    p = synth.config_moe(fp8=fp8)
    print("generated", p["M"], p["N"], p["K"], "experts", p["E"], flush=True)
    r = Run(g, p, qg.workspace())
    print(r.plan(), flush=True)
    D = r.run()
    bm = int(dict(kv.split("=") for kv in r.plan().split())["bm"])
    rows = moe_rows(p, bm)
    print("checking", len(rows), "rows over every", bm, "-row m-tile", flush=True)
    check_against_oracle(p, D, rows=rows, what=f"MoE {'fp8' if fp8 else 'bf16'} full size")
