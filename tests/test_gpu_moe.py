"""GPU parity of the grouped MoE GEMM at its full size (64 experts, Zipf(1.1)
row counts summing to 65536, N = 2048, K = 7168), bf16 and block-scaled fp8,
on sampled rows: the first and last row of every non-empty expert and 64
seeded random rows."""
import numpy as np
import pytest
import torch

import quantized_gemm_bf16_amd as qg
import synth
from tests.gpu_util import Run, check_against_oracle

pytestmark = pytest.mark.gpu


def moe_rows(p, n_random=64, seed=77):
    off = np.asarray(p["offsets"])
    rows = set()
    for e in range(p["E"]):
        if off[e + 1] > off[e]:
            rows |= {int(off[e]), int(off[e + 1]) - 1}
    rows |= set(np.random.default_rng(seed).integers(0, p["M"], size=n_random).tolist())
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
    rows = moe_rows(p)
    print("checking", len(rows), "rows", flush=True)
    check_against_oracle(p, D, rows=rows, what=f"MoE {'fp8' if fp8 else 'bf16'} full size")
