"""Seeded random GPU parity across the kernel families.

Each case draws, from its own fixed seed, an element family (bf16, fp16,
int8, block-scaled e4m3, int4 weights, w8a8), a shape (M up to 300, N up to
600, K up to 1600; K a multiple of 128 for int4), the output and C types,
alpha and beta, and a schedule (the engine's choice, or a forced DP,
split-K 2-8 or stream-K with 2-300 programs). Every output is compared with
the oracle (int32 bit-exact, float within the tolerance rule). A and B rows
have a 16-byte pitch whose padding past K is poisoned; the partials
workspace is NaN-poisoned before each run and the row padding of D must stay
untouched (both in Run.run)."""
import numpy as np
import pytest

import quantized_gemm_bf16_amd as qg
import synth
from tests.gpu_util import Run, check_against_oracle

pytestmark = pytest.mark.gpu

FAMILIES = ["bf16", "f16", "i8", "e4m3", "w4a16", "w8a8"]
N_CASES = 360


def draw(i):
    r = np.random.default_rng(7000 + i)
    fam = FAMILIES[i % len(FAMILIES)]
    M = int(r.choice([1, 2, 5, 16, 17, 31, 33, 64, 65, 100, 129, 200, 300]))
    N = int(r.integers(1, 601))
    K = 128 * int(r.integers(1, 13)) if fam == "w4a16" else int(r.integers(1, 1601))
    seed = 100 + i
    alpha = float(r.choice([1.0, 0.75, -2.0]))
    use_c = bool(r.integers(0, 2))
    beta = float(r.choice([0.5, -1.25, 1.0])) if use_c else 0.0
    if fam in ("bf16", "f16"):
        out = str(r.choice(["f32", "bf16", "f16"]))
        c = str(r.choice(["f32", "bf16", "f16"])) if use_c else None
        p = synth.dense_problem(M, N, K, fam, out, c_dtype=c, alpha=alpha, beta=beta, seed=seed)
    elif fam == "i8":
        c = "i32" if use_c else None
        p = synth.dense_problem(M, N, K, "i8", "i32", c_dtype=c, alpha=1.0, beta=1.0 if use_c else 0.0, seed=seed)
    elif fam == "e4m3":
        out = str(r.choice(["f32", "bf16", "f16"]))
        c = str(r.choice(["f32", "bf16"])) if use_c else None
        p = synth.dense_fp8_problem(M, N, K, out_dtype=out, c_dtype=c, alpha=alpha, beta=beta, seed=seed)
    elif fam == "w8a8":
        out = str(r.choice(["f32", "bf16", "f16"]))
        c = str(r.choice(["f32", "bf16"])) if use_c else None
        p = synth.w8a8_problem(M, N, K, out_dtype=out, c_dtype=c, alpha=alpha, beta=beta, seed=seed)
    else:
        out = str(r.choice(["f32", "bf16", "f16"]))
        p = synth.w4a16_problem(M, N, K, seed=seed, out_dtype=out, asym=bool(r.integers(0, 2)))
    sched = str(r.choice(["auto", "dp", "split", "streamk"]))
    return fam, p, sched, int(r.integers(2, 9)), int(r.integers(2, 301))


@pytest.fixture(scope="module")
def env():
    return qg.Gemm(), qg.workspace()


@pytest.mark.parametrize("i", range(N_CASES))
def test_fuzz_case(env, i):
    g, ws = env
    fam, p, sched, split, programs = draw(i)
    if p["kind"] == "dense":
        # row pitch at the next 16-byte boundary; the pitch padding holds NaN
        # codes / extreme int8 values, which must not reach D
        per = 16 if p["in_dtype"] in ("i8", "e4m3") else 8
        r = Run(g, p, ws, ldk=-(-p["K"] // per) * per)
    else:
        r = Run(g, p, ws)
    if sched == "auto":
        op = r.op()
    elif sched == "dp":
        op = r.op(policy=qg.POLICY_FORCE, schedule=qg.SCHED_DP)
    elif sched == "split":
        op = r.op(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=split)
    else:
        # two partial slots per program: with big tiles, many programs do not
        # fit the 32 MiB partials workspace (refused with QG_ERR_WORKSPACE);
        # halve the count until the plan fits
        while True:
            op = r.op(policy=qg.POLICY_FORCE, schedule=qg.SCHED_STREAMK, programs=programs)
            try:
                r.plan(op)
                break
            except qg.QGemmError as e:
                assert e.status == qg.ERR_WORKSPACE and programs > 2, str(e)
                programs //= 2
    what = f"case {i}: {fam} M={p['M']} N={p['N']} K={p['K']} out={p['out_dtype']} c={p.get('c_dtype')} " \
           f"alpha={p['alpha']} beta={p['beta']} {sched} | {r.plan(op)}"
    print(what, flush=True)
    D = r.run(op)
    check_against_oracle(p, D, what=what)
    assert int(ws.barriers.abs().sum().item()) == 0, f"{what}: arrival counters not left zero"


# Grouped (MoE: per-expert row counts, some experts empty) and batched
# (equal batches, B per batch or shared) problems, with the engine's plan.
GROUPED_CASES = 100
GROUPED_KINDS = ["grouped", "grouped_fp8", "batched", "batched_fp8", "batched_i8"]


def draw_grouped(i):
    r = np.random.default_rng(9000 + i)
    kind = GROUPED_KINDS[i % len(GROUPED_KINDS)]
    N = int(r.integers(1, 401))
    seed = 500 + i
    if kind.startswith("grouped"):
        E = int(r.integers(1, 25))
        counts = r.integers(0, 300, size=E)
        counts[r.random(E) < 0.25] = 0
        if counts.sum() == 0:
            counts[0] = 1
        K = int(r.integers(1, 901))
        out = str(r.choice(["bf16", "f32"]))
        p = synth.grouped_problem(counts, N, K, in_dtype=str(r.choice(["bf16", "f16"])), out_dtype=out, seed=seed,
                                  fp8=kind == "grouped_fp8")
        return kind, p
    batch, M, K = int(r.integers(1, 9)), int(r.integers(1, 130)), 16 * int(r.integers(1, 50))
    use_c = bool(r.integers(0, 2))
    if kind == "batched_i8":
        p = synth.batched_problem(batch, M, N, K, in_dtype="i8", c_dtype="i32" if use_c else None, beta=1.0,
                                  seed=seed)
    else:
        fp8 = kind == "batched_fp8"
        p = synth.batched_problem(batch, M, N, K, in_dtype="bf16", out_dtype=str(r.choice(["bf16", "f32"])),
                                  c_dtype=str(r.choice(["bf16", "f32"])) if use_c else None,
                                  alpha=float(r.choice([1.0, -0.5])), beta=float(r.choice([0.5, 1.0])) if use_c else 0.0,
                                  seed=seed, share_b=bool(r.integers(0, 2)), fp8=fp8)
    return kind, p


@pytest.mark.parametrize("i", range(GROUPED_CASES))
def test_fuzz_grouped_case(env, i):
    g, ws = env
    kind, p = draw_grouped(i)
    if kind.startswith("grouped"):
        per = 16 if p["in_dtype"] == "e4m3" else 8
        r = Run(g, p, ws, ldk=-(-p["K"] // per) * per)
    else:
        r = Run(g, p, ws)
    op = r.op()
    what = f"grouped case {i}: {kind} E={p['E']} rows={p['M']} N={p['N']} K={p['K']} out={p['out_dtype']} " \
           f"c={p.get('c_dtype')} | {r.plan(op)}"
    print(what, flush=True)
    D = r.run(op)
    check_against_oracle(p, D, what=what)
