#!/usr/bin/env python3
"""Throughput of the GEMM engine on one MI355X.

A step is one call of qg_run on the 4096^3 bf16 problem (A, B ~ N(0, 1/64),
alpha 1, beta 0, bf16 out): host dispatch, the tile schedule, the LDS-staged
MFMA mainloop and the epilogue, launched on torch's current stream. Inputs are
resident in HBM before timing starts; several input sets are rotated so that
the working set exceeds the 256 MB Infinity Cache and steps do not hit data
left in cache by the previous step. The timed steps are captured once in a HIP
graph and replayed, so host-side call overhead does not open gaps between
launches. The headline `value` is TFLOP/s over the timed steps. A second
workload -- the skinny decode GEMM M=16, N=4096, K=14336 with split-K 8 (and
stream-K) -- is timed the same way and reported in GB/s of algorithmic bytes
under "decode". The weight-only int4 GEMM (64 x 8192 x 8192) and the grouped
MoE GEMM (64 experts, 65536 Zipf-distributed rows, N 2048, K 7168; bf16 and
block-scaled fp8) are reported under "w4a16", "moe" and "moe_fp8".

`roofline` describes the dominant kernel: algorithmic flops per launch over
its mean launch time, measured with HIP events on the launch stream, against
the dense bf16 MFMA peak (256 CUs x 4096 flop/clk x 2.4 GHz = 2516.6 TFLOP/s).
`cpu_baseline` times the fp64 CPU oracle on a bounded row sample of the same
problem on this host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU * 4096 flop/clk * 2.4 GHz (dense, no sparsity)
PEAK_FP8_TFLOPS = 5033.2    # dense fp8 MFMA, twice the bf16 rate
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "quantized_gemm_bf16_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel: str, workload: str):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    e = d.get(workload)
    if not e or e.get("kernel") != kernel or e.get("source_hash") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


class Workload:
    """Rotating device input sets for one problem and a bound qg_run call.
    With same_data, one problem is generated and uploaded `nsets` times (the
    copies only differ in address, which is all the caches see)."""

    def __init__(self, g, ws, make_problem, nsets, op, same_data=False):
        import torch
        import quantized_gemm_bf16_amd as qg
        from tests.gpu_util import Run
        if same_data:
            p = make_problem(0)
            self.runs = [Run(g, p, ws) for _ in range(nsets)]
            del p
        else:
            self.runs = [Run(g, make_problem(i), ws) for i in range(nsets)]
        self.op = op if op is not None else self.runs[0].op()
        self.qg = qg
        self.torch = torch

    def step(self, i):
        st = self.runs[i % len(self.runs)].launch(self.op)
        if st != self.qg.OK:
            raise self.qg.QGemmError(st, "qg_run")

    def time(self, steps, warmup):
        """Warm up eagerly, capture `steps` qg_run calls in one HIP graph and time
        its replay with HIP events on the launch stream (no host gaps between
        launches, so the per-launch figure is device time)."""
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(steps):
                self.step(i)
        graph.replay()  # warm replay
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        total = e0.elapsed_time(e1)
        return dict(total_ms=total, wall_s=wall, kernel_ms_mean=total / steps)


def cpu_baseline(p, flops_per_row, target_s=15.0):
    """The oracle, as it is, on a row sample sized to about `target_s` seconds."""
    import numpy as np
    import oracle
    rows = [0, 1]
    t0 = time.perf_counter()
    oracle.gemm(p, rows=rows)
    dt = max(time.perf_counter() - t0, 1e-3)
    n = int(min(p["M"], max(2, round(target_s / (dt / len(rows))))))
    rows = sorted(set(np.random.default_rng(7).choice(p["M"], size=n, replace=False).tolist()))
    t0 = time.perf_counter()
    oracle.gemm(p, rows=rows)
    dt = time.perf_counter() - t0
    return dict(value=len(rows) * flops_per_row / dt / 1e12, unit="TFLOP/s", cores=oracle.num_threads(),
                kind="oracle",
                sample=f"{len(rows)} of {p['M']} rows of the {p['M']}x{p['N']}x{p['K']} product "
                       f"({len(rows) * p['N']} outputs, fp64, {dt:.1f} s)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", choices=["square", "decode", "w4a16", "moe", "moe_fp8"], default=None,
                    help="time one workload only (profiling)")
    ap.add_argument("--no-extra", action="store_true", help="skip the W4A16 and MoE workloads")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run only a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the engine runs on a single device).", file=sys.stderr)
        return 2

    import torch
    import quantized_gemm_bf16_amd as qg
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1

    if args.copy_mib:
        n = args.copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n}))
        return 0

    g = qg.Gemm()
    ws = qg.workspace()

    out = {}
    M = N = K = 4096
    flops = 2.0 * M * N * K
    if args.only in (None, "square"):
        sq = Workload(g, ws, lambda i: synth.dense_problem(M, N, K, "bf16", "bf16", seed=synth.SEED_A + 10 * i),
                      nsets=4, op=qg.operation())
        kname = sq.runs[0].plan().split()[0].split("=")[1]
        t = sq.time(args.steps, args.warmup)
        ms_step = t["total_ms"] / args.steps
        out["square"] = dict(t, kernel=kname, plan=sq.runs[0].plan(), tflops=flops / (ms_step * 1e-3) / 1e12,
                             kernel_tflops=flops / (t["kernel_ms_mean"] * 1e-3) / 1e12)

    if args.only in (None, "decode"):
        dec_bytes = 16 * 14336 * 2 + 4096 * 14336 * 2 + 2 * 16 * 4096 * 2
        res = {}
        for name, op in [("splitk8", qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=8)),
                         ("streamk", qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_STREAMK, programs=256))]:
            # set 0 is the decode workload itself; the others only differ in seed
            dw = Workload(g, ws, lambda i: synth.dense_problem(16, 4096, 14336, "bf16", "bf16", c_dtype="bf16",
                                                               alpha=1.0, beta=1.0, a_std=0.02, b_std=0.02,
                                                               seed=synth.SEED_A + 10 * i), nsets=3, op=op)
            t = dw.time(max(20, args.steps // 2), max(5, args.warmup // 2))
            res[name] = dict(kernel_us_mean=t["kernel_ms_mean"] * 1e3,
                             gbs=dec_bytes / (t["kernel_ms_mean"] * 1e-3) / 1e9,
                             frac_hbm=dec_bytes / (t["kernel_ms_mean"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
                             plan=dw.runs[0].plan(op))
            del dw
        out["decode"] = dict(bytes_per_call=dec_bytes, **res)

    extra = not args.no_extra and args.only is None
    if extra or args.only == "w4a16":
        # B 33.5 MB + scales 1 MB per set: 9 sets exceed the 256 MB Infinity Cache
        w4_bytes = 64 * 8192 * 2 + 8192 * 8192 // 2 + 8192 * 64 * 2 + 64 * 8192 * 2
        ww = Workload(g, ws, lambda i: synth.config_w4a16(), nsets=9, op=None, same_data=True)
        t = ww.time(args.steps, args.warmup)
        us = t["kernel_ms_mean"] * 1e3
        out["w4a16"] = {"kernel_us_mean": round(us, 3), "GB/s": round(w4_bytes / (us * 1e-6) / 1e9, 1),
                        "frac_hbm": round(w4_bytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                        "TFLOP/s": round(2.0 * 64 * 8192 * 8192 / (us * 1e-6) / 1e12, 2),
                        "bytes_per_call": w4_bytes, "plan": ww.runs[0].plan()}
        del ww
    for fp8 in (False, True):
        name = "moe_fp8" if fp8 else "moe"
        if not (extra or args.only == name):
            continue
        # one set of 2.8 GB (bf16) / 1.4 GB (fp8) is far beyond every cache
        mw = Workload(g, ws, lambda i: synth.config_moe(fp8=fp8), nsets=1, op=None)
        p0 = mw.runs[0].p
        mflops = 2.0 * p0["M"] * p0["N"] * p0["K"]
        t = mw.time(max(10, args.steps // 5), max(3, args.warmup // 5))
        us = t["kernel_ms_mean"] * 1e3
        peak = PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS
        out[name] = {"kernel_us_mean": round(us, 1), "TFLOP/s": round(mflops / (us * 1e-6) / 1e12, 1),
                     "frac_peak": round(mflops / (us * 1e-6) / 1e12 / peak, 4), "peak": peak,
                     "flops_per_call": mflops, "plan": mw.runs[0].plan()}
        del mw, p0

    if args.only:
        print(json.dumps(out))
        return 0

    sq_ = out["square"]
    ms_step = sq_["total_ms"] / args.steps
    achieved = sq_["kernel_tflops"]
    line = {
        "metric": "TFLOP/s (% of bf16 MFMA peak) at 4096^3; HBM GB/s at M=16 decode GEMM",
        "value": round(sq_["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1/64) bf16, 4 rotating input sets)",
        "config": {"workload": "dense GEMM M=N=K=4096, bf16 in, fp32 accumulate, bf16 out, alpha 1, beta 0",
                   "M": M, "N": N, "K": K, "plan": sq_["plan"]},
        "frac_of_peak": round(sq_["tflops"] / PEAK_BF16_TFLOPS, 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "kernel": sq_["kernel"],
                     "kernel_us_mean": round(sq_["kernel_ms_mean"] * 1e3, 3),
                     "traffic": traffic_from_profile(sq_["kernel"], "square_4096_bf16")},
        "decode": {k: (round(v, 3) if isinstance(v, float) else v) for k, v in out["decode"].items()
                   if not isinstance(v, dict)},
    }
    for k in ("splitk8", "streamk"):
        d = out["decode"][k]
        line["decode"][k] = {"kernel_us_mean": round(d["kernel_us_mean"], 3), "GB/s": round(d["gbs"], 1),
                             "frac_hbm": round(d["frac_hbm"], 4), "plan": d["plan"]}
    for k in ("w4a16", "moe", "moe_fp8"):
        if k in out:
            line[k] = out[k]
    if not args.no_cpu:
        p = synth.config_square("bf16")
        line["cpu_baseline"] = cpu_baseline(p, 2.0 * N * K)
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
