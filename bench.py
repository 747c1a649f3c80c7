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
problem on this host's cores; `cpu_oracle` times it on every workload (a
row sample where the whole product would take minutes), with the CPU model,
the cores this process may run on, and a single-threaded run of the small
256^3 case.

Measured in the same process, next to the kernels they bound (`ceilings`):
an MFMA-only loop at the 4096^3 kernel's occupancy (the sustained matrix
rate, and the shader clock it ran at, from s_memtime / s_memrealtime) and a
streaming read of the decode weight's size (the sustained HBM read rate);
`frac_of_sustained` / `frac_of_stream` place the kernels against them.
`clocks` holds the shader / memory clock and board power read from sysfs
every 20 ms while each workload's timed graph is replayed for about a second
(`sustained_us` is the mean kernel time over that second, with the
sampling going on).
`host_us_per_call` is the host time of one qg_run on the decode problem
(a C loop of back-to-back calls): with the DEFAULT policy (memoised
heuristic), after MEASURE (dispatch-cache hit), FORCE, and the runtime's
cost of launching an empty kernel.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import threading
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


def log(msg):
    """Progress of the run on stderr (the JSON line alone goes to stdout)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def graph_time(step, steps, warmup, warm_ms=100.0):
    """Capture `steps` calls of step(i) in one HIP graph and time one replay
    with HIP events on the launch stream (no host gaps between launches, so
    the per-launch figure is device time). The `warmup` untimed steps run
    as replays of the same graph, followed by at least `warm_ms` of replays
    queued right before the timed one, so the timed steps start on a GPU
    that has been busy with this graph for a while. Returns the timing and
    the graph (for sustain())."""
    import torch
    for i in range(min(warmup, 3)):  # eager first calls (code objects, caches)
        step(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            step(i)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    # at least three: the first replays of a freshly captured graph run
    # slower (measured: 115.5 vs 109.3 us per 4096^3 kernel), then it is steady
    nwarm = max(3, -(-warmup // steps))
    for _ in range(nwarm):
        graph.replay()
    torch.cuda.synchronize()
    # then at least warm_ms of back-to-back replays right before the timed
    # one: short kernels timed after a few ms of work read 6-7 % slower than
    # over a sustained second (clocks and power still settling)
    per = (time.perf_counter() - w0) * 1e3 / nwarm
    for _ in range(int(warm_ms / max(per, 1e-3))):
        graph.replay()
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total = e0.elapsed_time(e1)
    return dict(total_ms=total, wall_s=wall, kernel_ms_mean=total / steps), graph


def _sysfs_device():
    """sysfs directory of device 0 (by PCI address), or of the only amdgpu card."""
    import torch
    pr = torch.cuda.get_device_properties(0)
    bus, dev, dom = (getattr(pr, k, None) for k in ("pci_bus_id", "pci_device_id", "pci_domain_id"))
    if bus is not None and dev is not None:
        path = f"/sys/bus/pci/devices/{int(dom or 0):04x}:{int(bus):02x}:{int(dev):02x}.0"
        if os.path.isdir(path):
            return path
    cards = {os.path.realpath(os.path.dirname(f)) for f in glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")}
    return cards.pop() if len(cards) == 1 else None


def _read(path):
    try:
        with open(path) as f:
            return f.read()
    except OSError:
        return None


def _dpm_mhz(text):
    """Current level of a pp_dpm_* table ('1: 2400Mhz *')."""
    for line in (text or "").splitlines():
        if line.rstrip().endswith("*"):
            m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
            if m:
                return float(m.group(1))
    return None


class ClockSampler:
    """Reads the shader clock, memory clock and board power of device 0 from
    sysfs every few milliseconds on a background thread."""

    def __init__(self, dev, period_s=0.02):
        self.dev, self.period = dev, period_s
        self.samples = {"sclk_mhz": [], "mclk_mhz": [], "power_w": []}
        self._stop = threading.Event()
        self._files = {}
        if dev:
            hw = sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*")))
            for key, names in (("sclk_hz", ["freq1_input"]), ("power_uw", ["power1_average", "power1_input"])):
                for h in hw:
                    f = next((os.path.join(h, n) for n in names if os.path.exists(os.path.join(h, n))), None)
                    if f:
                        self._files[key] = f
                        break
            for key in ("pp_dpm_sclk", "pp_dpm_mclk"):
                if os.path.exists(os.path.join(dev, key)):
                    self._files[key] = os.path.join(dev, key)

    def _sample(self):
        f = self._files
        v = _read(f["sclk_hz"]) if "sclk_hz" in f else None
        sclk = float(v) / 1e6 if v and v.strip().isdigit() else (_dpm_mhz(_read(f["pp_dpm_sclk"]))
                                                                if "pp_dpm_sclk" in f else None)
        mclk = _dpm_mhz(_read(f["pp_dpm_mclk"])) if "pp_dpm_mclk" in f else None
        v = _read(f["power_uw"]) if "power_uw" in f else None
        power = float(v) / 1e6 if v and v.strip().isdigit() else None
        for k, x in (("sclk_mhz", sclk), ("mclk_mhz", mclk), ("power_w", power)):
            if x is not None:
                self.samples[k].append(x)

    def _loop(self):
        while not self._stop.is_set():
            self._sample()
            time.sleep(self.period)

    def __enter__(self):
        self._t = threading.Thread(target=self._loop, daemon=True)
        self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._t.join()

    def summary(self):
        if not self.dev:
            return {"unavailable": "no sysfs directory found for device 0"}
        out = {"n": len(self.samples["sclk_mhz"]), "source": {k: v for k, v in self._files.items()}}
        for k, xs in self.samples.items():
            if xs:
                out[k] = {"mean": round(statistics.mean(xs), 1), "min": round(min(xs), 1), "max": round(max(xs), 1)}
            else:
                out[k] = None
        return out


def sustain(graph, steps, per_kernel_ms, dev, seconds=1.0):
    """Replays a captured graph of `steps` launches back to back for about
    `seconds` while sampling clocks and power; returns the mean kernel time
    over that stretch and the sample summary."""
    import torch
    n = max(1, int(round(seconds * 1e3 / max(per_kernel_ms * steps, 1e-3))))
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with ClockSampler(dev) as cs:
        e0.record(stream)
        for _ in range(n):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
    return dict(sustained_us=round(e0.elapsed_time(e1) * 1e3 / (n * steps), 3), replays=n, **cs.summary())


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
        self.graph = None

    def step(self, i):
        st = self.runs[i % len(self.runs)].launch(self.op)
        if st != self.qg.OK:
            raise self.qg.QGemmError(st, "qg_run")

    def time(self, steps, warmup, dev=None):
        t, self.graph = graph_time(self.step, steps, warmup)
        if dev is not False:
            t["clocks"] = sustain(self.graph, steps, t["kernel_ms_mean"], dev)
        return t


def timeline(runs, op, launches=30, k_tiles=None):
    """Where the time of one split-K or data-parallel launch goes:
    qg_run_timed (the same plan, kernel and result as qg_run) launched
    `launches` times back to back over the workload's rotating input sets (as
    in the timed replays, so that the caches see the same stream); the last
    launch's per-unit timestamps (100 MHz clock) are summarised in
    microseconds. `mainloop_end_us` is when the last unit's mainloop ended,
    counted from the first unit's start; `fixup_read_us` and `store_us` are
    over the units that completed a tile. With `k_tiles` (k-tiles per unit),
    `cycles_per_k_tile` is the mean mainloop time in shader cycles (each
    unit's mainloop time at that unit's measured shader clock) per k-tile."""
    import numpy as np
    import torch
    import quantized_gemm_bf16_amd as qg
    st, units = runs[0].launch_timed(op, None)
    if units <= 0:
        return None
    stamps = torch.full((units * 8,), -1, dtype=torch.int64, device="cuda")
    for i in range(launches):
        st, _ = runs[i % len(runs)].launch_timed(op, stamps)
        if st != qg.OK:
            raise qg.QGemmError(st, "qg_run_timed")
    torch.cuda.synchronize()
    s = stamps.view(units, 8).cpu().numpy().astype(np.float64)
    done = s[:, 5] == 1
    t0 = s[:, 0].min()
    end = np.where(done, s[:, 4], s[:, 2])
    us = lambda x: round(float(x) / 100.0, 3)
    return {"units": int(units), "completing_units": int(done.sum()),
            "span_us": us(end.max() - t0), "last_start_us": us(s[:, 0].max() - t0),
            "mainloop_us_mean": us((s[:, 1] - s[:, 0]).mean()), "mainloop_us_max": us((s[:, 1] - s[:, 0]).max()),
            "mainloop_end_us": us(s[:, 1].max() - t0), "arrive_us_mean": us((s[:, 2] - s[:, 1]).mean()),
            "fixup_read_us": us((s[done, 3] - s[done, 2]).mean()), "store_us": us((s[done, 4] - s[done, 3]).mean()),
            "shader_clock_ghz": round(float(((s[:, 7] - s[:, 6]) / ((end - s[:, 0]) * 10.0)).mean()), 3),
            **({"cycles_per_k_tile": round(float(((s[:, 1] - s[:, 0]) * (s[:, 7] - s[:, 6]) / (end - s[:, 0])).mean())
                                           / k_tiles, 1), "k_tiles_per_unit": int(k_tiles)} if k_tiles else {}),
            "method": "qg_run_timed, 8 timestamps per unit, last of %d launches over %d input sets"
                      % (launches, len(runs))}


def ceiling_mfma(dev, grid=256, iters=2048, steps=20):
    """MFMA-only loop at one 8-wave workgroup per CU: sustained bf16 rate and
    the shader clock measured inside the loop."""
    import torch
    from quantized_gemm_bf16_amd import ceiling as qc
    sink = torch.empty(grid, dtype=torch.float32, device="cuda")
    clk = torch.zeros(2 * grid, dtype=torch.int64, device="cuda")
    t, graph = graph_time(lambda i: qc.mfma_loop(grid, iters, sink, clk), steps, 3)
    flops = grid * (qc.MFMA_THREADS // 64) * iters * qc.MFMA_FLOPS_PER_ROUND
    c = clk.view(-1, 2).cpu().double()
    sclk_ghz = float(c[:, 0].sum() / c[:, 1].sum()) * 0.1  # s_memrealtime ticks at 100 MHz
    tflops = flops / (t["kernel_ms_mean"] * 1e-3) / 1e12
    cl = sustain(graph, steps, t["kernel_ms_mean"], dev, seconds=0.5) if dev is not False else None
    return {"tflops": round(tflops, 1), "kernel_us_mean": round(t["kernel_ms_mean"] * 1e3, 3),
            "flops_per_launch": flops, "shader_clock_ghz_in_loop": round(sclk_ghz, 3),
            "flops_per_clk_per_cu": round(tflops * 1e12 / (sclk_ghz * 1e9 * 256), 1),
            "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
            "shape": f"{grid} workgroups x 8 waves x {iters} rounds of 4 v_mfma_f32_32x32x16_bf16", "clocks": cl}


def ceiling_stream(dev, nbytes, nsets=3, steps=30):
    """Streaming read of `nbytes` (rotating `nsets` buffers, together beyond
    the 256 MB Infinity Cache); the best of a few grid sizes."""
    import torch
    from quantized_gemm_bf16_amd import ceiling as qc
    bufs = [torch.full((nbytes // 4,), i + 1, dtype=torch.int32, device="cuda") for i in range(nsets)]
    blocks = -(-nbytes // qc.STREAM_BLOCK_BYTES)
    best = None
    for grid in sorted({blocks, -(-blocks // 2), 1024, 2048}):
        sink = torch.empty(grid * qc.STREAM_THREADS, dtype=torch.int32, device="cuda")
        t, graph = graph_time(lambda i: qc.stream_read(bufs[i % nsets], nbytes, grid, sink), steps, 3)
        gbs = nbytes / (t["kernel_ms_mean"] * 1e-3) / 1e9
        if best is None or gbs > best["GB/s"]:
            best = {"GB/s": round(gbs, 1), "kernel_us_mean": round(t["kernel_ms_mean"] * 1e3, 3), "grid": grid,
                    "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "graph": graph, "ms": t["kernel_ms_mean"]}
    graph, ms = best.pop("graph"), best.pop("ms")
    best["clocks"] = sustain(graph, steps, ms, dev, seconds=0.5) if dev is not False else None
    best["bytes_per_launch"] = nbytes
    return best


def issue_overlap(grid=256, iters=4096):
    """Shader cycles per round of qgc_issue_mix, until both waves of a SIMD
    are done: four 16x16x32 bf16 MFMAs per wave alone, sixteen VALU
    instructions of one kind per wave alone, and both interleaved; `hidden`
    is the share of the MFMA-only time that the VALU work hides,
    (mfma + valu - both) / mfma."""
    import torch
    from quantized_gemm_bf16_amd import ceiling as qc
    sink = torch.empty(grid, dtype=torch.float32, device="cuda")
    clk = torch.zeros(grid, dtype=torch.int64, device="cuda")

    def cycles(mode, kind):
        for _ in range(3):
            qc.issue_mix(mode, kind, grid, iters, sink, clk)
        torch.cuda.synchronize()
        return float(clk.double().mean()) / iters

    mf = cycles(1, 0)
    out = {"mfma": round(mf, 1)}
    for kind, name in qc.ISSUE_KINDS.items():
        v, b = cycles(2, kind), cycles(3, kind)
        out[name] = round(v, 1)
        out[name + "+mfma"] = round(b, 1)
        out["hidden_" + name] = round((mf + v - b) / mf, 3)
    out["unit"] = (f"shader cycles per round until both waves of a SIMD are done; a round is, per wave, "
                   f"{qc.ISSUE_MFMA_PER_ROUND} v_mfma_f32_16x16x32_bf16 and/or {qc.ISSUE_VALU_PER_ROUND} VALU "
                   f"instructions of the kind")
    return out


def graph_launch_floor(launches=100, reps=3):
    """Device time per launch of an empty kernel replayed from a HIP graph
    (the floor under every graph-replayed GEMM launch); median of reps."""
    import torch
    from quantized_gemm_bf16_amd import ceiling as qc
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        qc.empty()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for _ in range(launches):
                qc.empty()
        xs = []
        for _ in range(reps + 2):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            g.replay()
            e1.record(s)
            e1.synchronize()
            xs.append(e0.elapsed_time(e1) * 1e3 / launches)
    return round(statistics.median(xs[2:]), 3)


def host_timing(g, ws, n=500):
    """Host microseconds per qg_run on the decode problem (M=16), from a C loop
    of n back-to-back calls; median of three loops."""
    import torch
    import quantized_gemm_bf16_amd as qg
    from quantized_gemm_bf16_amd import ceiling as qc
    import synth
    from tests.gpu_util import Run
    r = Run(g, synth.config_decode(M=16), ws)

    def per_call(op):
        r.launch(op)
        torch.cuda.synchronize()
        xs = []
        for _ in range(3):
            xs.append(qc.host_us_per_run(n, g, op, r.p["alpha"], r.A, r.Ad, r.U, r.Ud, r.B, r.Bd, r.V, r.Vd,
                                         r.p["beta"], r.C, r.Cd, r.D, r.Dd, ws.desc))
            torch.cuda.synchronize()
        return round(statistics.median(xs), 3)

    out = {"default_memo": per_call(qg.operation())}
    st = r.launch(qg.operation(policy=qg.POLICY_MEASURE))
    torch.cuda.synchronize()
    if st == qg.OK:
        out["cache_hit"] = per_call(qg.operation(policy=qg.POLICY_REUSE))
    out["force"] = per_call(qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=8))
    # M = 0: qg_run validates the call and returns before planning or launching
    Ad0, Cd0, Dd0 = (qg.layout("bf16", 0, 14336), qg.layout("bf16", 0, 4096, ld=r.ldn),
                     qg.layout("bf16", 0, 4096, ld=r.ldn))
    out["validate_only_m0"] = round(statistics.median(
        qc.host_us_per_run(n, g, qg.operation(), 1.0, r.A, Ad0, None, None, r.B, r.Bd, None, None, 1.0, r.C, Cd0,
                           r.D, Dd0, ws.desc) for _ in range(3)), 3)
    for key, nb in (("empty_kernel_launch", 0), ("empty_kernel_256B_args_launch", 256)):
        xs = []
        for _ in range(3):
            xs.append(qc.host_us_per_empty(n, nb))
            torch.cuda.synchronize()
        out[key] = round(statistics.median(xs), 3)
    out["calls_per_loop"] = n
    out["problem"] = "decode M=16 N=4096 K=14336 bf16, C bf16, beta 1"
    return out


def cpu_model():
    for line in (_read("/proc/cpuinfo") or "").splitlines():
        if line.startswith("model name"):
            return line.split(":", 1)[1].strip()
    return None


def oracle_time(p, rows=None):
    import oracle
    t0 = time.perf_counter()
    oracle.gemm(p, rows=rows)
    return time.perf_counter() - t0


def oracle_rows_time(p, nrows=None):
    """The oracle (as it is) on a whole product, or on a seeded row sample
    with the full time extrapolated by rows."""
    import numpy as np
    if nrows is None or nrows >= p["M"]:
        return {"seconds": round(oracle_time(p), 3), "rows": "all"}
    rows = sorted(set(np.random.default_rng(11).choice(p["M"], size=nrows, replace=False).tolist()))
    dt = oracle_time(p, rows)
    return {"seconds_sample": round(dt, 3), "rows": f"{len(rows)} of {p['M']}",
            "seconds_full_estimate": round(dt * p["M"] / len(rows), 1)}


def oracle_timings(configs):
    """Host description and the oracle's time on the small 256^3 case (with
    all threads and with one), merged with the per-workload timings."""
    import oracle
    import synth
    out = {"cpu_model": cpu_model(), "affinity_cores": len(os.sched_getaffinity(0)),
           "omp_threads": oracle.num_threads()}
    tiny = synth.config_tiny()
    cfg = {"tiny_256^3_f32": {"seconds": round(oracle_time(tiny), 4), "rows": "all"}}
    prev = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        out["tiny_256^3_single_thread_s"] = round(oracle_time(tiny), 4)
    finally:
        oracle.set_num_threads(prev)
    cfg.update(configs)
    out["configs"] = cfg
    return out


def cpu_baseline(p, flops_per_row, target_s=15.0):
    """The oracle, as it is, on a row sample sized to about `target_s` seconds.
    Returns the cpu_baseline entry and the sample's timing."""
    import numpy as np
    import oracle
    rows = [0, 1]
    dt = max(oracle_time(p, rows), 1e-3)
    n = int(min(p["M"], max(2, round(target_s / (dt / len(rows))))))
    rows = sorted(set(np.random.default_rng(7).choice(p["M"], size=n, replace=False).tolist()))
    dt = oracle_time(p, rows)
    entry = dict(value=len(rows) * flops_per_row / dt / 1e12, unit="TFLOP/s", cores=oracle.num_threads(),
                 kind="oracle",
                 sample=f"{len(rows)} of {p['M']} rows of the {p['M']}x{p['N']}x{p['K']} product "
                        f"({len(rows) * p['N']} outputs, fp64, {dt:.1f} s)")
    return entry, {"seconds_sample": round(dt, 3), "rows": f"{len(rows)} of {p['M']}",
                   "seconds_full_estimate": round(dt * p["M"] / len(rows), 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle timings")
    ap.add_argument("--only", choices=["square", "decode", "w4a16", "moe", "moe_fp8", "ceilings", "host"],
                    default=None, help="time one workload only (profiling)")
    ap.add_argument("--no-extra", action="store_true", help="skip the W4A16 and MoE workloads")
    ap.add_argument("--no-clocks", action="store_true", help="skip the sustained replay with clock sampling")
    ap.add_argument("--no-timeline", action="store_true",
                    help="skip the qg_run_timed launches (profiling: the timed replay's dispatches come last)")
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
    dev = False if args.no_clocks else _sysfs_device()
    only = args.only
    cpu = not args.no_cpu and only is None
    oracle_cfg = {}

    out = {}
    M = N = K = 4096
    flops = 2.0 * M * N * K
    if only in (None, "square"):
        sq = Workload(g, ws, lambda i: synth.dense_problem(M, N, K, "bf16", "bf16", seed=synth.SEED_A + 10 * i),
                      nsets=4, op=qg.operation())
        kname = sq.runs[0].plan().split()[0].split("=")[1]
        t = sq.time(args.steps, args.warmup, dev)
        ms_step = t["total_ms"] / args.steps
        log(f"square {t['kernel_ms_mean'] * 1e3:.1f} us per launch")
        out["square"] = dict(t, kernel=kname, plan=sq.runs[0].plan(), tflops=flops / (ms_step * 1e-3) / 1e12,
                             kernel_tflops=flops / (t["kernel_ms_mean"] * 1e-3) / 1e12)
        pd = dict(kv.split("=") for kv in sq.runs[0].plan().split())
        if pd["schedule"] in ("dp", "splitk") and not args.no_timeline:
            kt = -(-(-(-K // int(pd["bk"]))) // int(pd["split"]))
            out["square"]["timeline"] = timeline(sq.runs, sq.op, k_tiles=kt)
            log(f"square timeline {out['square']['timeline']}")
        del sq

    if only in (None, "decode"):
        dec_bytes = 16 * 14336 * 2 + 4096 * 14336 * 2 + 2 * 16 * 4096 * 2
        res = {}
        for name, op in [("splitk8", qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_SPLITK, split_k=8)),
                         ("streamk", qg.operation(policy=qg.POLICY_FORCE, schedule=qg.SCHED_STREAMK, programs=256))]:
            # set 0 is the decode workload itself; the others only differ in seed
            dw = Workload(g, ws, lambda i: synth.dense_problem(16, 4096, 14336, "bf16", "bf16", c_dtype="bf16",
                                                               alpha=1.0, beta=1.0, a_std=0.02, b_std=0.02,
                                                               seed=synth.SEED_A + 10 * i), nsets=3, op=op)
            t = dw.time(max(20, args.steps), max(5, args.warmup), dev)
            res[name] = dict(kernel_us_mean=t["kernel_ms_mean"] * 1e3,
                             gbs=dec_bytes / (t["kernel_ms_mean"] * 1e-3) / 1e9,
                             frac_hbm=dec_bytes / (t["kernel_ms_mean"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
                             plan=dw.runs[0].plan(op), clocks=t.get("clocks"),
                             kernel=dw.runs[0].plan(op).split()[0].split("=")[1])
            log(f"decode {name} {t['kernel_ms_mean'] * 1e3:.2f} us per launch")
            if name == "splitk8" and not args.no_timeline:
                res[name]["timeline"] = timeline(dw.runs, op)
                log(f"decode {name} timeline {res[name]['timeline']}")
            if cpu and name == "splitk8":
                oracle_cfg["decode_16x4096x14336_bf16"] = oracle_rows_time(dw.runs[0].p)
            del dw
        out["decode"] = dict(bytes_per_call=dec_bytes, **res)

    extra = not args.no_extra and only is None
    if extra or only == "w4a16":
        # B 33.5 MB + scales 1 MB per set: 9 sets exceed the 256 MB Infinity Cache
        w4_bytes = 64 * 8192 * 2 + 8192 * 8192 // 2 + 8192 * 64 * 2 + 64 * 8192 * 2
        ww = Workload(g, ws, lambda i: synth.config_w4a16(), nsets=9, op=None, same_data=True)
        t = ww.time(args.steps, args.warmup, dev)
        us = t["kernel_ms_mean"] * 1e3
        log(f"w4a16 {us:.2f} us per launch")
        out["w4a16"] = {"kernel_us_mean": round(us, 3), "GB/s": round(w4_bytes / (us * 1e-6) / 1e9, 1),
                        "frac_hbm": round(w4_bytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                        "TFLOP/s": round(2.0 * 64 * 8192 * 8192 / (us * 1e-6) / 1e12, 2),
                        "bytes_per_call": w4_bytes, "plan": ww.runs[0].plan(), "clocks": t.get("clocks")}
        kn = ww.runs[0].plan().split()[0].split("=")[1]
        out["w4a16"]["traffic"] = traffic_from_profile(kn, "w4a16_64x8192x8192")
        if "schedule=splitk" in out["w4a16"]["plan"] and not args.no_timeline:
            out["w4a16"]["timeline"] = timeline(ww.runs, ww.op)
            log(f"w4a16 timeline {out['w4a16']['timeline']}")
        if cpu:
            oracle_cfg["w4a16_64x8192x8192"] = oracle_rows_time(ww.runs[0].p)
        del ww
    for fp8 in (False, True):
        name = "moe_fp8" if fp8 else "moe"
        if not (extra or only == name):
            continue
        # one set of 2.8 GB (bf16) / 1.4 GB (fp8) is far beyond every cache
        mw = Workload(g, ws, lambda i: synth.config_moe(fp8=fp8), nsets=1, op=None)
        p0 = mw.runs[0].p
        mflops = 2.0 * p0["M"] * p0["N"] * p0["K"]
        t = mw.time(max(10, args.steps // 5), max(3, args.warmup // 5), dev)
        us = t["kernel_ms_mean"] * 1e3
        log(f"{name} {us:.1f} us per launch")
        peak = PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS
        out[name] = {"kernel_us_mean": round(us, 1), "TFLOP/s": round(mflops / (us * 1e-6) / 1e12, 1),
                     "frac_peak": round(mflops / (us * 1e-6) / 1e12 / peak, 4), "peak": peak,
                     "flops_per_call": mflops, "plan": mw.runs[0].plan(), "clocks": t.get("clocks")}
        del mw
        if cpu:
            oracle_cfg[f"{name}_64x2048x7168"] = oracle_rows_time(p0, 256)
        del p0

    if only in (None, "ceilings"):
        out["ceilings"] = {"mfma_bf16": ceiling_mfma(dev)}
        log(f"mfma ceiling {out['ceilings']['mfma_bf16']['tflops']} TFLOP/s")
        out["ceilings"]["stream_read"] = ceiling_stream(dev, 4096 * 14336 * 2)
        log(f"stream ceiling {out['ceilings']['stream_read']['GB/s']} GB/s")
        out["ceilings"]["issue_overlap"] = issue_overlap()
        log(f"issue overlap {out['ceilings']['issue_overlap']}")
        out["ceilings"]["graph_launch_floor_us"] = graph_launch_floor()
        log(f"graph launch floor {out['ceilings']['graph_launch_floor_us']} us")
    if only in (None, "host"):
        out["host_us_per_call"] = host_timing(g, ws)
        log(f"host {out['host_us_per_call']}")

    if only:
        print(json.dumps(out))
        return 0

    sq_ = out["square"]
    ms_step = sq_["total_ms"] / args.steps
    achieved = sq_["kernel_tflops"]
    mf = out["ceilings"]["mfma_bf16"]
    stream = out["ceilings"]["stream_read"]
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
                     "traffic": traffic_from_profile(sq_["kernel"], "square_4096_bf16"),
                     "frac_of_sustained": round(achieved / mf["tflops"], 4),
                     "sustained_ceiling": "ceilings.mfma_bf16.tflops (MFMA-only loop, same process)"},
        "clocks": sq_.get("clocks"),
        "timeline": sq_.get("timeline"),
        "ceilings": out["ceilings"],
        "decode": {k: (round(v, 3) if isinstance(v, float) else v) for k, v in out["decode"].items()
                   if not isinstance(v, dict)},
    }
    for k in ("splitk8", "streamk"):
        d = out["decode"][k]
        line["decode"][k] = {"kernel_us_mean": round(d["kernel_us_mean"], 3), "GB/s": round(d["gbs"], 1),
                             "frac_hbm": round(d["frac_hbm"], 4),
                             "frac_of_stream": round(d["gbs"] / stream["GB/s"], 4),
                             "traffic": traffic_from_profile(d["kernel"], f"decode_16x4096x14336_{k}"),
                             "plan": d["plan"], "clocks": d["clocks"]}
    for k in ("w4a16", "moe", "moe_fp8"):
        if k in out:
            line[k] = out[k]
    line["host_us_per_call"] = out["host_us_per_call"]
    if not args.no_cpu:
        p = synth.config_square("bf16")
        line["cpu_baseline"], sample = cpu_baseline(p, 2.0 * N * K)
        log("cpu baseline done")
        del p
        line["cpu_oracle"] = oracle_timings({"square_4096^3_bf16": sample, **oracle_cfg})
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
