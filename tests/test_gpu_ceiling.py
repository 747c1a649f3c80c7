"""GPU checks of the measurement library (libqgceil.so) that the benchmark
reports ceilings with: the streaming read covers every byte once, the MFMA
loop reports a plausible clock and rate, the issue-overlap loops report
plausible cycle counts, the host loops and the graph launch floor return
figures."""
import numpy as np
import pytest
import torch

import quantized_gemm_bf16_amd as qg

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qc():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from quantized_gemm_bf16_amd import ceiling
    return ceiling


@pytest.mark.parametrize("nbytes, grid", [(16, 1), (32768, 1), (1 << 20, 7), ((5 << 20) + 48, 64), (117440512, 3584)])
def test_stream_read_reads_every_dword_once(qc, nbytes, grid):
    # XOR of every thread's fold is the XOR of the buffer; a dword read twice
    # or never would change it (random data)
    g = np.random.default_rng(nbytes % 1000)
    host = g.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.full((grid * qc.STREAM_THREADS,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    qc.stream_read(src, nbytes, grid, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


def test_mfma_loop_clock_and_rate(qc):
    grid, iters = 256, 512
    sink = torch.empty(grid, dtype=torch.float32, device="cuda")
    clk = torch.zeros(2 * grid, dtype=torch.int64, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    qc.mfma_loop(grid, iters, sink, clk)
    e0.record()
    qc.mfma_loop(grid, iters, sink, clk)
    e1.record()
    torch.cuda.synchronize()
    c = clk.view(-1, 2).cpu().double()
    assert (c > 0).all()
    ghz = float(c[:, 0].sum() / c[:, 1].sum()) * 0.1
    assert 0.5 < ghz < 3.0, ghz
    flops = grid * 8 * iters * qc.MFMA_FLOPS_PER_ROUND
    tflops = flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    # below the dense bf16 peak at the measured clock (4096 flop/clk/CU), and not absurdly low
    assert 100 < tflops <= 4096 * 256 * ghz * 1e9 / 1e12 * 1.02, (tflops, ghz)
    assert np.isfinite(sink.cpu().numpy()).all()


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_issue_mix_cycles(qc, kind):
    grid, iters = 256, 256
    sink = torch.empty(grid, dtype=torch.float32, device="cuda")
    clk = torch.zeros(grid, dtype=torch.int64, device="cuda")
    per = {}
    for mode in (1, 2, 3):
        qc.issue_mix(mode, kind, grid, iters, sink, clk)
        torch.cuda.synchronize()
        c = clk.cpu().double().numpy() / iters
        assert (c > 0).all() and np.isfinite(sink.cpu().numpy()).all()
        per[mode] = float(c.mean())
    # two waves per SIMD, timed until both are done: a round is at least
    # 2 waves x 4 MFMAs x 16 cycles; both together take at least each alone
    # (10 % slack for run-to-run noise) and at most their sum plus slack
    assert per[1] >= 0.9 * 128, per
    assert per[3] >= 0.9 * max(per[1], per[2]) and per[3] <= 1.3 * (per[1] + per[2]), per


def test_graph_launch_floor(qc):
    import bench
    us = bench.graph_launch_floor(launches=20, reps=2)
    assert 0.05 < us < 100, us


def test_host_loops(qc):
    import synth
    from tests.gpu_util import Run
    g, ws = qg.Gemm(), qg.workspace()
    r = Run(g, synth.dense_problem(16, 256, 512, "bf16", "bf16", seed=3), ws)
    op = qg.operation()
    us = qc.host_us_per_run(10, g, op, 1.0, r.A, r.Ad, None, None, r.B, r.Bd, None, None, 0.0, None, None, r.D, r.Dd,
                            ws.desc)
    torch.cuda.synchronize()
    assert 0 < us < 10000
    assert 0 < qc.host_us_per_empty(10) < 10000
    assert 0 < qc.host_us_per_empty(10, 256) < 10000
    torch.cuda.synchronize()
