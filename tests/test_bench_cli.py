"""bench.py's command line on the CPU: a request for more than one GPU is
refused with a message before anything touches a device, and no result line
is printed."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    env = dict(os.environ)
    env["HIP_VISIBLE_DEVICES"] = "-1"  # never a device, even where one exists
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          env=env, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = run_bench("--gpus", n, "--steps", "1", "--warmup", "0")
        assert r.returncode == 2, r.stderr
        assert f"--gpus {n} is not supported" in r.stderr
        assert r.stdout.strip() == "", r.stdout


def test_no_device_exits_without_a_result_line():
    r = run_bench("--steps", "1", "--warmup", "0", "--no-cpu")
    assert r.returncode == 1, r.stderr
    assert "needs a GPU" in r.stderr
    assert r.stdout.strip() == "", r.stdout
