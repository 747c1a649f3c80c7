"""Builds libqgemm.so (gfx950 only) in-tree with hipcc.

Every source under csrc/ is compiled on its own (in parallel) into _build/,
then linked into quantized_gemm_bf16_amd/libqgemm.so. The measurement
companion libqgceil.so (ceiling kernels for the benchmark) is built from
ceil/ the same way. Usage:
    python quantized_gemm_bf16_amd/build.py [--jobs N] [--save-temps]
(run as a script: importing the package itself needs the built library)
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqgemm.so")
CEIL_SRC = os.path.join(PKG, "ceil")
CEIL_LIB = os.path.join(PKG, "libqgceil.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-x", "hip",
         # keep hipcc from forming packed fp32 instructions
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def sources(d=CSRC):
    return sorted(os.path.join(d, f) for f in os.listdir(d) if f.endswith((".hip", ".cpp")))


def _compile(src, save_temps):
    obj = os.path.join(OUT_DIR, os.path.splitext(os.path.basename(src))[0] + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", src, "-o", obj]
    if save_temps:
        cmd.insert(1, "--save-temps")
    r = subprocess.run(cmd, cwd=OUT_DIR, capture_output=True, text=True)
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
    return obj, msgs


def _link(objs, lib):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)


def build(jobs: int = 0, save_temps: bool = False, verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs, ceil_srcs = sources(), sources(CEIL_SRC)
    jobs = jobs or min(len(srcs) + len(ceil_srcs), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, save_temps), srcs + ceil_srcs))
    objs = []
    for obj, msgs in results:
        objs.append(obj)
        if verbose and msgs:
            print("\n".join(msgs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], CEIL_LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--save-temps", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.save_temps, a.verbose))


if __name__ == "__main__":
    sys.exit(main())
