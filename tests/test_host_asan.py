"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

The engine's host translation units (validation, planning, dispatch cache,
the no-allocation entry point's host side) are compiled with the sanitizers
on the host side only; the kernel translation units are the regular build's
objects (their device code is never sanitized, and no kernel is launched:
without a GPU every handle is offline). tests/asan/abi_asan.cpp drives every
exported call, including import of truncated, mutated and random cache text.
"""
import importlib.util
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_gemm_bf16_amd", "csrc")
HOST_TUS = ["qg_engine.cpp", "qg_registry.cpp", "qg_noalloc.hip"]
# sanitizers on the host side only (-Xarch_host before each flag)
SAN = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer"]


def _build_module():
    spec = importlib.util.spec_from_file_location("_qg_build_asan",
                                                  os.path.join(ROOT, "quantized_gemm_bf16_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    return b


@pytest.mark.timeout(900)
def test_c_abi_under_host_sanitizers(tmp_path):
    b = _build_module()
    if not os.path.exists(b.HIPCC):
        pytest.skip("hipcc not found")
    kernel_srcs = [s for s in b.sources() if os.path.basename(s) not in HOST_TUS]
    kernel_objs = [os.path.join(b.OUT_DIR, os.path.splitext(os.path.basename(s))[0] + ".o") for s in kernel_srcs]
    stale = [o for s, o in zip(kernel_srcs, kernel_objs)
             if not os.path.exists(o) or os.path.getmtime(o) < max(os.path.getmtime(os.path.join(CSRC, f))
                                                                   for f in os.listdir(CSRC))]
    if stale:
        b.build()
    objs = []
    for src in [os.path.join(CSRC, f) for f in HOST_TUS] + [os.path.join(ROOT, "tests", "asan", "abi_asan.cpp")]:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([b.HIPCC] + b.FLAGS + SAN + ["-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stdout + r.stderr
        objs.append(obj)
    exe = str(tmp_path / "abi_asan")
    r = subprocess.run([b.HIPCC, f"--offload-arch={b.ARCH}"] + SAN + ["-o", exe] + objs + kernel_objs,
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=99"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=98"
    env["HIP_VISIBLE_DEVICES"] = "-1"  # offline even where a GPU exists
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    if r.returncode == 77:
        pytest.skip("a GPU is visible to the test program")
    assert r.returncode == 0 and "abi_asan: ok" in out, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]


def test_hipcc_lines_keep_sanitizers_host_only():
    # every sanitizer flag above applies to the host side only
    for i, f in enumerate(SAN):
        if f.startswith("-f"):
            assert SAN[i - 1] == "-Xarch_host"
    assert shutil.which("true")
