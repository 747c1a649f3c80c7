import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_sessionstart(session):
    # The C-ABI library and the oracle are built in-tree; build them if absent
    # (a machine that only runs the tests receives them prebuilt).
    lib = os.path.join(ROOT, "quantized_gemm_bf16_amd", "libqgemm.so")
    if not os.path.exists(lib):
        # loaded by path: the package's own import needs the library
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_qg_build", os.path.join(ROOT, "quantized_gemm_bf16_amd", "build.py"))
        b = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(b)
        b.build()
