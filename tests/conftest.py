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
    # (the GPU machine receives them prebuilt).
    lib = os.path.join(ROOT, "quantized_gemm_bf16_amd", "libqgemm.so")
    if not os.path.exists(lib):
        from quantized_gemm_bf16_amd import build as _b
        _b.build()
