import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running (full-size workloads)")


def _ensure_built():
    """Build only what is missing (the build entry point rebuilds everything)."""
    import oracle
    import synth
    if not os.path.exists(oracle.LIB):
        oracle.build()
    if not os.path.exists(synth.HOST_LIB):
        from synth import build as sb
        sb.build_host()


_ensure_built()


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library through its Python binding; skips when no GPU is present."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_streaming_gemv_q8_amd as wsg
    wsg.lib()  # raises loudly if the HIP library is missing
    return wsg
