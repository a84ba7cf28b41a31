import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (minutes)")


@pytest.fixture(scope="session")
def oracle():
    from oracle import oracle as O
    return O


@pytest.fixture(autouse=True)
def _parity_log_section():
    """Checks log under the workload their own test names (gpu_util.begin)."""
    yield
    gu = sys.modules.get("gpu_util")
    if gu is not None:
        gu._current["workload"] = None


def _ensure_built():
    lib = os.path.join(ROOT, "mixture_experts_expert_amd", "libmoe.so")
    if not os.path.exists(lib):
        from mixture_experts_expert_amd import build
        build.build()
    olib = os.path.join(ROOT, "oracle", "liboracle.so")
    if not os.path.exists(olib):
        from oracle import build as obuild
        obuild.build()


_ensure_built()
