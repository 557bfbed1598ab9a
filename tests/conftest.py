import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs through the C ABI")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle._load()          # builds liboracle.so with gcc when it is missing
    return oracle


@pytest.fixture(autouse=True)
def plan_opts():
    """Setter for the kernel choice / split count of the plans the GPU tests
    create through gpu_util.run_gemm (and of those they build with
    gpu_util.plan()); reset to the planner's own choice after each test."""
    import gpu_util
    import tiled_gemm_amd as tg

    def set_opts(kernel=None, splits=0):
        gpu_util.PLAN_OPTS["kernel"] = tg.KERNELS[kernel or "auto"]
        gpu_util.PLAN_OPTS["splits"] = int(splits)
    set_opts()
    yield set_opts
    set_opts()
