import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: larger CPU cases")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle


@pytest.fixture(scope="session")
def dev():
    """The GPU for `gpu` tests; fails loudly (not skips) when absent."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("gpu test run without a visible GPU")
    return torch.device("cuda", torch.cuda.current_device())


@pytest.fixture(scope="session")
def pt(dev):
    """The HIP library binding; fails loudly when the extension is missing."""
    import moe_expert_grouped_gemm_amd as pt
    pt.load()
    return pt
