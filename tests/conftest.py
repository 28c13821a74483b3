import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


# Test infrastructure only: the host-AddressSanitizer test runs the C-ABI
# battery against an instrumented copy of the library named here.
if os.environ.get("MXQ_TEST_LIB"):
    from float8_quantization_moe_amd import mxq as _mxq
    _mxq.LIB_PATH = os.environ["MXQ_TEST_LIB"]


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


@pytest.fixture
def group_knobs():
    """Force the group-scaling route for one test (mxq_set_group_scale_knobs);
    the automatic choice is restored afterwards."""
    from float8_quantization_moe_amd import mxq
    yield mxq.mxq_set_group_scale_knobs
    mxq.mxq_set_group_scale_knobs()
