import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: longer CPU test")


# BDATTN_TEST_DEBUG_CHECKS=1: every plan the tests make runs the record-checking
# kernels (BD_ATTN_FLAG_DEBUG_CHECKS), and every GPU test must end with no rejected
# work record on the device (the planted-record tests clear what they provoke).
if os.environ.get("BDATTN_TEST_DEBUG_CHECKS") == "1":
    import pytest

    from block_diffusion_attention_amd import binding as _b

    _plan_init = _b.Plan.__init__

    def _checked_plan_init(self, meta, flags=0):
        _plan_init(self, meta, flags | _b.FLAG_DEBUG_CHECKS)

    _b.Plan.__init__ = _checked_plan_init

    @pytest.fixture(autouse=True)
    def _no_rejected_records(request):
        yield
        if request.node.get_closest_marker("gpu") is not None:
            n = _b.device_check_errors(reset=True)
            assert n == 0, f"{n} workgroups rejected a work record"
