import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running case")


@pytest.fixture
def golden_dir():
    return GOLDEN


# TIDAR_LIBRARY=checked runs every call through the checked build: each GPU
# test then starts with cleared bounds-test records and appends what it left
# (if anything) to the file TIDAR_CHECK_LOG names, for reading after the run.
if os.environ.get("TIDAR_LIBRARY") == "checked":

    @pytest.fixture(autouse=True)
    def _check_records(request):
        if request.node.get_closest_marker("gpu") is None:
            yield
            return
        import diffusion_drafted_self_amd as tidar
        tidar.check_read(clear=True)
        yield
        rec = tidar.check_read(clear=True)
        if rec[0]:
            with open(os.environ.get("TIDAR_CHECK_LOG", "check_records.log"), "a") as f:
                f.write(f"{request.node.nodeid} {tidar.CHECK_CODES.get(rec[0], rec[0])} {rec}\n")
