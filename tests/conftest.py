import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for p in (ROOT, os.path.dirname(os.path.abspath(__file__))):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(params=[128, 256], ids=["tile128", "tile256"])
def tile(request):
    """Run a GEMM test with the matrix-core stages forced to 128 x 128 or to 256 x 256
    output tiles (swg_set_gemm_tile), so both tile configurations meet every shape."""
    import swish_activation_backward_amd as swg
    print(f"[case] gemm tile {request.param}", flush=True)
    swg.swg_set_gemm_tile(request.param)
    yield request.param
    swg.swg_set_gemm_tile(0)
