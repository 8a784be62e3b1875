import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: large CPU-side work")


import pytest  # noqa: E402


@pytest.fixture(scope="session")
def built_lib():
    """Path of libbitlinear.so, building it first only if nothing is built."""
    from bitlinear_w1_a8_amd import binding, build
    if not os.path.exists(binding.LIB_PATH):
        build.build(verbose=False)
    return binding.LIB_PATH
