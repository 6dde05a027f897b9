import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


def pytest_addoption(parser):
    parser.addoption("--stat-samples", type=int, default=12000,
                     help="emitted tokens per chi-square test (mlxcel PR #992 uses 12000)")


@pytest.fixture
def stat_samples(request):
    return request.config.getoption("--stat-samples")
