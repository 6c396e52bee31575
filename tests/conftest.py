import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP library)")


@pytest.fixture(scope="session", autouse=True)
def _built_oracle():
    """Build the oracle only when nothing is built yet."""
    import oracle
    oracle.build(force=False)
    yield


@pytest.fixture(scope="session")
def hiplib():
    """The HIP library, built only when nothing is built yet."""
    from paged_kv_cache_269_amd import build as hipbuild
    if not os.path.exists(hipbuild.LIB_PATH):
        hipbuild.build()
    import paged_kv_cache_269_amd as pa
    return pa


@pytest.fixture(scope="session")
def cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")
