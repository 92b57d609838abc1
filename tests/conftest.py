import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def golden():
    import json
    with open(os.path.join(ROOT, "tests", "golden", "page_values.json")) as f:
        return json.load(f)


@pytest.fixture(scope="session")
def kvq():
    """The ABI binding with libkvq.so loaded (built first only if it is missing)."""
    from kv_cache_compression_kvq_amd import abi
    if not os.path.exists(abi.LIB_PATH):
        from kv_cache_compression_kvq_amd import build
        build.build()
    abi.lib()
    return abi
