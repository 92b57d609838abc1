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


def pytest_terminal_summary(terminalreporter):
    """Largest parity errors seen per workload tag (GPU runs), for the record."""
    import sys as _sys
    H = _sys.modules.get("tests.gpu_harness")
    if H is None or not getattr(H, "ERRORS", None):
        return
    tr = terminalreporter
    tr.section("largest errors against the oracle")
    tr.write_line(f"{'tag':<24}{'out max-abs':>14}{'out rel-L2':>14}{'H2O rel':>14}")
    for tag, e in sorted(H.ERRORS.items()):
        cols = [f"{e[k]:.3e}" if k in e else "-" for k in ("out_abs", "out_rel_l2", "h2o_rel")]
        tr.write_line(f"{tag:<24}{cols[0]:>14}{cols[1]:>14}{cols[2]:>14}")
