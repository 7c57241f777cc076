import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)

GOLDEN = os.path.join(ROOT, "tests", "golden")

_SERVICE = None


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")
    # The full-size parity checks evaluate the CPU oracle in worker processes
    # of a service forked here, before anything in this process touches the
    # GPU (collection below queries it in sessions that may run GPU tests).
    global _SERVICE
    if not config.getoption("collectonly", False):
        from oracle_service import OracleService

        _SERVICE = OracleService()


def pytest_unconfigure(config):
    global _SERVICE
    if _SERVICE is not None:
        _SERVICE.close()
        _SERVICE = None


@pytest.fixture(scope="session")
def oracle_service():
    if _SERVICE is None:
        pytest.skip("no oracle service in this session")
    return _SERVICE


def pytest_collection_modifyitems(config, items):
    # GPU tests run only where a GPU is present; on a CPU host they are skipped
    # (select them with -m gpu on a machine with an MI355X).  Sessions that
    # deselect them never query the GPU.
    if (config.getoption("markexpr", "") or "").replace(" ", "").startswith("notgpu"):
        return
    try:
        import torch

        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU on this host")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
