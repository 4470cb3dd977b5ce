import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    """Skip GPU tests cleanly when no GPU is visible (they need an MI355X)."""
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


# Work space reserved once for the null stream, which every GPU test uses unless it says
# otherwise: enough for every split reduction the tests run (the largest, a split-K of up
# to 255 partial tiles of 256 x 256 fp32, is 255 MiB).
TEST_WORKSPACE_BYTES = 256 << 20
TEST_WORKSPACE_COUNTERS = 1 << 20


@pytest.fixture(autouse=True, scope="session")
def _reserve_workspace():
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        import tensor_transformer_linear_col_amd as tp
        tp.tp_workspace_reserve(TEST_WORKSPACE_BYTES, TEST_WORKSPACE_COUNTERS)
        torch.cuda.synchronize()
    yield


def golden_path(name: str) -> str:
    return os.path.join(ROOT, "tests", "golden", name)


def read_golden(name: str) -> dict:
    out = {}
    with open(golden_path(name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            out[key.strip()] = val.split()
    return out
