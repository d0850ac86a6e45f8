import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


# Sanitizer runs (tests/test_sanitizers.py) point the oracle and the binding
# at instrumented builds of the same sources through these variables.
if os.environ.get("PALIMPSA_ORACLE_LIB"):
    import oracle
    oracle._LIB = os.environ["PALIMPSA_ORACLE_LIB"]
if os.environ.get("PALIMPSA_TEST_LIB"):
    from bayesian_metaplastic_memory_amd import _binding
    _binding.LIB_PATH = os.environ["PALIMPSA_TEST_LIB"]


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running full-size case")


def pytest_collection_modifyitems(config, items):
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
