import os
import sys

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if REPO not in sys.path:
    sys.path.insert(0, REPO)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def gpu_lib():
    """The built HIP library on a GPU; fails loudly (no fallback) if either is missing."""
    import torch

    import top_sparse_mqa_amd as smqa

    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    if not smqa.LIB_PATH.exists():
        pytest.fail(f"{smqa.LIB_PATH} missing: build with `python -m top_sparse_mqa_amd.build` first")
    return smqa.load_library()
