import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long statistical run")


@pytest.fixture
def golden():
    import json

    def load(name):
        with open(os.path.join(GOLDEN, name)) as f:
            return json.load(f)
    return load


@pytest.fixture(scope="session")
def sv():
    """The binding of libspecverify.so; builds the library first if it is absent."""
    import importlib.util
    path = os.path.join(ROOT, "speculative_decoding_verification_gemm_amd", "build.py")
    spec = importlib.util.spec_from_file_location("_specverify_build", path)
    _build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(_build)
    if not os.path.exists(_build.LIB):
        _build.build()
    import speculative_decoding_verification_gemm_amd as mod
    return mod


@pytest.fixture(scope="session")
def dev(sv):
    """cuda:0, which must be an MI355X for the gpu-marked tests."""
    import torch
    assert torch.cuda.is_available(), "gpu-marked test needs a GPU"
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert name.startswith("gfx950"), f"needs gfx950, found {name}"
    return torch.device("cuda:0")
