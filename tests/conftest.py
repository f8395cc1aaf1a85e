import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def env():
    """(torch, the library binding, cuda:0) for the GPU tests."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X")
    import gemm_q4_q8_amd as qg
    return torch, qg, torch.device("cuda:0")


def golden(name: str) -> dict:
    """Parse a tests/golden key = value fixture ('#' starts a comment)."""
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            out[k] = v
    return out
