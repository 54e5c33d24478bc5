import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built libmha.so")


def load_golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


@pytest.fixture(scope="session")
def gpu():
    """Skip when no GPU is visible; on a GPU machine the library must load."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import transformer_head_scaled_fwd_amd as mha
    mha.load()          # raises loudly if libmha.so is missing
    return torch.device("cuda:0")
