import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_collection_modifyitems(config, items):
    if torch.cuda.is_available():
        return
    skip = pytest.mark.skip(reason="no GPU in this process")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bf16 bit patterns of a CPU bf16 tensor as a uint16 numpy array."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def k_bits_of(inp) -> np.ndarray:
    """Bits of the cache storage (whole pitch); the oracle reads [..., :576] itself."""
    return bits(inp.k_storage.cpu())


def f64(t: torch.Tensor) -> np.ndarray:
    """bf16 -> float64 through torch (an exact conversion independent of the oracle's)."""
    return t.detach().cpu().to(torch.float64).numpy()
