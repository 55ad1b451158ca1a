import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    oracle.lib()
    return oracle


_LAYER_CACHE = {}


def cached_layer(name: str, **overrides):
    """Seeded workload inputs, drawn once per test session."""
    key = (name, tuple(sorted(overrides.items())))
    if key not in _LAYER_CACHE:
        from bit_block_scaled_topk_amd import synth
        _LAYER_CACHE[key] = synth.make_layer(name, **overrides)
    return _LAYER_CACHE[key]
