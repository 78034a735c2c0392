import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU-side test")


def oracle_inputs(w, device="cpu"):
    """(E, W) for the oracle from the seeded workload draws: float64 numpy arrays."""
    from oracle.link import as_f64
    import workloads as wl

    E = as_f64(wl.embedding_table(w, device))
    cache = {}

    def W(layer):
        if layer not in cache:
            cache[layer] = {k: as_f64(v) for k, v in wl.layer_weights(w, layer, device).items()}
        return cache[layer]

    return E, W


@pytest.fixture
def rng():
    return np.random.default_rng(1234)
