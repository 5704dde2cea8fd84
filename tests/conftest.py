import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size checks that take more than a few seconds")


def oracle_weights(w: dict) -> dict:
    """Storage-dtype CPU tensors (from synth.make_weights) -> fp32 numpy arrays for the oracle."""
    f = lambda t: None if t is None else t.float().numpy()
    return {
        "embed": f(w["embed"]), "final_norm": f(w["final_norm"]), "lm_head": f(w["lm_head"]),
        "layers": [{k: f(v) for k, v in layer.items()} for layer in w["layers"]],
    }


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")
