import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs through the HIP C-ABI")


@pytest.fixture
def tune():
    """tune(gemm=n, splitk=s, f8=c, ...) forces library tuning knobs for the rest of the test
    (through sl_set_tuning); the previous values are restored at teardown."""
    import sharded_linear_amd as sl
    saved = []

    def set_knobs(**knobs):
        if "gemm" in knobs:
            cfg = knobs.pop("gemm")
            knobs = {"fwd": cfg, "dgrad": cfg, "wgrad": cfg, **knobs}
        for k, v in knobs.items():
            saved.append((k, sl.sl_set_tuning(k, v)))

    yield set_knobs
    for k, v in reversed(saved):
        sl.sl_set_tuning(k, v)
