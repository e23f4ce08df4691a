import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU-side oracle work")


def load_golden(name):
    import json
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture
def golden():
    return load_golden


@pytest.fixture
def tuning():
    """Set libpkv tuning knobs for one test (pkv_set_tuning); every knob the
    test touched is put back to its value before the test."""
    from paged_attention_slot_amd import ops
    saved = {}

    def set_knob(name, value):
        if name not in saved:
            saved[name] = ops.get_tuning(name)
        ops.set_tuning(name, int(value or 0))
    yield set_knob
    for name, value in saved.items():
        ops.set_tuning(name, value)
