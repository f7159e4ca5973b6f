import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running host test")


import pytest  # noqa: E402


@pytest.fixture
def tuning():
    """Sets library tuning overrides for one test and restores the automatic
    choices afterwards."""
    from full_gqa_attention_layer_amd import hgqa
    knobs = []

    def set_knob(knob, value):
        knobs.append(knob)
        hgqa.set_tuning(knob, value)

    yield set_knob
    for knob in knobs:
        hgqa.set_tuning(knob, 0)
