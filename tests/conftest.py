import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test (large shapes)")


@pytest.fixture(scope="session")
def tiny_weights():
    from block_verify_amd.shapes import TINY, SEED_TARGET
    from block_verify_amd.synth import make_weights
    return make_weights(TINY, SEED_TARGET)


@pytest.fixture(scope="session")
def tiny_prompt():
    from block_verify_amd.shapes import TINY
    from block_verify_amd.synth import make_prompt
    return make_prompt(TINY.vocab, 128)
