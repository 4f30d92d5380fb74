import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP library)")
    config.addinivalue_line("markers", "slow: larger CPU-only oracle checks")


@pytest.fixture(scope="session")
def tiny_weights():
    from autoregressive_tts_decode_amd import config, synth
    return synth.make_weights(config.TINY, seed=0)


@pytest.fixture(scope="session")
def tiny_cfg():
    from autoregressive_tts_decode_amd import config
    return config.TINY.as_dict()
