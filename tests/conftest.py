import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and libcoli.so")
    config.addinivalue_line("markers", "slow: full-size oracle runs (minutes of CPU)")


@pytest.fixture(scope="session")
def orc():
    from oracle import oracle
    oracle.lib()
    return oracle


@pytest.fixture(scope="session")
def glm_bank():
    """256 experts of width 6144 x 2048, int4 (4.8 GB host), plus the shared
    expert: the decode, layer and prefill workloads' expert bank."""
    from weight_streaming_gemv_qgemv_amd import synth
    bank = synth.expert_bank(3000, 2, 256, 6144, 2048)
    shared = synth.shared_mlp(3000, 2, 6144, 2048)
    return bank, shared
