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


def pytest_terminal_summary(terminalreporter):
    """The router tests' smallest relative gap between neighbouring choices
    (a case below 2^-20 fails as ambiguous)."""
    try:
        from gpu_helpers import ROUTER_GAPS
    except ImportError:
        return
    if not ROUTER_GAPS:
        return
    what, gap = min(ROUTER_GAPS, key=lambda t: t[1])
    terminalreporter.write_line(
        f"router choice gaps: {len(ROUTER_GAPS)} cases, smallest {gap:.3e} ({what}); "
        f"ambiguous below {2.0 ** -20:.3e}")
