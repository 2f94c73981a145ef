import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long CPU-side oracle run")


def _ensure_host_libs():
    """Build the CPU libraries (generator, oracle) when nothing is built yet."""
    import synth
    import oracle
    if not os.path.exists(synth._LIB_PATH):
        synth.build()
    if not os.path.exists(oracle._LIB_PATH):
        oracle.build()


_ensure_host_libs()
