import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running (full-size) GPU case")


def _ensure_built():
    """Build whatever is missing (never rebuilds what exists)."""
    import oracle
    import synth

    if not os.path.exists(oracle.LIB):
        oracle.build()
    if not (os.path.exists(synth.HOST_LIB) and os.path.exists(synth.DEV_LIB)):
        synth.build()
    try:
        import delta_rule_linear_kda_amd.build as kbuild
    except ImportError:
        return
    if not os.path.exists(kbuild.LIB_PATH):
        kbuild.build()


_ensure_built()
