import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def _ensure_built():
    """Build the oracle and the HIP library only if nothing is built yet."""
    oracle_lib = os.path.join(ROOT, "oracle", "libg2oracle.so")
    hip_lib = os.path.join(ROOT, "attention_g2attn_prefill_amd", "libg2attn.so")
    if not os.path.exists(oracle_lib):
        from oracle import build as ob
        ob.build()
    if not os.path.exists(hip_lib):
        from attention_g2attn_prefill_amd import build as hb
        hb.build()


_ensure_built()


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")
