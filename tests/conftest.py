import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size configurations (minutes of CPU time)")


_INPUT_CACHE = {}


@pytest.fixture(scope="session")
def config_inputs():
    """Cached seeded inputs per configuration id (they are large)."""
    from sparse_attention_decode_csa_amd import inputs as I

    def get(cid):
        if cid not in _INPUT_CACHE:
            _INPUT_CACHE.clear()   # keep at most one big configuration alive
            _INPUT_CACHE[cid] = I.make_inputs(cid)
        return _INPUT_CACHE[cid]
    return get
