import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def _ensure_built():
    """Build the in-tree libraries only when nothing is built yet."""
    need = [os.path.join(ROOT, "synth", "libsynth_host.so"),
            os.path.join(ROOT, "synth", "libsynth_dev.so"),
            os.path.join(ROOT, "gradient_sync_zero_amd", "libgsz.so")]
    if not all(os.path.exists(p) for p in need):
        import __graft_entry__
        __graft_entry__.build()


@pytest.fixture(scope="session", autouse=True)
def _built():
    _ensure_built()
