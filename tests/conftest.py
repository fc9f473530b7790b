import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

_NEEDED = [
    os.path.join(ROOT, "long_context_sparse_12_amd", "liblcs.so"),
    os.path.join(ROOT, "synth", "libsynth_host.so"),
    os.path.join(ROOT, "synth", "libsynth_dev.so"),
    os.path.join(ROOT, "oracle", "liboracle.so"),
]
if not all(os.path.exists(p) for p in _NEEDED):
    import __graft_entry__

    __graft_entry__.build()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
