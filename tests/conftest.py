import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU work (full-size oracle runs)")


def _ensure_cpu_libs():
    # The generator and the oracle are plain C compiled with gcc; build them
    # only when nothing is built yet (build() in __graft_entry__ always rebuilds).
    import synth
    import oracle
    if not os.path.exists(synth.LIB_PATH):
        synth.build()
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()


_ensure_cpu_libs()


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)
