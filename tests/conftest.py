import os
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

_TOWER = {"children": None, "dir": None}


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")
    config.addinivalue_line("markers", "tower_full: compares the full-size 27-block tower with oracle traces "
                                       "computed by background processes")


def pytest_collection_finish(session):
    """Start the full-size oracle traces as soon as the selected tests are
    known, so that they run beside the other GPU tests.  Only when such a
    test is selected and a GPU is present (device_count does not initialise
    the GPU runtime)."""
    jobs = set()
    for item in session.items:
        m = item.get_closest_marker("tower_full")
        if m is not None:
            jobs.update(m.kwargs.get("jobs", ()))
    if not jobs:
        return
    import torch
    if torch.cuda.device_count() < 1:
        return
    from tower_traces import Children
    _TOWER["dir"] = tempfile.mkdtemp(prefix="vit_tower_")
    _TOWER["children"] = Children(sorted(jobs), _TOWER["dir"])


def pytest_sessionfinish(session, exitstatus):
    ch = _TOWER["children"]
    if ch is not None:
        ch.stop()
        import shutil
        shutil.rmtree(_TOWER["dir"], ignore_errors=True)


@pytest.fixture(scope="session")
def tower_children():
    if _TOWER["children"] is None:
        pytest.fail("full-size oracle traces were not started (no GPU visible at collection)")
    return _TOWER["children"]


@pytest.fixture(scope="session")
def gpu():
    """Device handle for GPU tests; fails loudly if the HIP library is absent."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible to torch")
    import vision_transformer_encoder_amd as vit
    vit.require_library()
    return torch.device("cuda:0")
