import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def repo_root():
    return ROOT


@pytest.fixture(autouse=True)
def _workspace_guard_bands(request, monkeypatch):
    """GPU tests: every workspace a test creates through DuoKV keeps its guard bands (the
    pattern duo_kv_init writes after each region) intact, checked when the handle is
    closed during the test and, for the handles still open, after it."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    import weakref
    from mixed_head_kv_amd import binding as B
    from parity_util import guard_violations
    live, bad = weakref.WeakSet(), []
    init, close = B.DuoKV.__init__, B.DuoKV.close

    def checked_init(self, *a, **kw):
        init(self, *a, **kw)
        live.add(self)

    def checked_close(self):
        if self.h:
            bad.extend(guard_violations(self))
        close(self)

    monkeypatch.setattr(B.DuoKV, "__init__", checked_init)
    monkeypatch.setattr(B.DuoKV, "close", checked_close)
    yield
    for kv in list(live):
        if kv.h:
            bad.extend(guard_violations(kv))
    assert not bad, f"workspace guard bands overwritten at byte offsets {bad[:8]}"
