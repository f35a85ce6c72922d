import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # Print the case name before each GPU test so a failing run names it.
    pass


@pytest.fixture(autouse=True)
def _announce(request):
    if request.node.get_closest_marker("gpu") is not None:
        print(f"\n[gpu-case] {request.node.nodeid}", flush=True)
    yield


def pytest_terminal_summary(terminalreporter):
    # Errors of the full-size parity runs, shown even under -q.
    mod = sys.modules.get("helpers")
    lines = getattr(mod, "SUMMARY", None) if mod is not None else None
    if lines:
        terminalreporter.write_sep("-", "parity statistics (every output against the oracle)")
        for line in lines:
            terminalreporter.write_line(line)
    worst = getattr(mod, "BWD_WORST", None) if mod is not None else None
    if worst:
        terminalreporter.write_sep("-", "backward errors as fractions of their derived bars")
        for dtype, (e, l2, le, ll) in sorted(worst.items()):
            terminalreporter.write_line(f"{dtype}: worst element {e:.4f} ({le}); worst L2 {l2:.4f} ({ll})")
