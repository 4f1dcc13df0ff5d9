import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """Top-k checks whose set differences reached past one score tolerance (all are still
    within two: see tests/parity.py)."""
    parity = sys.modules.get("tests.parity")
    if parity is None:
        return
    beyond = parity.BEYOND_TAU
    c = parity.TOPK_CHECKS
    terminalreporter.write_line(
        f"top-k row checks against the oracle: {c['rows']}; rows whose set differs: {c['rows_differing']} "
        f"({c['entries_differing']} entries, all within two tolerances of the K-th score); entries beyond one "
        f"tolerance: {sum(beyond.values())} in {len(beyond)} checks" +
        (f": {dict(list(beyond.items())[:20])}" if beyond else ""))
