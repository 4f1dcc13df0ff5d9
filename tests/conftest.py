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
    beyond = getattr(parity, "BEYOND_TAU", None)
    if parity is None:
        return
    n_checks = len(beyond)
    terminalreporter.write_line(f"top-k set differences beyond one tolerance: {sum(beyond.values())} entries "
                                f"in {n_checks} row checks" + (f": {dict(list(beyond.items())[:20])}" if beyond else ""))
