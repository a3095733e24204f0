import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """The worst tolerance margins of the comparisons this session made."""
    gc = sys.modules.get("tests.gpu_common")
    if gc is not None and gc.MARGINS:
        terminalreporter.write_sep("-", "parity margins (worst over the session)")
        terminalreporter.write_line(gc.margins_report("session"))
