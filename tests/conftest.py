import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """Worst errors against the oracle of every full-size workload compared
    in this run (every head), shown even when output is captured."""
    mod = sys.modules.get("full_compare")
    lines = getattr(mod, "REPORT", None) if mod else None
    if lines:
        terminalreporter.section("errors against the fp64 oracle, every head")
        for ln in lines:
            terminalreporter.write_line(ln)
