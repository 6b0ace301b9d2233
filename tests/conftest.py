import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large host-side work (full-size workloads)")


def pytest_terminal_summary(terminalreporter):
    import helpers
    if helpers.MARGINS:
        terminalreporter.section("parity margins (worst error / bound)")
        for line in helpers.MARGINS:
            terminalreporter.write_line(line)
