import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running statistical test")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print the GPU parity counts (near-ties excluded per test and how they resolved)."""
    here = os.path.dirname(os.path.abspath(__file__))
    if here not in sys.path:
        sys.path.insert(0, here)
    import tie_report
    if tie_report.LINES:
        terminalreporter.section("parity counts (bit-exact / near-ties)")
        for line in tie_report.LINES:
            terminalreporter.write_line(line)
