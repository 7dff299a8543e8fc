import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libquest")


def pytest_terminal_summary(terminalreporter):
    parity = sys.modules.get("parity")
    cases = getattr(parity, "RATE_READING_CASES", [])
    if cases:
        terminalreporter.write_line("in-band differences allowed by the rate reading of the 1e-5 mismatch bound:")
        for c in cases:
            terminalreporter.write_line(f"  {c}")
