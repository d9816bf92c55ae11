import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests share one process and one device; run them after the CPU tests.
    items.sort(key=lambda it: 1 if it.get_closest_marker("gpu") else 0)


def pytest_terminal_summary(terminalreporter):
    """Per-output parity figures of the GPU tests (tokens compared, relative Frobenius error, max abs
    error over the reference rms, near-tie tokens), so that a quiet run still records them."""
    try:
        import parity_util
    except ImportError:
        return
    if not parity_util.RESULTS:
        return
    tr = terminalreporter
    tr.section("oracle parity")
    tr.write_line("%-34s %7s %11s %12s %6s" % ("output", "tokens", "rel Frob", "maxabs/rms", "ties"))
    for r in parity_util.RESULTS:
        mr = "-" if r["max_over_rms"] is None else "%.4f" % r["max_over_rms"]
        nt = "-" if r.get("near_ties") is None else str(r["near_ties"])
        tr.write_line("%-34s %7d %11.3e %12s %6s" % (r["label"][:34], r["n"], r["fro"], mr, nt))
