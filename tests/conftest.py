import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU check")


def pytest_collection_modifyitems(config, items):
    # GPU tests carry the gpu marker explicitly; nothing else to do here.
    return


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Parity margins of the GPU comparisons of this session: per output, the
    largest max-scaled error as a fraction of its tolerance and the largest
    relative L2 error, with the test that produced each."""
    try:
        from tests import gpu_util
    except Exception:
        return
    rec = gpu_util.RECORD
    if not rec:
        return
    tr = terminalreporter
    tr.write_line(f"parity margins over {len(rec)} GPU-vs-oracle comparisons "
                  "(max scaled error / tolerance; relative L2 error):")
    for out in sorted({r["out"] for r in rec}):
        rs = [r for r in rec if r["out"] == out]
        a = max(rs, key=lambda r: r["max_scaled"] / r["tol"])
        b = max(rs, key=lambda r: r["rel_l2"])
        tr.write_line(f"  {out:>6}: worst {a['max_scaled'] / a['tol']:.3f} of tol ({a['max_scaled']:.2e} vs "
                      f"{a['tol']:g}, {a['test']}); worst rel-L2 {b['rel_l2']:.2e} ({b['test']})")
