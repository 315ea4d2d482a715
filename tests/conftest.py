import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")
    config.addinivalue_line("markers", "slow: large CPU work (full-size workload generation)")


def _gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Every attention comparison against the oracle, with its observed errors (printed whether or
    not output capture is on)."""
    parity = sys.modules.get("_parity")
    records = getattr(parity, "RECORDS", None)
    if not records:
        return
    tr = terminalreporter
    tr.section("attention errors against the fp64 oracle")
    tr.write_line(f"{'comparison':<44} {'elements':>9} {'max abs':>9} {'mean abs':>9} "
                  f"{'err/derived':>11}")
    for r in records:
        ratio = "" if r["ratio"] is None else f"{r['ratio']:.3f}"
        tr.write_line(f"{r['what'][:44]:<44} {r['n']:>9} {r['max']:>9.2e} {r['mean']:>9.2e} "
                      f"{ratio:>11}")
