import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def pytest_collection_modifyitems(config, items):
    # GPU tests skip (with a reason) only when no GPU is visible at all; on a GPU
    # machine a missing or broken HIP library makes them fail, never fall back.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Margins of the floating-point parity checks (rel-L2 and max-abs / RMS
    against their limits), printed and written as JSON beside the run's other
    outputs (or to $QLORA_PARITY_MARGINS)."""
    from tests import parity
    if not parity.MARGINS:
        return
    import json
    rows = parity.MARGINS
    tr = terminalreporter
    tr.section("parity margins (rel-L2 limit %.0e, max/RMS limit %.0e)" % (parity.REL_L2, parity.MAX_ABS_OVER_RMS))
    worst_rel = max(rows, key=lambda t: t[2])
    worst_mx = max(rows, key=lambda t: t[3])
    tr.write_line(f"{len(rows)} checks; worst rel-L2 {worst_rel[2]:.3e} ({worst_rel[0]} {worst_rel[1]}); "
                  f"worst max/RMS {worst_mx[3]:.3e} ({worst_mx[0]} {worst_mx[1]})")
    for test, name, rel, mx in rows:
        tr.write_line(f"  {rel:.3e} {mx:.3e}  {name:4s} {test}")
    path = os.environ.get("QLORA_PARITY_MARGINS", os.path.join(ROOT, "gpurun_out", "parity_margins.json"))
    try:
        os.makedirs(os.path.dirname(path), exist_ok=True)
        with open(path, "w") as fh:
            json.dump([dict(test=t, output=n, rel_l2=r, max_over_rms=m) for t, n, r, m in rows], fh, indent=0)
    except OSError:
        pass
