import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP path)")
    config.addinivalue_line("markers", "slow: long CPU-side check")


def pytest_collection_modifyitems(config, items):
    # GPU tests need a device; on a CPU-only machine they are skipped rather
    # than failed (the HIP library itself still refuses to run without one).
    try:
        import torch

        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU on this machine")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Near-tie counts of every routing comparison the GPU tests made: tokens
    whose oracle gap between the k-th and (k+1)-th score (set) or between
    kept scores (order) is below 1e-6, and how many of them the GPU routed
    differently (those are exempt from the exact check)."""
    try:
        from parity import NEAR_TIE_LOG
    except Exception:  # pragma: no cover
        return
    if not NEAR_TIE_LOG:
        return
    tr = terminalreporter
    tr.write_sep("-", "near-tie report (oracle gap < 1e-6)")
    tot = dict(tokens=0, near_set=0, near_order=0, exempt_set=0, exempt_order=0)
    for r in NEAR_TIE_LOG:
        for key in tot:
            tot[key] += r[key]
        if r["near_set"] or r["near_order"] or r["exempt_set"] or r["exempt_order"]:
            tr.write_line(f"{r['test']}: {r['tokens']} tokens, set gap {r['near_set']} "
                          f"(differ {r['exempt_set']}), order gap {r['near_order']} "
                          f"(differ {r['exempt_order']})")
    tr.write_line(f"all {len(NEAR_TIE_LOG)} routing checks: {tot['tokens']} tokens, set gap "
                  f"{tot['near_set']} (differ {tot['exempt_set']}), order gap "
                  f"{tot['near_order']} (differ {tot['exempt_order']})")
