import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter):
    """One line per parity case: tokens checked, near-tie tokens (K-th and
    (K+1)-th biased scores within 1e-5 in the oracle), tokens whose GPU set
    differs from the oracle's, the largest relative gate-weight error, the
    relative L2 error of the output over all checked tokens and its largest
    per-token value, and the largest element error as a fraction of its
    budget (tests/parity.py)."""
    parity = sys.modules.get("parity")
    rows = getattr(parity, "RESULTS", None) if parity else None
    if not rows:
        return
    tr = terminalreporter
    tr.write_sep("-", "parity summary (GPU vs oracle)")
    for r in rows:
        parts = [f"{r['case']}: n={r['tokens']}"]
        if "near_tie" in r:
            parts.append(f"near_tie={r['near_tie']} differ={r['differ']} w_rel={r['w_max_rel']:.1e}")
        if "rel_l2" in r:
            parts.append(f"l2={r['rel_l2']:.2e} tok_max={r['tok_max']:.2e} elem={r['elem_ratio']:.2f}")
        if "hist" in r:
            parts.append(f"hist={r['hist']} experts={r['experts']}")
        tr.write_line(" ".join(parts))
