import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size case, minutes of CPU work")


def pytest_collection_modifyitems(config, items):
    # GPU tests need a device; without one they are skipped, not failed.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU on this host")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """The worst parity error per compared quantity over the session (every
    GPU comparison goes through the harness's recorder)."""
    harness = sys.modules.get("beamrun")  # imported by the GPU tests only
    PARITY = getattr(harness, "PARITY", None)
    if not PARITY:
        return
    worst = {}
    for r in PARITY:
        w = worst.get(r["name"])
        if w is None or r["max_rel"] > w["max_rel"]:
            worst[r["name"]] = r
    tr = terminalreporter
    tr.write_line(f"parity: {len(PARITY)} comparisons; worst max|err|/rms(ref) per quantity "
                  "(router: max |err|/bound)")
    for name, r in sorted(worst.items(), key=lambda kv: -kv[1]["max_rel"])[:14]:
        tr.write_line(f"  {name:28s} {r['max_rel']:.2e}  rms(err) {r['rms_rel']:.1e}  "
                      f"{r['test'].split('::')[-1][:60]}")
