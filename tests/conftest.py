import os
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


def pytest_sessionfinish(session, exitstatus):
    """Writes the boundary-case counts and worst relative L2 of every GPU parity
    configuration checked in this session to parity_report.json in the folder
    PARITY_REPORT_DIR names (by default the system's temporary folder)."""
    import json
    import sys
    helpers = sys.modules.get("tests.gpu_helpers")
    reports = getattr(helpers, "SESSION_REPORTS", None) if helpers else None
    if not reports:
        return
    out = os.environ.get("PARITY_REPORT_DIR") or tempfile.gettempdir()
    os.makedirs(out, exist_ok=True)
    total = dict(configs=len(reports), heads=0, targets=0, boundary_cases=0, boundary_mismatches=0,
                 worst_rel_l2=0.0)
    for r in reports.values():
        for key in ("heads", "targets", "boundary_cases", "boundary_mismatches"):
            total[key] += r[key]
        total["worst_rel_l2"] = max(total["worst_rel_l2"], r["worst_rel_l2"])
    with open(os.path.join(out, "parity_report.json"), "w") as f:
        json.dump({"exit_status": int(exitstatus), "total": total, "by_config": reports}, f, indent=1,
                  sort_keys=True)
