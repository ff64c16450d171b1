import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: larger CPU cases")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Per-comparison parity statistics of the GPU tests (raw max and mean absolute error against
    the float64 oracle, the bf16 rounding floor of the reference), one JSON line each, so that the
    session's log keeps them; also written to $PKV_PARITY_STATS_DIR/parity_stats.jsonl when that
    variable names a folder."""
    import json
    harness = sys.modules.get("gpu_harness")
    log = getattr(harness, "PARITY_LOG", None)
    if not log:
        return
    lines = [json.dumps(rec, sort_keys=True) for rec in log]
    worst = max(log, key=lambda r: r["max_abs"])
    worst_mean = max(log, key=lambda r: r["mean_abs"])
    terminalreporter.write_sep("-", f"parity statistics ({len(log)} comparisons)")
    for line in lines:
        terminalreporter.write_line("PARITY " + line)
    terminalreporter.write_line(
        f"PARITY-SUMMARY comparisons={len(log)} max_abs={worst['max_abs']:.4e} ({worst['label']}) "
        f"max_mean_abs={worst_mean['mean_abs']:.4e} ({worst_mean['label']}) "
        f"relaxed_elements={sum(r['n_relaxed'] for r in log)}")
    out = os.environ.get("PKV_PARITY_STATS_DIR", "")
    if out and os.path.isdir(out):
        with open(os.path.join(out, "parity_stats.jsonl"), "w") as f:
            f.write("\n".join(lines) + "\n")
