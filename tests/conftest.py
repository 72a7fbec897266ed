import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_collection_modifyitems(config, items):
    # GPU tests need a visible device; on a CPU-only host they are skipped, not failed.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


# The workloads whose every walk is compared (the five of the selection benchmark), reported
# last so that they sit next to the final pass/fail line.
_HEADLINE = ("prefill_tiny_", "prefill_short_", "prefill_mid_planted_", "prefill_long64k_", "prefill_long128k_",
             "prefill_long256k_", "decode128k_")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    try:
        import parity_log
    except ImportError:
        return
    recs = parity_log.RECORDS
    if not recs:
        return
    tr = terminalreporter
    tr.write_sep("-", f"selection parity against the oracle ({len(recs)} workloads)")
    head = [r for r in recs if r["config"].startswith(_HEADLINE) and "_mean" not in r["config"]]
    for r in recs:
        if r not in head:
            tr.write_line(_short(r))
    for r in head:
        tr.write_line(_short(r))


def _short(r) -> str:
    gap = r.get("min_gap")
    return (f"{r['config']}: {r['walks']} walks, {r['exact']} bit-exact, {r['near_tie_walks']} near-tie "
            f"(by level {r['near_tie_by_level']}), mismatches {r['mismatch_near_tie'] + r['hard_fail']} "
            f"(valid {r['mismatch_valid']}, invalid {r['mismatch_invalid']}, undecided {r['mismatch_unverified']}, "
            f"outside a near-tie {r['hard_fail']}), smallest gap {gap if gap is None else f'{gap:.3g}'}")
