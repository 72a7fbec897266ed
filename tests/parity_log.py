"""Per-config parity records of the GPU tests (selection walks against the oracle).

Each record counts the walks compared, the bit-exact ones, the near-tie walks (the
oracle's K-th and (K+1)-th scores closer than 1e-3 at some scored level, by level),
and the mismatches by outcome of the near-tie validation. conftest.py prints every
record at the end of the session (one JSON line each) and, when PISA_PARITY_LOG names a
file, appends them to it.
"""
from __future__ import annotations

import json
import os

RECORDS: list = []


def add(record: dict) -> None:
    RECORDS.append(record)
    line = json.dumps(record, sort_keys=True)
    print(line, flush=True)
    path = os.environ.get("PISA_PARITY_LOG")
    if path:
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path, "a") as f:
            f.write(line + "\n")
