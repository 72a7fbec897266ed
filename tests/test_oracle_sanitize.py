"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/oracle_sanitize_main.c calls every entry point of oracle/pisa_oracle.c on small
inputs: ragged lengths, group sizes 1-16, K = 1-32, the three scores, traces, node
scores, attention, and near-tie validation, including an invalid target whose tied
ancestors fill the band while K - 1 candidates are surely kept. The driver is built with
gcc and both sanitizers (host code only; no GPU is involved) and must exit cleanly.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-O2", "-g", "-std=c11", "-fopenmp", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           os.path.join(HERE, "oracle_sanitize_main.c"), os.path.join(ROOT, "oracle", "pisa_oracle.c"),
           "-lm", "-o", exe]
    subprocess.check_call(cmd)
    env = dict(os.environ, OMP_NUM_THREADS="4", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "all checks passed" in r.stdout


def test_validate_rejects_target_over_tied_band():
    """16 leaves, only the leaf level scored: leaves 0..6 score log 64 + 1/8, leaves 7..15
    tie exactly at log 64 (zero keys). A target of eight band leaves that omits the seven
    surely kept ones is unreachable (0); swapping one tied leaf for another is reachable (1)."""
    N, C, d, K = 1024, 64, 64, 8
    q = np.zeros((N, 1, d), np.float32)
    q[:, 0, 0] = 1.0
    k = np.zeros((N, 1, d), np.float32)
    k[: 7 * C, 0, 0] = 1.0
    pyr = oracle.build_pyramid(k)
    t = N - 1
    idx, gap, _ = oracle.walk(q[[t]], np.array([t]), k, pyr, K)
    assert idx[0, 0].tolist() == list(range(8))
    assert gap[0, 0] == 0.0
    assert oracle.validate(q[t], t, 0, k, pyr, K, np.arange(8, 16), 1e-3) == 0
    assert oracle.validate(q[t], t, 0, k, pyr, K, [0, 1, 2, 3, 4, 5, 6, 15], 1e-3) == 1
    assert oracle.validate(q[t], t, 0, k, pyr, K, [1, 2, 3, 4, 5, 6, 14, 15], 1e-3) == 0
