"""The parity rule's host logic (tests/pisa_testlib.compare_selection), on the CPU.

The "GPU" results here are built from the oracle's own walks and then altered, so each
outcome of the rule is exercised: bit-exact walks, a tied alternative that validates, a
set that no resolution of the ties reaches, and a mismatch outside any near-tie.
"""
import numpy as np

import oracle
from pisa_testlib import compare_selection


def _zero_key_case():
    # all keys zero: every full leaf ties exactly (gap 0) wherever more than K are eligible
    N, K = 2048, 4
    rng = np.random.default_rng(1)
    q = rng.standard_normal((N, 4, 64), dtype=np.float32)
    k = np.zeros((N, 1, 64), np.float32)
    return q, k, oracle.build_pyramid(k), K


def test_identical_results_are_exact():
    q, k, pyr, K = _zero_key_case()
    ts = np.arange(0, 2048, 7)
    idx, gap, lvl = oracle.walk(q[ts], ts, k, pyr, K)
    rep = compare_selection(idx.copy(), ts, q, k, pyr, K)
    assert rep.ok() and rep.exact == rep.walks == len(ts)
    assert rep.near_tie_walks == int((gap < 1e-3).sum()) > 0
    assert sum(rep.near_tie_by_level.values()) == rep.near_tie_walks
    rec = rep.record("zero_keys")
    assert rec["config"] == "zero_keys" and rec["walks"] == len(ts) and rec["min_gap"] == 0.0


def test_tied_alternative_validates_and_wrong_set_fails():
    q, k, pyr, K = _zero_key_case()
    t = 2047
    ts = np.array([t])
    idx, gap, _ = oracle.walk(q[ts], ts, k, pyr, K)
    assert gap[0, 0] == 0.0
    # the lowest-index resolution of the ties selects leaves 0..3; leaves 0, 1, 2, 3 lie under
    # level-2 nodes 0 and 1, so swapping the pair (2, 3) for (4, 5) changes a tied upper choice
    assert idx[0, 0].tolist() == [0, 1, 2, 3]
    alt = np.array([[[0, 1, 4, 5]]], np.int32)
    rep = compare_selection(alt, ts, q, k, pyr, K)
    assert rep.ok() and rep.mismatch_valid == 1 and rep.exact == 0
    bad = np.array([[[0, 1, 2, -1]]], np.int32)          # one slot dropped: no resolution gives it
    rep = compare_selection(bad, ts, q, k, pyr, K)
    assert not rep.ok() and rep.mismatch_invalid == 1


def test_mismatch_outside_a_near_tie_is_a_hard_failure():
    rng = np.random.default_rng(2)
    N, K = 1024, 4
    q = rng.standard_normal((N, 4, 64), dtype=np.float32)
    k = rng.standard_normal((N, 1, 64), dtype=np.float32)
    pyr = oracle.build_pyramid(k)
    ts = np.arange(N)
    idx, gap, _ = oracle.walk(q, ts, k, pyr, K)
    far = np.nonzero((gap[:, 0] > 1e-2) & (ts >= 8 * 64))[0]
    i = int(far[0])
    got = idx.copy()
    got[i, 0, 0] = (got[i, 0, 0] + 1) % (ts[i] // 64 + 1) if got[i, 0, 0] + 1 not in got[i, 0] else -1
    rep = compare_selection(got, ts, q, k, pyr, K)
    assert not rep.ok() and rep.hard_fail == 1 and rep.first_fail[0] == int(ts[i])
