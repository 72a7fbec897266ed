"""Pins of the oracle's two truncated scores (the ablation variants of the pages).

The reading note's "Scoring: LogSumExp" section expands the LSE of a
candidate's m child logits around their mean: dropping log m, the first-order
truncation is the mean of the logits ("PISA-1") and the second-order one the
mean plus half their variance ("PISA-2"). The oracle's "mean" and
"mean_half_var" scores are checked here against things other than their own
formula: the linearity of the mean (the mean of the logits of a node's raw keys
is the logit of the node's mean key), the order of the expansion's remainder
(third order for the second-order score, second for the first-order one),
hand-derived values, and flat top-K when only the leaf level is scored.
"""
import math

import numpy as np
import pytest

import oracle
from block_selection_amd import synth


def _rand_qk(N, Hq, Hkv, d=64, seed=1):
    rng = np.random.default_rng(seed)
    q = synth.bf16_round(rng.standard_normal((N, Hq, d), dtype=np.float32))
    k = synth.bf16_round(rng.standard_normal((N, Hkv, d), dtype=np.float32))
    return q, k


def test_mean_score_is_the_logit_of_the_node_mean():
    """Mean of child logits = logit of the raw-key mean: fully eligible nodes, and leaf prefixes."""
    N, Hq, Hkv, d = 4096, 8, 2, 64
    GQ = Hq // Hkv
    q, k = _rand_qk(N, Hq, Hkv, seed=3)
    pyr = oracle.build_pyramid(k)
    rng = np.random.default_rng(0)
    cases = [(1, 5, 5 * 64 + 17), (1, 10, 10 * 64), (1, 63, 4095), (2, 7, 4095), (3, 2, 4095),
             (5, 1, 4095), (7, 0, 4095), (4, 3, 4095)]
    for lvl, node, t in cases:
        span = 64 * 2 ** (lvl - 1)
        lo = node * span
        hi = min(lo + span, t + 1) if lvl == 1 else lo + span   # upper nodes: all children eligible
        for j in range(Hkv):
            kmean = k[lo:hi, j].astype(np.float64).mean(axis=0)
            qt = q[int(rng.integers(0, N))].astype(np.float64)
            want = sum(float(qt[j * GQ + h] @ kmean) / math.sqrt(d) for h in range(GQ))
            got = oracle.node_score(qt.astype(np.float32), t, j, k, pyr, lvl, node, score="mean")
            assert abs(got - want) <= 1e-9 * max(1.0, abs(want)), (lvl, node, t, j, got, want)


@pytest.mark.parametrize("level,node", [(1, 3), (2, 5), (4, 1)])
def test_truncation_orders_of_the_lse_expansion(level, node):
    """LSE - log m - (mean + var/2) shrinks at least as the cube of the logit spread, LSE - log m - mean as its square."""
    N, Hq, Hkv = 2048, 4, 1
    q, k = _rand_qk(N, Hq, Hkv, seed=11)
    pyr = oracle.build_pyramid(k)
    t = N - 1
    m = 64 if level == 1 else 2
    q0 = q[100].astype(np.float64)
    err = {"mean": [], "mean_half_var": []}
    for eps in (0.08, 0.04, 0.02):
        qe = (q0 * eps).astype(np.float32)
        lse = oracle.node_score(qe, t, 0, k, pyr, level, node, score="lse") - Hq * math.log(m)
        for s in err:
            err[s].append(abs(lse - oracle.node_score(qe, t, 0, k, pyr, level, node, score=s)))
    # first-order score: remainder exactly second order (half the variance is missing);
    # second-order score: at least third order (fourth for two children, whose logits are
    # symmetric about their mean). A wrong variance factor or normalisation leaves a
    # second-order remainder and fails the second check.
    for a, b in zip(err["mean"], err["mean"][1:]):
        assert 0.8 * 4 < a / b < 1.25 * 4, err["mean"]
    for a, b in zip(err["mean_half_var"], err["mean_half_var"][1:]):
        assert a / b > 0.8 * 8, err["mean_half_var"]


def test_hand_derived_values():
    """Two leaves with mean logits a and b under one level-2 node; a leaf with alternating logits."""
    d, C = 64, 64
    N = 4 * C
    k = np.zeros((N, 1, d), np.float32)
    # q has sqrt(d) in its first coordinate, so a key's logit is its first coordinate
    k[0:C, 0, 0] = 1.5                      # leaf 0: every logit 1.5
    k[C:2 * C, 0, 0] = -0.5                 # leaf 1: every logit -0.5
    k[2 * C:3 * C, 0, 0] = np.tile([1.0, -1.0], C // 2)   # leaf 2: logits +1, -1, ...
    q = np.zeros((1, 3, d), np.float32)     # three heads of one group
    q[0, :, 0] = math.sqrt(d)
    pyr = oracle.build_pyramid(k)
    t = N - 1
    # level-2 node 0 over leaves 0, 1: mean 0.5; variance ((1.5 - -0.5) / 2)^2 = 1
    assert oracle.node_score(q[0], t, 0, k, pyr, 2, 0, score="mean") == pytest.approx(3 * 0.5, abs=1e-12)
    assert oracle.node_score(q[0], t, 0, k, pyr, 2, 0, score="mean_half_var") == pytest.approx(3 * 1.0, abs=1e-12)
    # leaf 2: mean 0, population variance 1
    assert oracle.node_score(q[0], t, 0, k, pyr, 1, 2, score="mean") == pytest.approx(0.0, abs=1e-12)
    assert oracle.node_score(q[0], t, 0, k, pyr, 1, 2, score="mean_half_var") == pytest.approx(3 * 0.5, abs=1e-12)
    # masked to its first three keys (+1, -1, +1): mean 1/3, variance 8/9
    t3 = 2 * C + 2
    assert oracle.node_score(q[0], t3, 0, k, pyr, 1, 2, score="mean_half_var") == pytest.approx(
        3 * (1 / 3 + 4 / 9), abs=1e-12)


def _flat_topk(q_row, k, t, j, K, GQ, score):
    d = k.shape[2]
    out = []
    for b in range(t // 64 + 1):
        keys = k[b * 64:min(b * 64 + 64, t + 1), j].astype(np.float64)
        s = 0.0
        for h in range(GQ):
            z = keys @ q_row[j * GQ + h].astype(np.float64) / math.sqrt(d)
            s += z.mean() + (0.5 * z.var() if score == "mean_half_var" else 0.0)
        out.append((-s, b))
    out.sort()
    sel = sorted(b for _, b in out[:K])
    return sel + [-1] * (K - len(sel))


@pytest.mark.parametrize("score", ["mean", "mean_half_var"])
@pytest.mark.parametrize("N,K", [(1024, 8), (1000, 8), (512, 4)])
def test_walk_equals_flat_topk_when_no_upper_level_is_scored(score, N, K):
    """Only the leaf level scored: the walk is flat top-K of the truncated raw-key score."""
    assert oracle.level_sizes(N)[1] <= K
    Hq, Hkv = 4, 2
    q, k = _rand_qk(N, Hq, Hkv, seed=N + K + 7)
    pyr = oracle.build_pyramid(k)
    ts = np.arange(N)
    idx, _, _ = oracle.walk(q, ts, k, pyr, K, score=score)
    rng = np.random.default_rng(1)
    for t in sorted(set(rng.integers(0, N, 40).tolist()) | {0, N - 1, K * 64 - 1, K * 64}):
        if t >= N:
            continue
        for j in range(Hkv):
            assert idx[t, j].tolist() == _flat_topk(q[t], k, t, j, K, Hq // Hkv, score), (t, j)


def test_scores_agree_when_every_child_logit_is_equal():
    """Equal child logits: LSE - log m = mean = mean + var/2 (zero variance)."""
    d, C = 64, 64
    N = 8 * C
    k = np.zeros((N, 1, d), np.float32)
    k[:, 0, 0] = 0.75
    q = np.zeros((1, 2, d), np.float32)
    q[0, :, 0] = math.sqrt(d)
    pyr = oracle.build_pyramid(k)
    for lvl, node, m in ((1, 3, 64), (2, 1, 2), (3, 0, 2)):
        lse = oracle.node_score(q[0], N - 1, 0, k, pyr, lvl, node, score="lse") - 2 * math.log(m)
        for s in ("mean", "mean_half_var"):
            assert oracle.node_score(q[0], N - 1, 0, k, pyr, lvl, node, score=s) == pytest.approx(lse, abs=1e-12)
