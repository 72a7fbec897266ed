"""Pins of the oracle's flat stage-one selection (oracle.flat_select).

The flat selection scores every eligible leaf summary against the query -- per block,
the sum over the GQA group's heads of q.kbar/sqrt(d) -- and keeps the K best (reading
note "Block Sparse Attention with Log-Linear Complexity", "Background: two stages, and
the bottleneck in the first"; the pyramid replaces exactly this scan). Pins that do not
restate that formula:
  * constant-key blocks give scores known in closed form (GQ * c_b / 8): the hand-derived
    selections, including exact ties broken toward the lower index and the causal cut;
  * for a position at the end of its block, a block's flat score equals the mean of its
    raw-key logits (oracle.node_score with the "mean" score, a separate code path that
    averages per-key logits): the flat set equals the top K by that score, and equals the
    mean-score walk wherever only the leaf level of the walk is scored;
  * brute force over all K-subsets: the selected set has the largest score total;
  * the own block is scored by its full mean, later keys included (a block whose later
    keys are large is selected at its first position);
  * structure: ascending, -1 padded, min(K, eligible) blocks, all eligible;
  * flat_validate accepts tied alternatives and rejects wrong sets.
"""
import itertools

import numpy as np
import pytest

import oracle

C, d = 64, 64


def _const_blocks(values, Hkv=1):
    N = len(values) * C
    k = np.zeros((N, Hkv, d), np.float32)
    for b, c in enumerate(values):
        k[b * C:(b + 1) * C, :, 0] = c
    return k


def test_closed_form_constant_blocks_with_ties():
    # 16 blocks; block b's keys are c_b * e_0, every query head is e_0: score = 4 * c_b / 8
    c = [0.5, 2.0, 2.0, -1.0, 3.0, 0.0, 2.0, 1.0, -2.0, 4.0, 2.0, 0.25, 1.0, 3.0, -3.0, 2.0]
    k = _const_blocks(c)
    N = k.shape[0]
    q = np.zeros((N, 4, d), np.float32)
    q[:, :, 0] = 1.0
    pyr = oracle.build_pyramid(k)
    K = 4
    # ranking over all 16 blocks: 9 (4.0), 4 (3.0), 13 (3.0), then the 2.0 tie 1, 2, 6, 10, 15 -> 1
    cases = {N - 1: [1, 4, 9, 13],
             # t in block 7: eligible 0..7, ranking 4 (3.0), then 2.0: 1, 2, 6 -> {1, 2, 4, 6}
             7 * C: [1, 2, 4, 6],
             # t in block 2: eligible 0..2 (at most K): all of them
             2 * C + 5: [0, 1, 2, -1],
             # t in block 4: eligible 0..4: 4 (3.0), 1, 2 (2.0), 0 (0.5) -> {0, 1, 2, 4}
             4 * C: [0, 1, 2, 4]}
    ts = np.array(sorted(cases))
    idx, gap = oracle.flat_select(q[ts], ts, pyr, N, K)
    for i, t in enumerate(ts):
        assert idx[i, 0].tolist() == cases[t], t
    # t = N - 1: 4th place is block 1 (2.0), 5th block 2 (2.0): an exact tie, gap 0;
    # t = 7 * C: 4th place block 6 (2.0), 5th block 7 (1.0): gap (2 - 1) / 2
    assert gap[list(ts).index(N - 1), 0] == 0.0
    assert gap[list(ts).index(7 * C), 0] == pytest.approx(0.5, abs=1e-12)


def test_closed_form_gap_values():
    c = [1.0, 2.0, 3.0, 4.0, 0.0, 0.0]
    k = _const_blocks(c)
    N = k.shape[0]
    q = np.zeros((N, 2, d), np.float32)
    q[:, :, 0] = 1.0                      # score = 2 * c_b / 8 = c_b / 4
    pyr = oracle.build_pyramid(k)
    ts = np.array([N - 1, 2 * C, 3 * C + 10])
    idx, gap = oracle.flat_select(q[ts], ts, pyr, N, 3)
    assert idx[0, 0].tolist() == [1, 2, 3] and gap[0, 0] == pytest.approx((2.0 - 1.0) / 4, abs=1e-12)
    assert idx[1, 0].tolist() == [0, 1, 2] and np.isinf(gap[1, 0])          # exactly K eligible
    assert idx[2, 0].tolist() == [1, 2, 3] and gap[2, 0] == pytest.approx(0.25, abs=1e-12)


def _random(N, Hq, Hkv, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((N, Hq, d), dtype=np.float32)
    k = rng.standard_normal((N, Hkv, d), dtype=np.float32)
    return q, k, oracle.build_pyramid(k)


def _mean_score_topk(q, k, pyr, t, j, K):
    n = t // C + 1
    s = np.array([oracle.node_score(q[t], t, j, k, pyr, 1, b, score="mean") for b in range(n)])
    order = sorted(range(n), key=lambda b: (-s[b], b))
    sel = sorted(order[:K])
    return sel + [-1] * (K - len(sel)), s


@pytest.mark.parametrize("Hq,Hkv,K", [(8, 2, 3), (6, 3, 5), (16, 1, 8)])
def test_equals_top_k_of_the_leaf_mean_score(Hq, Hkv, K):
    N = 1500
    q, k, pyr = _random(N, Hq, Hkv, seed=Hq + K)
    ts = np.array([63, 127, 64 * 7 + 63, 64 * 15 + 63, 64 * 22 + 63])
    idx, gap = oracle.flat_select(q[ts], ts, pyr, N, K)
    for i, t in enumerate(ts):
        for j in range(Hkv):
            want, s = _mean_score_topk(q, k, pyr, int(t), j, K)
            assert idx[i, j].tolist() == want, (t, j)
            if len(s) > K:
                ss = np.sort(s)[::-1]
                assert gap[i, j] == pytest.approx(ss[K - 1] - ss[K], abs=1e-9)


def test_equals_mean_score_walk_when_only_leaves_are_scored():
    # N = 1024: 16 leaves, 8 level-2 nodes; at K = 8 the walk keeps every level above the
    # leaves whole and scores the leaves alone, by the mean of their raw-key logits
    N, K = 1024, 8
    q, k, pyr = _random(N, 8, 2, seed=3)
    ts = np.arange(63, N, 64)
    idx, _ = oracle.flat_select(q[ts], ts, pyr, N, K)
    w_idx, _, _ = oracle.walk(q[ts], ts, k, pyr, K, score="mean")
    assert np.array_equal(idx, w_idx)


def test_brute_force_best_subset():
    N, K = 512, 3
    q, k, pyr = _random(N, 4, 1, seed=7)
    t = N - 1
    idx, _ = oracle.flat_select(q[[t]], np.array([t]), pyr, N, K)
    s = [oracle.node_score(q[t], t, 0, k, pyr, 1, b, score="mean") for b in range(N // C)]
    best = max(itertools.combinations(range(N // C), K), key=lambda sub: sum(s[b] for b in sub))
    assert idx[0, 0].tolist() == sorted(best)


def test_own_block_scored_by_its_full_mean():
    # block 5's keys from position 5*64 + 1 on are large along the query: at t = 5*64 only key
    # 320 of the block exists, yet the block's summary (its full mean) makes it the best
    N, K = 1024, 2
    rng = np.random.default_rng(5)
    q = np.zeros((N, 2, d), np.float32)
    q[:, :, 0] = 1.0
    k = rng.standard_normal((N, 1, d), dtype=np.float32) * 0.1
    k[5 * C + 1:6 * C, 0, 0] = 50.0
    pyr = oracle.build_pyramid(k)
    t = 5 * C
    idx, _ = oracle.flat_select(q[[t]], np.array([t]), pyr, N, K)
    assert 5 in idx[0, 0].tolist()
    w_idx, _, _ = oracle.walk(q[[t]], np.array([t]), k, pyr, K, score="mean")
    assert 5 not in w_idx[0, 0].tolist()     # the walk's leaf score sees key 320 only


def test_structure():
    N, K = 3001, 8
    q, k, pyr = _random(N, 8, 2, seed=11)
    ts = np.arange(N)
    idx, gap = oracle.flat_select(q, ts, pyr, N, K)
    for t in range(0, N, 37):
        for j in range(2):
            row = idx[t, j]
            n = min(K, t // C + 1)
            assert (row[:n] >= 0).all() and (row[n:] == -1).all()
            assert np.all(np.diff(row[:n]) > 0) and row[n - 1] <= t // C
            assert np.isinf(gap[t, j]) == (t // C + 1 <= K)


def test_flat_validate():
    c = [1.0, 2.0, 2.0, 2.0, 0.0, 3.0]
    k = _const_blocks(c)
    N = k.shape[0]
    q = np.zeros((N, 1, d), np.float32)
    q[:, 0, 0] = 1.0
    pyr = oracle.build_pyramid(k)
    t, K = N - 1, 3
    idx, gap = oracle.flat_select(q[[t]], np.array([t]), pyr, N, K)
    assert idx[0, 0].tolist() == [1, 2, 5] and gap[0, 0] == 0.0
    assert oracle.flat_validate(q[t], t, 0, pyr, N, K, [1, 2, 5], 1e-3) == 1
    assert oracle.flat_validate(q[t], t, 0, pyr, N, K, [3, 5, 1], 1e-3) == 1   # the other tied block
    assert oracle.flat_validate(q[t], t, 0, pyr, N, K, [1, 2, 3], 1e-3) == 0   # misses block 5
    assert oracle.flat_validate(q[t], t, 0, pyr, N, K, [1, 5, 5], 1e-3) == 0   # duplicate
    assert oracle.flat_validate(q[t], t, 0, pyr, N, K, [1, 5, -1], 1e-3) == 0  # too few
    assert oracle.flat_validate(q[3 * C], 3 * C, 0, pyr, N, K, [1, 2, 4], 1e-3) == 0   # 4 not eligible
