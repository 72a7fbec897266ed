"""Pins of the oracle's exact flat selection (oracle.flat_exact_select).

Every eligible leaf block is scored as the walk scores a leaf candidate -- per block, the sum
over the GQA group's heads of the LSE of q.k/sqrt(d) over the block's raw keys up to t
(reading note "Block Sparse Attention with Log-Linear Complexity", "Scoring: LogSumExp" and
section 4.1) -- and the K best are kept, with no hierarchy. Pins that do not restate the C
code:
  * numpy brute force on small inputs: per block a log-sum-exp taken around its maximum in
    float64, the group sum, then a stable sort by (score desc, block asc);
  * wherever the walk scores only the leaf level (at most K nodes on level 2), the walk's
    selection (oracle.walk, the leaf scoring of the hierarchy) is the exact flat selection;
  * a block made of one repeated key scores log(m) + q.k/8 per head exactly (m keys <= t): the
    hand-derived selection, with the causal cut inside the query's own block;
  * structure: ascending, -1 padded, min(K, eligible) blocks, all eligible;
  * flat_exact_validate accepts the selection and a tied alternative, and rejects a set
    missing a surely-kept block or holding an ineligible one.
"""
import numpy as np

import oracle

C, d = 64, 64


def _brute(q_row, t, k, K, j):
    N, Hkv, _ = k.shape
    GQ = q_row.shape[0] // Hkv
    n = min(t // C + 1, -(-N // C))
    scores = []
    for b in range(n):
        keys = k[b * C:min((b + 1) * C, t + 1, N), j].astype(np.float64)
        tot = 0.0
        for hh in range(GQ):
            z = keys @ q_row[j * GQ + hh].astype(np.float64) / np.sqrt(d)
            m = z.max()
            tot += m + np.log(np.exp(z - m).sum())
        scores.append(tot)
    order = sorted(range(n), key=lambda b: (-scores[b], b))
    keep = sorted(order[:K])
    return keep + [-1] * (K - len(keep)), scores


def test_brute_force_small():
    rng = np.random.default_rng(4)
    N, Hq, Hkv, K = 700, 6, 2, 3
    q = rng.standard_normal((N, Hq, d)).astype(np.float32)
    k = rng.standard_normal((N, Hkv, d)).astype(np.float32)
    ts = np.array([0, 1, 63, 64, 65, 127, 128, 200, 300, 450, 640, 699])
    idx, gap = oracle.flat_exact_select(q[ts], ts, k, K)
    for i, t in enumerate(ts):
        for j in range(Hkv):
            want, sc = _brute(q[t], int(t), k, K, j)
            assert idx[i, j].tolist() == want, (t, j)
            srt = sorted(sc, reverse=True)
            if len(sc) > K:
                assert abs(gap[i, j] - (srt[K - 1] - srt[K])) < 1e-9
            else:
                assert gap[i, j] == np.inf


def test_equals_walk_when_only_leaves_are_scored():
    # N = 1000, K = 8: 16 leaves, 8 level-2 nodes: the walk keeps every level-2 node and
    # scores every eligible leaf by its exact LSE, i.e. the exact flat selection
    rng = np.random.default_rng(5)
    N, Hq, Hkv, K = 1000, 8, 2, 8
    q = rng.standard_normal((N, Hq, d)).astype(np.float32)
    k = rng.standard_normal((N, Hkv, d)).astype(np.float32)
    pyr = oracle.build_pyramid(k)
    ts = np.arange(N)
    w_idx, _, _ = oracle.walk(q, ts, k, pyr, K)
    f_idx, _ = oracle.flat_exact_select(q, ts, k, K)
    np.testing.assert_array_equal(w_idx, f_idx)


def test_repeated_key_blocks_closed_form():
    # block b: every key is c_b * e_0; one query head, q = e_0: per block log(m) + c_b / 8
    # with m = the block's keys up to t
    c = [0.0, 3.0, 1.0, 2.5, -1.0, 2.0]
    N = len(c) * C
    k = np.zeros((N, 1, d), np.float32)
    for b, v in enumerate(c):
        k[b * C:(b + 1) * C, 0, 0] = v
    q = np.zeros((N, 1, d), np.float32)
    q[:, 0, 0] = 1.0
    K = 2
    # t = 5 * C + 1: block 5 has 2 keys: log 2 + 0.25 = 0.943 against log 64 + c/8 for the rest:
    # 1 (3.0: 4.53), 3 (2.5: 4.47) -> {1, 3}
    # t = 3 * C: block 3 has 1 key: 0.3125 < blocks 1 (4.53), 2 (4.28) -> {1, 2}
    ts = np.array([3 * C, 5 * C + 1])
    idx, _ = oracle.flat_exact_select(q[ts], ts, k, K)
    assert idx[0, 0].tolist() == [1, 2]
    assert idx[1, 0].tolist() == [1, 3]


def test_structure_and_validate():
    rng = np.random.default_rng(6)
    N, Hq, Hkv, K = 900, 4, 1, 5
    q = rng.standard_normal((N, Hq, d)).astype(np.float32)
    k = rng.standard_normal((N, Hkv, d)).astype(np.float32)
    ts = np.array([10, 130, 300, 899])
    idx, gap = oracle.flat_exact_select(q[ts], ts, k, K)
    for i, t in enumerate(ts):
        row = idx[i, 0]
        n_el = min(int(t) // C + 1, -(-N // C))
        kept = row[row >= 0]
        assert len(kept) == min(K, n_el)
        assert np.all(np.diff(kept) > 0) and np.all(kept < n_el)
        assert np.all(row[len(kept):] == -1)
        assert oracle.flat_exact_validate(q[t], int(t), 0, k, K, row, 1e-3) == 1
    # t = 899 (15 eligible): the best block swapped for the 6th is rejected when the best is
    # more than eps above the K-th
    t = 899
    _, sc = _brute(q[t], t, k, K, 0)
    order = sorted(range(len(sc)), key=lambda b: (-sc[b], b))
    assert sc[order[0]] > sc[order[K - 1]] + 1e-3
    assert oracle.flat_exact_validate(q[t], t, 0, k, K, np.array(sorted(order[1:K + 1])), 1e-3) == 0
    # t = 130 (blocks 0..2 eligible, all kept): a set holding block 14 (not eligible) is rejected
    assert oracle.flat_exact_validate(q[130], 130, 0, k, K, np.array([0, 1, 2, 14, -1]), 1e-3) == 0
    assert oracle.flat_exact_validate(q[130], 130, 0, k, K, np.array([0, 1, 2, -1, -1]), 1e-3) == 1
    # a tied alternative: give two blocks identical keys, so their scores tie exactly
    k2 = k.copy()
    k2[4 * C:5 * C] = k2[3 * C:4 * C]
    t2 = 10 * C
    idx2, gap2 = oracle.flat_exact_select(q[[t2]], np.array([t2]), k2, K)
    sel = idx2[0, 0].tolist()
    if (3 in sel) != (4 in sel):
        alt = sorted([4 if b == 3 else 3 if b == 4 else b for b in sel])
        assert oracle.flat_exact_validate(q[t2], t2, 0, k2, K, alt, 1e-3) == 1
