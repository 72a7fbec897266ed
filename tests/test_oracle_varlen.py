"""Pins of the oracle's packed-document (varlen) selection.

The reading note's continued-pretraining runs pack documents into one input while
keeping their boundaries, with no attention from one document into another. The
oracle reads this as: each document is selected as a sequence of its own (own
pyramid, positions and leaf indices counted from the document's start). The pins
check that reading against what it fixes, not against the oracle's own code:
  * brute force: where no level above the leaves is scored, every query's
    selection is flat exact top-K by raw-key LogSumExp over the leaves of its own
    document up to its own position (numpy, fp64);
  * independence: redrawing the other documents' queries and keys changes nothing
    (a pyramid over the whole pack, or blocks straddling a boundary, would);
  * document order: a reversed pack gives each document the same selection;
  * a one-document pack is the plain sequence; empty documents change nothing;
  * indices stay inside the query's own document and causal prefix.
"""
import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
from block_selection_amd import synth


def _flat_local(q_row, k_doc, t, j, K, GQ):
    """Flat exact top-K over the document's leaves 0 .. t//64 (keys <= t of the document)."""
    nl = t // 64 + 1
    sc = []
    for b in range(nl):
        hi = min((b + 1) * 64, t + 1)
        s = 0.0
        for h in range(j * GQ, (j + 1) * GQ):
            z = k_doc[b * 64:hi, j].astype(np.float64) @ q_row[h].astype(np.float64) / 8.0
            s += logsumexp(z)
        sc.append((-s, b))
    sc.sort()
    sel = sorted(b for _, b in sc[:K])
    return sel + [-1] * (K - len(sel))


@pytest.mark.parametrize("lengths,K", [([1, 63, 64, 65, 200, 511, 512, 129], 4),
                                       ([300, 7, 1000, 2, 700], 8)])
def test_flat_bruteforce_per_document(lengths, K):
    """No scored upper level in any document: flat top-K inside the query's document."""
    Hq, Hkv = 4, 2
    v = synth.make_varlen(int(sum(lengths)), Hq, Hkv, "bf16", lengths=lengths, seed=len(lengths))
    for n in lengths:
        assert oracle.level_sizes(n)[1:2] == [] or oracle.level_sizes(n)[1] <= K
    idx, _, lvl = oracle.varlen_walk(v.q, v.k, v.cu, K)
    assert np.all((lvl == 1) | (lvl == -1))
    rng = np.random.default_rng(3)
    for d in range(len(lengths)):
        lo, hi = int(v.cu[d]), int(v.cu[d + 1])
        ts = sorted({0, hi - lo - 1} | set(rng.integers(0, hi - lo, 6).tolist()))
        for t in ts:
            for j in range(Hkv):
                assert idx[lo + t, j].tolist() == _flat_local(v.q[lo + t], v.k[lo:hi], t, j, K, Hq // Hkv), (d, t, j)


def _pack(lengths, seed, Hq=4, Hkv=2):
    return synth.make_varlen(int(sum(lengths)), Hq, Hkv, "bf16", lengths=lengths, seed=seed)


def test_documents_are_independent():
    """Redrawing every other document leaves a document's selections bitwise unchanged."""
    lengths, K = [1500, 2600, 900], 4                   # upper levels are scored (M_2 > K)
    a = _pack(lengths, 5)
    b = _pack(lengths, 6)
    keep = 1
    lo, hi = int(a.cu[keep]), int(a.cu[keep + 1])
    q, k = b.q.copy(), b.k.copy()
    q[lo:hi], k[lo:hi] = a.q[lo:hi], a.k[lo:hi]
    ia, ga, la = oracle.varlen_walk(a.q, a.k, a.cu, K)
    ib, gb, lb = oracle.varlen_walk(q, k, a.cu, K)
    assert np.any(la[lo:hi] >= 2)
    np.testing.assert_array_equal(ia[lo:hi], ib[lo:hi])
    np.testing.assert_array_equal(ga[lo:hi], gb[lo:hi])
    assert not np.array_equal(ia[:lo], ib[:lo])


def test_document_order_does_not_matter():
    lengths, K = [700, 1800, 333, 1025], 4
    v = _pack(lengths, 8)
    idx, gap, _ = oracle.varlen_walk(v.q, v.k, v.cu, K)
    order = list(reversed(range(len(lengths))))
    segs = [(int(v.cu[d]), int(v.cu[d + 1])) for d in order]
    q = np.concatenate([v.q[lo:hi] for lo, hi in segs])
    k = np.concatenate([v.k[lo:hi] for lo, hi in segs])
    cu = np.concatenate([[0], np.cumsum([hi - lo for lo, hi in segs])]).astype(np.int32)
    idx2, gap2, _ = oracle.varlen_walk(q, k, cu, K)
    for pos, (lo, hi) in enumerate(segs):
        np.testing.assert_array_equal(idx2[cu[pos]:cu[pos + 1]], idx[lo:hi])
        np.testing.assert_array_equal(gap2[cu[pos]:cu[pos + 1]], gap[lo:hi])


def test_single_document_pack_is_the_sequence():
    N, K = 3000, 4
    v = _pack([N], 9)
    idx, gap, _ = oracle.varlen_walk(v.q, v.k, v.cu, K)
    pyr = oracle.build_pyramid(v.k)
    ref, rgap, _ = oracle.walk(v.q, np.arange(N), v.k, pyr, K)
    np.testing.assert_array_equal(idx, ref)
    np.testing.assert_array_equal(gap, rgap)


def test_empty_documents_change_nothing():
    K = 4
    v = _pack([400, 0, 900, 0, 0, 650], 10)
    w = synth.VarlenInputs(v.q, v.k, np.unique(v.cu).astype(np.int32))
    a = oracle.varlen_walk(v.q, v.k, v.cu, K)[0]
    b = oracle.varlen_walk(w.q, w.k, w.cu, K)[0]
    np.testing.assert_array_equal(a, b)


def test_indices_stay_in_the_document_prefix():
    lengths, K = [64, 1, 2000, 129, 5000], 8
    v = _pack(lengths, 11)
    idx, _, _ = oracle.varlen_walk(v.q, v.k, v.cu, K)
    docs = oracle.doc_of(v.cu, np.arange(int(v.cu[-1])))
    tl = np.arange(int(v.cu[-1])) - v.cu[docs]
    for row in range(len(tl)):
        n_el = tl[row] // 64 + 1
        for j in range(2):
            sel = idx[row, j]
            got = sel[sel >= 0]
            assert len(got) == min(K, n_el)
            assert np.all(sel[len(got):] == -1)
            assert np.all(np.diff(got) > 0) and got.min() >= 0 and got.max() <= tl[row] // 64
