"""GPU parity of the packed-document (varlen) path against the oracle.

Every document of a pack must be selected as a sequence of its own: the packed
pyramid's rows of a document are compared with the oracle's pyramid of that
document (and bitwise with the single-sequence build on the GPU), and its
selections with the oracle's walks inside the document (near-ties validated), and
bitwise with the single-sequence prefill of that document on the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
from block_selection_amd import synth
from pisa_testlib import check_pyramid, compare_selection, run_prefill, to_device

pytestmark = pytest.mark.gpu


def _run_packed(v: synth.VarlenInputs, topk: int, dtype: str = "bf16", score: str = "lse"):
    from block_selection_amd import ops
    T, Hq, _ = v.q.shape
    Hkv = v.k.shape[1]
    D = len(v.cu) - 1
    print(f"packed T={T} D={D} Hq={Hq} Hkv={Hkv} K={topk} score={score}", flush=True)
    dims = ops.make_dims(1, Hq, Hkv, topk, dtype, score=score)
    qt, kt = to_device(v.q, dtype), to_device(v.k, dtype)
    cu = torch.from_numpy(np.ascontiguousarray(v.cu, np.int32)).cuda()
    pyr = ops.alloc_pack_pyramid(dims, T, D)
    pyr.fill_(float("nan"))
    out = torch.full((T, Hkv, topk), -7, dtype=torch.int32, device="cuda")
    ws = ops.alloc_pack_workspace(dims, T, D)
    ops.build_pyramid_packed(kt, cu, dims, pyr)
    ops.select_prefill_packed(qt, kt, pyr, cu, dims, out, ws)
    torch.cuda.synchronize()
    return dims, pyr.cpu().numpy(), out.cpu().numpy()


def _doc_pyramid(pyr: np.ndarray, dims, cu: np.ndarray, j: int) -> np.ndarray:
    """Document j's rows of the packed layout, as one sequence's pyramid [Hkv, sum M_l, d]."""
    from block_selection_amd import ops
    T, D = int(cu[-1]), len(cu) - 1
    n = int(cu[j + 1] - cu[j])
    parts = []
    for l, m in enumerate(oracle.level_sizes(n), start=1):
        start = ops.pack_level_offset(dims, T, D, l) + (int(cu[j]) >> (5 + l)) + j
        parts.append(pyr[:, start:start + m])
    return np.concatenate(parts, axis=1)


def _check_docs(v, dims, pyr, idx, topk, docs=None, rows_per_doc=None, score="lse", seed=0):
    rng = np.random.default_rng(seed)
    D = len(v.cu) - 1
    total = None
    for j in (range(D) if docs is None else docs):
        lo, hi = int(v.cu[j]), int(v.cu[j + 1])
        if hi == lo:
            continue
        n = hi - lo
        ref = oracle.build_pyramid(v.k[lo:hi])
        got = _doc_pyramid(pyr, dims, v.cu, j)
        check_pyramid(got[None], ref, n, n)
        if rows_per_doc is None or n <= rows_per_doc:
            ts = np.arange(n, dtype=np.int64)
        else:
            ts = np.unique(np.concatenate([[0, n - 1, min(n - 1, topk * 64)],
                                           rng.choice(n, rows_per_doc, replace=False)])).astype(np.int64)
        rep = compare_selection(idx[lo + ts], ts, v.q[lo:hi], v.k[lo:hi], ref, topk, score=score)
        assert rep.ok(), f"document {j} (rows {lo}..{hi}): {rep}"
        total = rep if total is None else _add(total, rep)
    print(f"packed parity: {total}", flush=True)
    return total


def _add(a, b):
    for f in ("walks", "exact", "near_tie_walks", "mismatch_near_tie", "mismatch_valid", "mismatch_invalid",
              "mismatch_unverified", "hard_fail"):
        setattr(a, f, getattr(a, f) + getattr(b, f))
    return a


EDGE_LENGTHS = [1, 63, 64, 65, 0, 200, 1000, 1024, 1025, 0, 3000, 5000, 2047, 129, 511, 513]


@pytest.mark.parametrize("K", [8, 4, 32])
def test_packed_edge_lengths(K):
    """Documents of 1, 63, 64, 65 ... tokens, empty ones between: every row against the oracle."""
    v = synth.make_varlen(sum(EDGE_LENGTHS), 32, 2, "bf16", lengths=EDGE_LENGTHS, seed=K)
    dims, pyr, idx = _run_packed(v, K)
    _check_docs(v, dims, pyr, idx, K)


def test_packed_equals_single_sequences_bitwise():
    """Each document's packed pyramid and selections are bitwise those of the document alone."""
    lengths = [700, 4097, 1, 2500, 0, 9000, 64]
    v = synth.make_varlen(sum(lengths), 32, 2, "bf16", lengths=lengths, seed=3)
    dims, pyr, idx = _run_packed(v, 8)
    for j in range(len(lengths)):
        lo, hi = int(v.cu[j]), int(v.cu[j + 1])
        if hi == lo:
            continue
        alone = run_prefill(v.q[None, lo:hi], v.k[None, lo:hi], 8, "bf16")
        got = _doc_pyramid(pyr, dims, v.cu, j)
        np.testing.assert_array_equal(got, alone.pyramid[0])
        np.testing.assert_array_equal(idx[lo:hi], alone.idx[0])


def test_packed_many_short_documents():
    """Hundreds of documents of 1 .. 300 tokens: several per walk piece and per range."""
    rng = np.random.default_rng(11)
    lengths = rng.integers(1, 300, 120).tolist()
    lengths[5] = 0
    v = synth.make_varlen(sum(lengths), 32, 2, "bf16", lengths=lengths, seed=12)
    dims, pyr, idx = _run_packed(v, 8)
    _check_docs(v, dims, pyr, idx, 8)


@pytest.mark.parametrize("Hq,Hkv", [(12, 3), (8, 8), (16, 1)])
def test_packed_group_shapes(Hq, Hkv):
    lengths = [3000, 129, 6000, 900]
    v = synth.make_varlen(sum(lengths), Hq, Hkv, "bf16", lengths=lengths, seed=Hq + Hkv)
    dims, pyr, idx = _run_packed(v, 8)
    _check_docs(v, dims, pyr, idx, 8, rows_per_doc=600)


@pytest.mark.parametrize("score", ["mean", "mean_half_var"])
def test_packed_truncated_scores(score):
    v = synth.make_varlen(sum(EDGE_LENGTHS), 32, 2, "bf16", lengths=EDGE_LENGTHS, seed=21)
    dims, pyr, idx = _run_packed(v, 8, score=score)
    _check_docs(v, dims, pyr, idx, 8, score=score)


def test_packed_continued_pretraining_shape():
    """16K-token packs with K = 32 (the continued-pretraining setting): random document lengths."""
    v = synth.make_varlen(16384, 32, 2, "bf16", mean_len=2048.0, seed=5)
    dims, pyr, idx = _run_packed(v, 32)
    _check_docs(v, dims, pyr, idx, 32, rows_per_doc=400)


def test_packed_long_pack_sampled():
    """262144 tokens in random documents (mean 8192): sampled rows of every document."""
    v = synth.make_varlen(262144, 32, 2, "bf16", mean_len=8192.0, seed=7)
    dims, pyr, idx = _run_packed(v, 8)
    rep = _check_docs(v, dims, pyr, idx, 8, rows_per_doc=24)
    assert rep.walks > 1000
    # rows of every document are written (no -7 left) and stay in their document
    T = int(v.cu[-1])
    docs = oracle.doc_of(v.cu, np.arange(T))
    tl = np.arange(T) - v.cu[docs]
    assert idx.min() >= -1
    assert np.all(idx.max(axis=2) <= (tl // 64)[:, None])
