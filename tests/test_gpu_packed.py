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


def _run_packed_attention(v: synth.VarlenInputs, vals: np.ndarray, idx: np.ndarray, topk: int):
    from block_selection_amd import ops
    T, Hq, _ = v.q.shape
    Hkv = v.k.shape[1]
    D = len(v.cu) - 1
    print(f"packed attention T={T} D={D} Hq={Hq} Hkv={Hkv} K={topk}", flush=True)
    dims = ops.make_dims(1, Hq, Hkv, topk, "bf16")
    cu = torch.from_numpy(np.ascontiguousarray(v.cu, np.int32)).cuda()
    out = torch.full((T, Hq, 64), float("nan"), dtype=torch.float32, device="cuda")
    it = torch.from_numpy(np.ascontiguousarray(idx, np.int32)).cuda()
    ops.sparse_attention_packed(to_device(v.q, "bf16"), to_device(v.k, "bf16"), to_device(vals, "bf16"), it, cu, dims,
                                out, ops.alloc_pack_attention_workspace(dims, T, D))
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("K", [8, 32])
def test_packed_attention(K):
    """Attention of every row over its own document's selected blocks: the oracle per document
    (on the oracle's selection), and bitwise the single-sequence attention of each document."""
    from block_selection_amd import ops
    v = synth.make_varlen(sum(EDGE_LENGTHS), 32, 2, "bf16", lengths=EDGE_LENGTHS, seed=40 + K)
    vals = synth.make_values(1, int(v.cu[-1]), 2, seed=K)[0]
    o_idx, _, _ = oracle.varlen_walk(v.q, v.k, v.cu, K)
    got = _run_packed_attention(v, vals, o_idx, K)
    assert np.all(np.isfinite(got))
    scale = float(np.abs(vals).max())
    worst = 0.0
    for j in range(len(EDGE_LENGTHS)):
        lo, hi = int(v.cu[j]), int(v.cu[j + 1])
        if hi == lo:
            continue
        n = hi - lo
        ref = oracle.attention(v.q[lo:hi], np.arange(n), v.k[lo:hi], vals[lo:hi], o_idx[lo:hi])
        worst = max(worst, float(np.abs(got[lo:hi] - ref).max()) / scale)
        # the same document alone through pisa_sparse_attention
        dims = ops.make_dims(1, 32, 2, K, "bf16")
        alone = torch.empty((1, n, 32, 64), dtype=torch.float32, device="cuda")
        ops.sparse_attention(to_device(v.q[None, lo:hi], "bf16"), to_device(v.k[None, lo:hi], "bf16"),
                             to_device(vals[None, lo:hi], "bf16"),
                             torch.from_numpy(np.ascontiguousarray(o_idx[None, lo:hi])).cuda(), n, n, dims, alone,
                             ops.alloc_attention_workspace(dims, n))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got[lo:hi], alone.cpu().numpy()[0])
    print(f"packed attention max |err| / max|v| = {worst:.3e}", flush=True)
    assert worst <= 1e-4


def test_packed_selection_then_attention_long():
    """A 65536-token pack: GPU selection, then GPU attention on it, sampled rows of every
    document against the oracle's selection and attention."""
    from block_selection_amd import ops
    v = synth.make_varlen(65536, 32, 2, "bf16", mean_len=4096.0, seed=9)
    vals = synth.make_values(1, 65536, 2, seed=9)[0]
    dims, pyr, idx = _run_packed(v, 8)
    got = _run_packed_attention(v, vals, idx, 8)
    rng = np.random.default_rng(2)
    scale = float(np.abs(vals).max())
    compared = 0
    for j in range(len(v.cu) - 1):
        lo, hi = int(v.cu[j]), int(v.cu[j + 1])
        if hi == lo:
            continue
        n = hi - lo
        ts = np.unique(np.concatenate([[0, n - 1], rng.choice(n, min(n, 16), replace=False)])).astype(np.int64)
        kd = v.k[lo:hi]
        o_idx, _, _ = oracle.walk(v.q[lo:hi][ts], ts, kd, oracle.build_pyramid(kd), 8)
        same = np.all(o_idx == idx[lo + ts], axis=(1, 2))
        ref = oracle.attention(v.q[lo:hi][ts], ts, kd, vals[lo:hi], o_idx)
        err = np.abs(got[lo + ts][same] - ref[same]).max() / scale if same.any() else 0.0
        assert err <= 1e-4, (j, err)
        compared += int(same.sum())
    print(f"packed selection + attention: {compared} rows compared", flush=True)
    assert compared > 200
