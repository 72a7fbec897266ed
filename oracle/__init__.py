"""Plain fp64 CPU oracle for the pyramid Top-K block selection (ctypes wrapper).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. It shares no code
with the HIP library under ``block_selection_amd/`` and never calls it.

The arithmetic lives in ``pisa_oracle.c`` (fp64, plain loops, OpenMP over
independent walks); this module only marshals numpy arrays. Each function
names the passage of the pages it follows in the C source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pisa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libpisa_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE double arithmetic, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wno-unknown-pragmas", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i64, i32, dbl, lng = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_long
    lib.pisa_oracle_num_levels.argtypes = [i64, i32, i32]
    lib.pisa_oracle_num_levels.restype = i32
    lib.pisa_oracle_level_sizes.argtypes = [i64, i32, i32, P, i32]
    lib.pisa_oracle_level_sizes.restype = i32
    lib.pisa_oracle_build_pyramid.argtypes = [P, i64, i32, i32, i32, i32, P, i32]
    lib.pisa_oracle_build_pyramid.restype = i32
    lib.pisa_oracle_walk.argtypes = [P, P, i64, P, P, i64, i32, i32, i32, i32, i32, i32, i32,
                                     P, P, P, i32]
    lib.pisa_oracle_walk.restype = i32
    lib.pisa_oracle_walk_trace.argtypes = [P, i64, i32, P, P, i64, i32, i32, i32, i32, i32, i32, i32,
                                           P, P, P, P, P, i32]
    lib.pisa_oracle_walk_trace.restype = i32
    lib.pisa_oracle_node_score.argtypes = [P, i64, i32, P, P, i64, i32, i32, i32, i32, i32,
                                           i32, i64, i32]
    lib.pisa_oracle_node_score.restype = dbl
    lib.pisa_oracle_validate.argtypes = [P, i64, i32, P, P, i64, i32, i32, i32, i32, i32, i32, i32,
                                         P, dbl, lng]
    lib.pisa_oracle_validate.restype = i32
    lib.pisa_oracle_attention.argtypes = [P, P, i64, P, P, P, i64, i32, i32, i32, i32, i32, P, i32]
    lib.pisa_oracle_attention.restype = i32
    lib.pisa_oracle_flat_select.argtypes = [P, P, i64, P, i64, i32, i32, i32, i32, i32, P, P, i32]
    lib.pisa_oracle_flat_select.restype = i32
    lib.pisa_oracle_flat_validate.argtypes = [P, i64, i32, P, i64, i32, i32, i32, i32, i32, P, dbl]
    lib.pisa_oracle_flat_validate.restype = i32
    lib.pisa_oracle_flat_exact_select.argtypes = [P, P, i64, P, i64, i32, i32, i32, i32, i32, P, P, i32]
    lib.pisa_oracle_flat_exact_select.restype = i32
    lib.pisa_oracle_flat_exact_validate.argtypes = [P, i64, i32, P, i64, i32, i32, i32, i32, i32, P, dbl]
    lib.pisa_oracle_flat_exact_validate.restype = i32
    _lib = lib
    return lib


# Candidate scores (per head, over the eligible children's logits; summed over the group):
# "lse" the LogSumExp, "mean" their mean, "mean_half_var" their mean plus half their
# (population) variance -- the first- and second-order truncations of the LSE expansion.
SCORES = {"lse": 0, "mean": 1, "mean_half_var": 2}


def _score(score: str) -> int:
    if score not in SCORES:
        raise ValueError(f"score must be one of {sorted(SCORES)}")
    return SCORES[score]


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def level_sizes(N: int, C: int = 64, g: int = 2) -> list:
    """[M_1, ..., M_L]: leaf blocks, then ceil-halving up to the single root."""
    buf = np.zeros(64, np.int64)
    L = _load().pisa_oracle_level_sizes(N, C, g, _p(buf), 64)
    if L < 0:
        raise ValueError("bad geometry")
    return [int(x) for x in buf[:L]]


def level_offsets(N: int, C: int = 64, g: int = 2) -> list:
    """Row offset of each level (1..L) inside one KV head's pyramid."""
    out, acc = [], 0
    for m in level_sizes(N, C, g):
        out.append(acc)
        acc += m
    return out


def build_pyramid(k: np.ndarray, C: int = 64, g: int = 2, nthreads: int = 0) -> np.ndarray:
    """k: float [N, Hkv, d] -> double [Hkv, sum(M_l), d] of raw-key means."""
    k = _f32(k)
    N, Hkv, d = k.shape
    total = sum(level_sizes(N, C, g))
    pyr = np.zeros((Hkv, total, d), np.float64)
    rc = _load().pisa_oracle_build_pyramid(_p(k), N, Hkv, d, C, g, _p(pyr), nthreads)
    if rc != 0:
        raise RuntimeError(f"oracle build_pyramid failed ({rc})")
    return pyr


def walk(q_rows: np.ndarray, t_rows, k: np.ndarray, pyr: np.ndarray, topk: int,
         C: int = 64, g: int = 2, nthreads: int = 0, score: str = "lse"):
    """Walks for the query rows of positions t_rows (one batch element).

    q_rows: float [n, Hq, d]; k: float [N, Hkv, d]; pyr from build_pyramid.
    Returns (idx int32 [n, Hkv, topk] ascending, -1 padded;
             min_gap double [n, Hkv] (inf if nothing was scored);
             gap_level int32 [n, Hkv]).
    """
    q_rows, k = _f32(q_rows), _f32(k)
    t_rows = np.ascontiguousarray(t_rows, dtype=np.int64)
    n, Hq, d = q_rows.shape
    N, Hkv, _ = k.shape
    assert t_rows.shape == (n,)
    pyr = np.ascontiguousarray(pyr, dtype=np.float64)
    idx = np.zeros((n, Hkv, topk), np.int32)
    gap = np.zeros((n, Hkv), np.float64)
    lvl = np.zeros((n, Hkv), np.int32)
    rc = _load().pisa_oracle_walk(_p(q_rows), _p(t_rows), n, _p(k), _p(pyr), N, Hq, Hkv, d, C, g,
                                  topk, _score(score), _p(idx), _p(gap), _p(lvl), nthreads)
    if rc != 0:
        raise RuntimeError(f"oracle walk failed ({rc})")
    return idx, gap, lvl


def walk_trace(q_row: np.ndarray, t: int, j: int, k: np.ndarray, pyr: np.ndarray, topk: int,
               C: int = 64, g: int = 2, score: str = "lse"):
    """One walk with every candidate recorded.

    Returns (idx [topk], records) where records is a list of
    (level, node, score or nan, kept) in the order the walk considered them.
    """
    q_row, k = _f32(q_row), _f32(k)
    Hq, d = q_row.shape
    N, Hkv, _ = k.shape
    cap = 4096
    lv = np.zeros(cap, np.int32)
    nd = np.zeros(cap, np.int64)
    sc = np.zeros(cap, np.float64)
    kp = np.zeros(cap, np.int32)
    idx = np.zeros(topk, np.int32)
    pyr = np.ascontiguousarray(pyr, dtype=np.float64)
    n = _load().pisa_oracle_walk_trace(_p(q_row), t, j, _p(k), _p(pyr), N, Hq, Hkv, d, C, g, topk,
                                       _score(score), _p(idx), _p(lv), _p(nd), _p(sc), _p(kp), cap)
    if n < 0:
        raise RuntimeError(f"oracle walk_trace failed ({n})")
    n = min(n, cap)
    recs = [(int(lv[i]), int(nd[i]), float(sc[i]), bool(kp[i])) for i in range(n)]
    return idx, recs


def node_score(q_row: np.ndarray, t: int, j: int, k: np.ndarray, pyr: np.ndarray, level: int,
               node: int, C: int = 64, g: int = 2, score: str = "lse") -> float:
    """Score of one node (sum over the group's heads of the score over its eligible children)."""
    q_row, k = _f32(q_row), _f32(k)
    Hq, d = q_row.shape
    N, Hkv, _ = k.shape
    pyr = np.ascontiguousarray(pyr, dtype=np.float64)
    return float(_load().pisa_oracle_node_score(_p(q_row), t, j, _p(k), _p(pyr), N, Hq, Hkv, d,
                                                C, g, level, node, _score(score)))


def validate(q_row: np.ndarray, t: int, j: int, k: np.ndarray, pyr: np.ndarray, topk: int,
             target, eps: float, budget: int = 200000, C: int = 64, g: int = 2,
             score: str = "lse") -> int:
    """1 if target is reachable by resolving near-ties within eps, 0 if not, -1 if undecided."""
    q_row, k = _f32(q_row), _f32(k)
    Hq, d = q_row.shape
    N, Hkv, _ = k.shape
    tg = np.ascontiguousarray(target, dtype=np.int32)
    assert tg.shape == (topk,)
    pyr = np.ascontiguousarray(pyr, dtype=np.float64)
    r = _load().pisa_oracle_validate(_p(q_row), t, j, _p(k), _p(pyr), N, Hq, Hkv, d, C, g, topk,
                                     _score(score), _p(tg), eps, budget)
    if r == -2:
        raise RuntimeError("oracle validate: bad arguments")
    return int(r)


def decode_step(k_all: np.ndarray, n: int, q_new: np.ndarray, topk: int, C: int = 64, g: int = 2,
                nthreads: int = 0, score: str = "lse", with_level: bool = False):
    """Selection after appending key n: rebuild over keys 0..n and walk at t = n.

    k_all: float [>= n+1, Hkv, d]; q_new: float [Hq, d].
    Returns (pyr, idx [Hkv, topk], min_gap [Hkv]), plus gap_level [Hkv] if with_level.
    """
    k = _f32(k_all[: n + 1])
    pyr = build_pyramid(k, C, g, nthreads)
    idx, gap, lvl = walk(q_new[None], np.array([n]), k, pyr, topk, C, g, nthreads, score)
    if with_level:
        return pyr, idx[0], gap[0], lvl[0]
    return pyr, idx[0], gap[0]


def attention(q_rows: np.ndarray, t_rows, k: np.ndarray, v: np.ndarray, idx: np.ndarray,
              C: int = 64, nthreads: int = 0) -> np.ndarray:
    """Stage two: per query row and head, softmax attention over the keys <= t of the
    blocks its KV head selected (idx [n, Hkv, K], -1 entries ignored). Returns double
    [n, Hq, d]."""
    q_rows, k, v = _f32(q_rows), _f32(k), _f32(v)
    t_rows = np.ascontiguousarray(t_rows, dtype=np.int64)
    n, Hq, d = q_rows.shape
    N, Hkv, _ = k.shape
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    assert idx.shape[:2] == (n, Hkv) and v.shape == k.shape and t_rows.shape == (n,)
    out = np.zeros((n, Hq, d), np.float64)
    rc = _load().pisa_oracle_attention(_p(q_rows), _p(t_rows), n, _p(k), _p(v), _p(idx), N, Hq, Hkv, d,
                                       C, idx.shape[2], _p(out), nthreads)
    if rc != 0:
        raise RuntimeError(f"oracle attention failed ({rc})")
    return out


def flat_select(q_rows: np.ndarray, t_rows, pyr: np.ndarray, N: int, topk: int, C: int = 64,
                nthreads: int = 0):
    """Flat stage-one selection: each query scores every eligible leaf summary (the sum over
    its group's heads of q.kbar/sqrt(d)) and keeps the K best.

    q_rows: float [n, Hq, d]; pyr from build_pyramid over N keys ([Hkv, rows, d]).
    Returns (idx int32 [n, Hkv, topk] ascending, -1 padded; min_gap double [n, Hkv]).
    """
    q_rows = _f32(q_rows)
    t_rows = np.ascontiguousarray(t_rows, dtype=np.int64)
    n, Hq, d = q_rows.shape
    Hkv = pyr.shape[0]
    assert t_rows.shape == (n,)
    pyr = np.ascontiguousarray(pyr, dtype=np.float64)
    idx = np.zeros((n, Hkv, topk), np.int32)
    gap = np.zeros((n, Hkv), np.float64)
    rc = _load().pisa_oracle_flat_select(_p(q_rows), _p(t_rows), n, _p(pyr), N, Hq, Hkv, d, C, topk, _p(idx),
                                         _p(gap), nthreads)
    if rc != 0:
        raise RuntimeError(f"oracle flat_select failed ({rc})")
    return idx, gap


def flat_validate(q_row: np.ndarray, t: int, j: int, pyr: np.ndarray, N: int, topk: int, target, eps: float,
                  C: int = 64) -> int:
    """1 if target is the flat selection under some resolution of the near-ties within eps, else 0."""
    q_row = _f32(q_row)
    Hq, d = q_row.shape
    tg = np.ascontiguousarray(target, dtype=np.int32)
    assert tg.shape == (topk,)
    pyr = np.ascontiguousarray(pyr, dtype=np.float64)
    r = _load().pisa_oracle_flat_validate(_p(q_row), t, j, _p(pyr), N, Hq, pyr.shape[0], d, C, topk, _p(tg), eps)
    if r == -2:
        raise RuntimeError("oracle flat_validate: bad arguments")
    return int(r)


# ------------------------------------------------------------------ packed documents --
# Packed inputs keep document boundaries and allow no attention across documents (reading
# note "Block Sparse Attention with Log-Linear Complexity", "Experiments: language
# modelling and downstream", the continued-pretraining settings). Reading:
# every document is selected exactly as if it were a sequence of its own -- its own pyramid
# over its own keys, its queries at positions counted from the document's first token, its
# leaf indices counted from the document's first leaf. Nothing of one document (keys,
# summaries, blocks straddling a boundary) reaches another's selection.

def doc_of(cu: np.ndarray, rows) -> np.ndarray:
    """Document of each packed row: the last i with cu[i] <= row (empty documents skipped)."""
    cu = np.asarray(cu, np.int64)
    return np.searchsorted(cu, np.asarray(rows, np.int64), side="right") - 1


def varlen_pyramids(k: np.ndarray, cu: np.ndarray, C: int = 64, g: int = 2, nthreads: int = 0) -> list:
    """One pyramid per document (None for an empty one): k float [T, Hkv, d], cu int [D+1]."""
    cu = np.asarray(cu, np.int64)
    out = []
    for i in range(len(cu) - 1):
        lo, hi = int(cu[i]), int(cu[i + 1])
        out.append(build_pyramid(k[lo:hi], C, g, nthreads) if hi > lo else None)
    return out


def varlen_walk(q: np.ndarray, k: np.ndarray, cu: np.ndarray, topk: int, rows=None, pyrs=None,
                C: int = 64, g: int = 2, nthreads: int = 0, score: str = "lse"):
    """Walks of the packed rows `rows` (default: all), each inside its own document.

    q float [T, Hq, d], k float [T, Hkv, d]. Returns (idx int32 [n, Hkv, topk] of
    document-local leaf indices, ascending, -1 padded; min_gap [n, Hkv]; gap_level [n, Hkv]).
    """
    cu = np.asarray(cu, np.int64)
    T = int(cu[-1])
    rows = np.arange(T, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    if pyrs is None:
        pyrs = varlen_pyramids(k, cu, C, g, nthreads)
    docs = doc_of(cu, rows)
    n, Hkv = len(rows), k.shape[1]
    idx = np.zeros((n, Hkv, topk), np.int32)
    gap = np.zeros((n, Hkv), np.float64)
    lvl = np.zeros((n, Hkv), np.int32)
    for dd in np.unique(docs):
        sel = np.nonzero(docs == dd)[0]
        lo, hi = int(cu[dd]), int(cu[dd + 1])
        i_, g_, l_ = walk(q[rows[sel]], rows[sel] - lo, k[lo:hi], pyrs[dd], topk, C, g, nthreads, score)
        idx[sel], gap[sel], lvl[sel] = i_, g_, l_
    return idx, gap, lvl


def flat_exact_select(q_rows: np.ndarray, t_rows, k: np.ndarray, topk: int, C: int = 64, nthreads: int = 0):
    """Exact flat selection: each query scores every eligible leaf block as the walk scores a
    leaf candidate (the sum over its group's heads of the LSE of q.k/sqrt(d) over the block's
    raw keys up to t) and keeps the K best.

    q_rows: float [n, Hq, d]; k: float [N, Hkv, d] raw keys.
    Returns (idx int32 [n, Hkv, topk] ascending, -1 padded; min_gap double [n, Hkv]).
    """
    q_rows = _f32(q_rows)
    k = _f32(k)
    t_rows = np.ascontiguousarray(t_rows, dtype=np.int64)
    n, Hq, d = q_rows.shape
    N, Hkv, _ = k.shape
    assert t_rows.shape == (n,)
    idx = np.zeros((n, Hkv, topk), np.int32)
    gap = np.zeros((n, Hkv), np.float64)
    rc = _load().pisa_oracle_flat_exact_select(_p(q_rows), _p(t_rows), n, _p(k), N, Hq, Hkv, d, C, topk, _p(idx),
                                               _p(gap), nthreads)
    if rc != 0:
        raise RuntimeError(f"oracle flat_exact_select failed ({rc})")
    return idx, gap


def flat_exact_validate(q_row: np.ndarray, t: int, j: int, k: np.ndarray, topk: int, target, eps: float,
                        C: int = 64) -> int:
    """1 if target is the exact flat selection under some resolution of the near-ties within
    eps, else 0."""
    q_row = _f32(q_row)
    k = _f32(k)
    Hq, d = q_row.shape
    N, Hkv, _ = k.shape
    tg = np.ascontiguousarray(target, dtype=np.int32)
    assert tg.shape == (topk,)
    r = _load().pisa_oracle_flat_exact_validate(_p(q_row), t, j, _p(k), N, Hq, Hkv, d, C, topk, _p(tg), eps)
    if r == -2:
        raise RuntimeError("oracle flat_exact_validate: bad arguments")
    return int(r)
