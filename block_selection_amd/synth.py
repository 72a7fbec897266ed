"""Seeded synthetic inputs for the pyramid Top-K block-selection stage.

This module only draws random numbers and rounds them to bfloat16. It holds
none of the selection arithmetic, so both the CPU oracle and the HIP path can
take their inputs from here without sharing any method code.

Workloads follow the selection-latency benchmark described on the
"Block Sparse Attention with Log-Linear Complexity" reading note (section 7.3)
and the ai4snews summary page (fourth paragraph): random bf16 queries and keys
from a fixed seed, batch 1, 32 query heads, 2 KV heads, d=64, C=64, K=8, g=2.

Conventions (fixed here, stated once):
  * generator: numpy ``default_rng(seed)`` (PCG64), ``standard_normal`` in
    float32;
  * draw order: Q ``[B, N, Hq, d]``, then K ``[B, N, Hkv, d]``, then (planted
    workload only) the planted leaf-block indices, then the shift direction u;
    decode workloads draw K for the prebuilt context, then per step k_new
    ``[B, Hkv, d]`` followed by q_new ``[B, Hq, d]``;
  * bf16 rounding: round-to-nearest-even from float32.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest-even); return the raw uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # round-to-nearest-even on the 16 dropped bits
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 bits to float32 (exact)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 array whose values are exactly the bfloat16 nearest-even roundings of x."""
    return bf16_to_f32(bf16_bits(x))


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and recipe of one synthetic prefill or decode workload."""
    name: str
    N: int                 # prefill length, or prebuilt context length for decode
    Hq: int
    Hkv: int
    topk: int
    dtype: str             # "f32" or "bf16"
    B: int = 1
    d: int = 64
    C: int = 64
    g: int = 2
    seed: int = 0
    planted_blocks: int = 0     # leaf blocks whose keys get +shift*u
    planted_shift: float = 0.5
    decode_steps: int = 0       # >0 marks a decode workload

    @property
    def GQ(self) -> int:
        return self.Hq // self.Hkv


# The five workloads. Sizes follow the selection-latency benchmark; the tiny one
# is small enough for the oracle to finish in seconds.
WORKLOADS = {
    "tiny": Workload("tiny", N=1024, Hq=4, Hkv=1, topk=4, dtype="f32"),
    "short": Workload("short", N=4096, Hq=32, Hkv=2, topk=8, dtype="bf16"),
    "mid_planted": Workload("mid_planted", N=32768, Hq=32, Hkv=2, topk=8, dtype="bf16",
                            planted_blocks=64),
    "long64k": Workload("long64k", N=65536, Hq=32, Hkv=2, topk=8, dtype="bf16"),
    "long128k": Workload("long128k", N=131072, Hq=32, Hkv=2, topk=8, dtype="bf16"),
    "long256k": Workload("long256k", N=262144, Hq=32, Hkv=2, topk=8, dtype="bf16"),
    "decode128k": Workload("decode128k", N=131072, Hq=32, Hkv=2, topk=32, dtype="bf16",
                           decode_steps=256),
}


@dataclasses.dataclass
class PrefillInputs:
    wl: Workload
    q: np.ndarray                 # float32 [B, N, Hq, d] (bf16-exact values when dtype=bf16)
    k: np.ndarray                 # float32 [B, N, Hkv, d]
    planted: Optional[np.ndarray] = None   # int64 leaf-block indices
    u: Optional[np.ndarray] = None         # float32 [d] unit vector

    def q_bits(self) -> np.ndarray:
        return bf16_bits(self.q)

    def k_bits(self) -> np.ndarray:
        return bf16_bits(self.k)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def make_prefill(wl: Workload, N: Optional[int] = None, seed: Optional[int] = None) -> PrefillInputs:
    """Draw Q and K for a prefill workload (optionally at another length N)."""
    N = wl.N if N is None else N
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    q = _normal(rng, (wl.B, N, wl.Hq, wl.d))
    k = _normal(rng, (wl.B, N, wl.Hkv, wl.d))
    planted = u = None
    if wl.planted_blocks:
        n_leaf = -(-N // wl.C)
        planted = np.sort(rng.choice(n_leaf, size=wl.planted_blocks, replace=False)).astype(np.int64)
        u = _normal(rng, (wl.d,))
        u = (u / np.linalg.norm(u.astype(np.float64))).astype(np.float32)
        for b in planted:
            lo, hi = int(b) * wl.C, min((int(b) + 1) * wl.C, N)
            k[:, lo:hi, :, :] += np.float32(wl.planted_shift) * u
    if wl.dtype == "bf16":
        q = bf16_round(q)
        k = bf16_round(k)
    return PrefillInputs(wl, q, k, planted, u)


@dataclasses.dataclass
class DecodeInputs:
    wl: Workload
    k_ctx: np.ndarray      # float32 [B, N0, Hkv, d]
    k_new: np.ndarray      # float32 [steps, B, Hkv, d]
    q_new: np.ndarray      # float32 [steps, B, Hq, d]


def make_decode(wl: Workload, steps: Optional[int] = None, N0: Optional[int] = None) -> DecodeInputs:
    """Draw the prebuilt context keys, then per step one key and one query row."""
    steps = wl.decode_steps if steps is None else steps
    N0 = wl.N if N0 is None else N0
    rng = np.random.default_rng(wl.seed)
    k_ctx = _normal(rng, (wl.B, N0, wl.Hkv, wl.d))
    k_new = np.empty((steps, wl.B, wl.Hkv, wl.d), np.float32)
    q_new = np.empty((steps, wl.B, wl.Hq, wl.d), np.float32)
    for s in range(steps):
        k_new[s] = _normal(rng, (wl.B, wl.Hkv, wl.d))
        q_new[s] = _normal(rng, (wl.B, wl.Hq, wl.d))
    if wl.dtype == "bf16":
        k_ctx, k_new, q_new = bf16_round(k_ctx), bf16_round(k_new), bf16_round(q_new)
    return DecodeInputs(wl, k_ctx, k_new, q_new)


@dataclasses.dataclass
class VarlenInputs:
    """A pack of documents laid end to end: T tokens, document i at rows cu[i] .. cu[i+1]-1."""
    q: np.ndarray          # float32 [T, Hq, d]
    k: np.ndarray          # float32 [T, Hkv, d]
    cu: np.ndarray         # int32 [D + 1], cu[0] = 0, nondecreasing, cu[D] = T

    def q_bits(self) -> np.ndarray:
        return bf16_bits(self.q)

    def k_bits(self) -> np.ndarray:
        return bf16_bits(self.k)


def doc_lengths(rng: np.random.Generator, T: int, mean_len: float) -> np.ndarray:
    """Document lengths filling T tokens: exponential draws of the given mean, rounded up
    to at least one token, the last one cut to fit."""
    out, tot = [], 0
    while tot < T:
        n = max(1, int(np.ceil(rng.exponential(mean_len))))
        n = min(n, T - tot)
        out.append(n)
        tot += n
    return np.asarray(out, np.int64)


def make_varlen(T: int, Hq: int, Hkv: int, dtype: str = "bf16", mean_len: float = 2048.0,
                lengths=None, seed: int = 0, d: int = 64) -> VarlenInputs:
    """Draw Q [T, Hq, d], then K [T, Hkv, d], then (unless given) the document lengths."""
    rng = np.random.default_rng(seed)
    q = _normal(rng, (T, Hq, d))
    k = _normal(rng, (T, Hkv, d))
    if lengths is None:
        lengths = doc_lengths(rng, T, mean_len)
    lengths = np.asarray(lengths, np.int64)
    if lengths.min(initial=0) < 0 or int(lengths.sum()) != T:
        raise ValueError("document lengths must be >= 0 and sum to T")
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    if dtype == "bf16":
        q, k = bf16_round(q), bf16_round(k)
    return VarlenInputs(q, k, cu)


def make_values(B: int, N: int, Hkv: int, dtype: str = "bf16", seed: int = 0, d: int = 64) -> np.ndarray:
    """Value rows V [B, N, Hkv, d] for attention over the selected blocks: standard normal
    draws from their own generator, numpy default_rng(seed + 1000003), rounded like Q and K."""
    rng = np.random.default_rng(seed + 1000003)
    v = _normal(rng, (B, N, Hkv, d))
    return bf16_round(v) if dtype == "bf16" else v
