"""Shared helpers for the GPU parity tests: seeded inputs on the device, the
HIP path through the C ABI, and the parity rule against the fp64 oracle.

Parity rule (selection): for every (position t, KV head) the GPU's index set
must equal the oracle's, except when the oracle's walk had a near-tie, i.e.
its K-th and (K+1)-th scores differed by less than NEAR_TIE at some scored
level. Such walks are counted; a mismatching one must also be reachable by
resolving the near-ties within NEAR_TIE (oracle.validate) and must never be
unreachable or undecided. Pyramid rule: per node, ||gpu - ref||_2 <= 1e-5 ||ref||_2 and
max|gpu - ref| <= 1e-5 max|ref|.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import oracle
from block_selection_amd import synth

NEAR_TIE = 1e-3
PYR_RTOL = 1e-5


def to_device(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """float32 array (bf16-exact values for bf16) -> contiguous device tensor."""
    if dtype == "bf16":
        bits = synth.bf16_bits(x)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


@dataclasses.dataclass
class GpuPrefill:
    pyramid: np.ndarray    # [B, Hkv, P, d] fp32 (capacity layout)
    idx: np.ndarray        # [B, N, Hkv, K] int32
    dims: object
    cap: int


def run_prefill(q: np.ndarray, k: np.ndarray, topk: int, dtype: str, cap: int | None = None,
                device="cuda", score: str = "lse") -> GpuPrefill:
    from block_selection_amd import ops
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    cap = N if cap is None else cap
    dims = ops.make_dims(B, Hq, Hkv, topk, dtype, score=score)
    kk = np.zeros((B, cap, Hkv, d), np.float32)
    kk[:, :N] = k
    qt, kt = to_device(q, dtype, device), to_device(kk, dtype, device)
    pyr = ops.alloc_pyramid(dims, cap, device)
    pyr.fill_(float("nan"))
    out = torch.full((B, N, Hkv, topk), -7, dtype=torch.int32, device=device)
    ws = ops.alloc_workspace(dims, N, cap, device=device)
    ops.build_pyramid(kt, N, cap, dims, pyr)
    ops.select_prefill(qt, kt, pyr, N, cap, dims, out, ws)
    torch.cuda.synchronize()
    return GpuPrefill(pyr.cpu().numpy(), out.cpu().numpy(), dims, cap)


def pyramid_levels(pyr_bh: np.ndarray, N: int, cap: int):
    """Split one (batch, head) capacity-layout slab into per-level arrays for N keys."""
    sizes = oracle.level_sizes(N)
    cap_offs = oracle.level_offsets(cap)
    return [pyr_bh[cap_offs[l]:cap_offs[l] + m] for l, m in enumerate(sizes)]


def check_pyramid(gpu_pyr: np.ndarray, ref_pyr: np.ndarray, N: int, cap: int) -> float:
    """gpu_pyr [B, Hkv, P, d] vs oracle ref [Hkv, total, d] (B = 1). Returns the worst ratio."""
    sizes = oracle.level_sizes(N)
    ref_offs = oracle.level_offsets(N)
    worst = 0.0
    for j in range(ref_pyr.shape[0]):
        got_levels = pyramid_levels(gpu_pyr[0, j], N, cap)
        for l, m in enumerate(sizes):
            ref = ref_pyr[j, ref_offs[l]:ref_offs[l] + m]
            got = got_levels[l].astype(np.float64)
            assert np.all(np.isfinite(got)), f"non-finite pyramid values at level {l + 1}"
            diff = got - ref
            n2 = np.linalg.norm(diff, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
            ninf = np.abs(diff).max(axis=1) / np.maximum(np.abs(ref).max(axis=1), 1e-30)
            worst = max(worst, float(n2.max()), float(ninf.max()))
            bad = np.nonzero((n2 > PYR_RTOL) | (ninf > PYR_RTOL))[0]
            assert bad.size == 0, (f"head {j} level {l + 1}: {bad.size} nodes beyond tolerance, "
                                   f"worst {max(n2.max(), ninf.max()):.3e} at node {bad[0]}")
    return worst


@dataclasses.dataclass
class ParityReport:
    walks: int = 0
    exact: int = 0
    near_tie_walks: int = 0
    near_tie_by_level: dict = dataclasses.field(default_factory=dict)
    min_gap: float = float("inf")
    mismatch_near_tie: int = 0
    mismatch_valid: int = 0
    mismatch_invalid: int = 0
    mismatch_unverified: int = 0
    min_gap_of_mismatches: float = float("inf")
    hard_fail: int = 0
    first_fail: tuple = ()

    def ok(self) -> bool:
        """Every walk bit-exact, or a near-tie whose GPU result validated as reachable."""
        return self.hard_fail == 0 and self.mismatch_invalid == 0 and self.mismatch_unverified == 0

    def record(self, name: str, **extra) -> dict:
        rec = {k: v for k, v in dataclasses.asdict(self).items() if k != "first_fail"}
        rec["near_tie_by_level"] = {str(k): v for k, v in sorted(self.near_tie_by_level.items())}
        for key in ("min_gap", "min_gap_of_mismatches"):
            rec[key] = None if rec[key] == float("inf") else rec[key]
        return {"config": name, **rec, **extra}

    def __str__(self):
        return (f"walks={self.walks} exact={self.exact} near_tie_walks={self.near_tie_walks} "
                f"mismatch(near-tie)={self.mismatch_near_tie} valid={self.mismatch_valid} "
                f"invalid={self.mismatch_invalid} unverified={self.mismatch_unverified} "
                f"hard_fail={self.hard_fail} first_fail={self.first_fail}")


def compare_selection(gpu_idx: np.ndarray, ts: np.ndarray, q: np.ndarray, k: np.ndarray,
                      ref_pyr: np.ndarray, topk: int, validate_budget: int = 200000,
                      ora=None, score: str = "lse") -> ParityReport:
    """gpu_idx [len(ts), Hkv, K] for positions ts (B = 1); q [N, Hq, d]; k [N, Hkv, d].

    Bit-exact walks are counted in bulk; only mismatches are looked at one by one. A
    mismatch is a hard failure unless the oracle's walk had a near-tie, in which case it
    must validate as a resolution of the ties (a search that runs out of budget is retried
    once with a budget 25 times larger, and counts as unverified -- a failure -- if it
    still cannot decide)."""
    ts = np.asarray(ts, np.int64)
    if ora is None:
        full = len(ts) == q.shape[0] and np.array_equal(ts, np.arange(q.shape[0]))
        ora = oracle.walk(q if full else q[ts], ts, k, ref_pyr, topk, score=score)
    o_idx, o_gap, o_lvl = ora
    rep = ParityReport()
    rep.walks = int(o_gap.size)
    eq = np.all(gpu_idx == o_idx, axis=-1)
    near = o_gap < NEAR_TIE
    rep.exact = int(eq.sum())
    rep.near_tie_walks = int(near.sum())
    if near.any():
        lv, cnt = np.unique(o_lvl[near], return_counts=True)
        rep.near_tie_by_level = {int(a): int(b) for a, b in zip(lv, cnt)}
    fin = np.isfinite(o_gap)
    if fin.any():
        rep.min_gap = float(o_gap[fin].min())
    for i, j in zip(*np.nonzero(~eq)):
        t = int(ts[i])
        gap = float(o_gap[i, j])
        if not near[i, j]:
            rep.hard_fail += 1
            if not rep.first_fail:
                rep.first_fail = (t, int(j), gpu_idx[i, j].tolist(), o_idx[i, j].tolist(), gap)
            continue
        rep.mismatch_near_tie += 1
        rep.min_gap_of_mismatches = min(rep.min_gap_of_mismatches, gap)
        v = oracle.validate(q[t], t, int(j), k, ref_pyr, topk, gpu_idx[i, j], NEAR_TIE, validate_budget,
                            score=score)
        if v < 0:
            v = oracle.validate(q[t], t, int(j), k, ref_pyr, topk, gpu_idx[i, j], NEAR_TIE,
                                25 * validate_budget, score=score)
        if v == 1:
            rep.mismatch_valid += 1
        elif v == 0:
            rep.mismatch_invalid += 1
            if not rep.first_fail:
                rep.first_fail = (t, int(j), gpu_idx[i, j].tolist(), o_idx[i, j].tolist(), gap, "invalid")
        else:
            rep.mismatch_unverified += 1
            if not rep.first_fail:
                rep.first_fail = (t, int(j), gpu_idx[i, j].tolist(), o_idx[i, j].tolist(), gap, "unverified")
    return rep


def sample_positions(N: int, n: int, topk: int, seed: int = 0) -> np.ndarray:
    """Edge positions (first, block boundaries, the at-most-K region, last) plus random ones."""
    rng = np.random.default_rng(seed)
    edges = {0, 1, 63, 64, 65, topk * 64 - 1, topk * 64, 2 * topk * 64, N // 2 - 1, N // 2,
             N - 65, N - 64, N - 2, N - 1}
    edges = {t for t in edges if 0 <= t < N}
    rest = rng.choice(N, size=min(n, N), replace=False)
    return np.array(sorted(edges | set(rest.tolist())), dtype=np.int64)
