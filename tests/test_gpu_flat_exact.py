"""GPU parity of the exact flat selection (pisa_select_flat_exact) against the oracle.

Every compared (position, KV head) must give the oracle's set bit for bit, or the oracle's
K-th and (K+1)-th exact block scores differ by less than 1e-3 and the GPU's set is one of the
tie resolutions (oracle.flat_exact_validate). Workloads: every position of the 4K selection
benchmark shape; sampled positions at 32K (planted) and 64K; edge lengths around one and two
blocks; group sizes 1-16 and budgets 1-32; a batch; all-zero keys (exact ties, lowest blocks
win). Where the walk scores only the leaf level (at most K nodes on level 2), the walk's
selection must equal the exact flat selection bit for bit: both score a leaf with the same
arithmetic.
"""
import numpy as np
import pytest
import torch

import oracle
import parity_log
from block_selection_amd import synth
from pisa_testlib import NEAR_TIE, ParityReport, run_prefill, to_device

pytestmark = pytest.mark.gpu


def run_flat_exact(q: np.ndarray, k: np.ndarray, topk: int) -> np.ndarray:
    from block_selection_amd import ops
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    dims = ops.make_dims(B, Hq, Hkv, topk, "bf16")
    qt, kt = to_device(q, "bf16"), to_device(k, "bf16")
    out = torch.full((B, N, Hkv, topk), -7, dtype=torch.int32, device="cuda")
    ops.select_flat_exact(qt, kt, N, N, dims, out, ops.alloc_flat_exact_workspace(dims, N))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def compare_flat_exact(gpu_idx, ts, q, k, topk) -> ParityReport:
    """gpu_idx [len(ts), Hkv, K]; q [N, Hq, d] and k [N, Hkv, d] of one batch element."""
    o_idx, o_gap = oracle.flat_exact_select(q[ts], ts, k, topk)
    rep = ParityReport(walks=int(o_gap.size))
    eq = np.all(gpu_idx == o_idx, axis=-1)
    near = o_gap < NEAR_TIE
    rep.exact, rep.near_tie_walks = int(eq.sum()), int(near.sum())
    fin = np.isfinite(o_gap)
    rep.min_gap = float(o_gap[fin].min()) if fin.any() else float("inf")
    for i, j in zip(*np.nonzero(~eq)):
        t = int(ts[i])
        if not near[i, j]:
            rep.hard_fail += 1
            if not rep.first_fail:
                rep.first_fail = (t, int(j), gpu_idx[i, j].tolist(), o_idx[i, j].tolist(), float(o_gap[i, j]))
            continue
        rep.mismatch_near_tie += 1
        rep.min_gap_of_mismatches = min(rep.min_gap_of_mismatches, float(o_gap[i, j]))
        if oracle.flat_exact_validate(q[t], t, int(j), k, topk, gpu_idx[i, j], NEAR_TIE) == 1:
            rep.mismatch_valid += 1
        else:
            rep.mismatch_invalid += 1
            if not rep.first_fail:
                rep.first_fail = (t, int(j), gpu_idx[i, j].tolist(), o_idx[i, j].tolist(), "invalid")
    return rep


def _case(name, q, k, topk, n_sample=None, seed=0):
    B, N = q.shape[:2]
    print(f"[case] flat_exact {name} B={B} N={N} Hq={q.shape[2]} Hkv={k.shape[2]} K={topk}", flush=True)
    got = run_flat_exact(q, k, topk)
    for b in range(B):
        if n_sample is None:
            ts = np.arange(N)
        else:
            rng = np.random.default_rng(seed)
            edges = {0, 1, 63, 64, 65, 127, 128, 64 * topk - 1, 64 * topk, 64 * topk + 1, N // 2, N - 65, N - 64,
                     N - 1}
            ts = np.array(sorted({t for t in edges if 0 <= t < N} | set(rng.choice(N, n_sample, replace=False).tolist())))
        rep = compare_flat_exact(got[b, ts], ts, q[b], k[b], topk)
        parity_log.add(rep.record(f"flat_exact_{name}_N{N}_K{topk}" + (f"_b{b}" if B > 1 else ""),
                                  positions=int(len(ts)), all_positions=n_sample is None))
        assert rep.ok(), str(rep)
    return got


def test_flat_exact_short_all_positions():
    wl = synth.WORKLOADS["short"]
    inp = synth.make_prefill(wl)
    _case("short", inp.q, inp.k, wl.topk)


@pytest.mark.parametrize("name,n_sample", [("mid_planted", 600), ("long64k", 200)])
def test_flat_exact_long_sampled(name, n_sample):
    wl = synth.WORKLOADS[name]
    inp = synth.make_prefill(wl)
    _case(name, inp.q, inp.k, wl.topk, n_sample=n_sample, seed=3)


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 127, 128, 129, 1000, 4001])
def test_flat_exact_edge_lengths(N):
    inp = synth.make_prefill(synth.Workload("ragged", N=N, Hq=32, Hkv=2, topk=8, dtype="bf16", seed=N))
    _case("ragged", inp.q, inp.k, 8)


@pytest.mark.parametrize("Hq,Hkv,K", [(8, 1, 1), (16, 2, 4), (6, 3, 16), (16, 1, 17), (32, 2, 32), (12, 3, 24),
                                      (20, 4, 7)])
def test_flat_exact_shape_variants(Hq, Hkv, K):
    inp = synth.make_prefill(synth.Workload("variant", N=5000, Hq=Hq, Hkv=Hkv, topk=K, dtype="bf16", seed=Hq + K))
    _case("variant", inp.q, inp.k, K, n_sample=1500, seed=K)


def test_flat_exact_batched():
    inp = synth.make_prefill(synth.Workload("batched", N=2500, Hq=8, Hkv=2, topk=8, dtype="bf16", B=3, seed=4))
    _case("batched", inp.q, inp.k, 8)


@pytest.mark.parametrize("N,Hq,Hkv,K", [(1000, 32, 2, 8), (2048, 16, 1, 16), (700, 6, 3, 6), (4096, 8, 2, 32)])
def test_flat_exact_equals_walk_on_leaf_only_shapes(N, Hq, Hkv, K):
    """At most K nodes on level 2: the walk scores every eligible leaf and keeps the K best,
    which is the exact flat selection, computed with the same leaf arithmetic: bit for bit."""
    assert -(-N // 128) <= K
    inp = synth.make_prefill(synth.Workload("leafonly", N=N, Hq=Hq, Hkv=Hkv, topk=K, dtype="bf16", seed=N + K))
    print(f"[case] flat_exact leaf-only N={N} Hq={Hq} Hkv={Hkv} K={K}", flush=True)
    walk = run_prefill(inp.q, inp.k, K, "bf16")
    flat = run_flat_exact(inp.q, inp.k, K)
    np.testing.assert_array_equal(walk.idx, flat)


def test_flat_exact_zero_keys_lowest_blocks():
    """All keys zero: every block's score is the group's sum of log(m) over its m keys up to t,
    so every full block ties and the lowest win; the query's own partial block (fewer keys)
    scores lower than any full one. Checked bit for bit at every position."""
    N, K = 3000, 8
    rng = np.random.default_rng(2)
    q = synth.bf16_round(rng.standard_normal((1, N, 16, 64), dtype=np.float32))
    k = np.zeros((1, N, 2, 64), np.float32)
    got = run_flat_exact(q, k, K)
    for t in range(N):
        full = (t + 1) // 64                  # blocks with all 64 keys up to t
        part = [] if (t + 1) % 64 == 0 else [t // 64]
        keep = list(range(min(K, full)))
        keep += part[:K - len(keep)]
        want = sorted(keep) + [-1] * (K - len(keep))
        assert got[0, t, 0].tolist() == want and got[0, t, 1].tolist() == want, t


def test_flat_exact_rejects_unsupported():
    from block_selection_amd import ops
    N = 256
    for dtype, score in (("f32", "lse"), ("bf16", "mean")):
        dims = ops.make_dims(1, 8, 2, 4, dtype, score=score)
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        q = torch.zeros((1, N, 8, 64), dtype=tdt, device="cuda")
        k = torch.zeros((1, N, 2, 64), dtype=tdt, device="cuda")
        out = torch.zeros((1, N, 2, 4), dtype=torch.int32, device="cuda")
        ws = torch.empty(ops.flat_exact_workspace_bytes(dims, N), dtype=torch.uint8, device="cuda")
        with pytest.raises(ops.PisaError):
            ops.select_flat_exact(q, k, N, N, dims, out, ws)
    dims = ops.make_dims(1, 8, 2, 4, "bf16")
    q = torch.zeros((1, N, 8, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, N, 2, 64), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((1, N, 2, 4), dtype=torch.int32, device="cuda")
    small = torch.empty(ops.flat_exact_workspace_bytes(dims, N) - 512, dtype=torch.uint8, device="cuda")
    with pytest.raises(ops.PisaError):
        ops.select_flat_exact(q, k, N, N, dims, out, small)
