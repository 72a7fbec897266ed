"""GPU parity of the flat stage-one selection (pisa_select_flat) against the oracle.

Every compared (position, KV head) must give the oracle's set bit for bit, or the oracle's
K-th and (K+1)-th flat scores differ by less than 1e-3 and the GPU's set is one of the
tie resolutions (oracle.flat_validate). Workloads: the selection benchmark's shapes (every
position at 4K, 32K planted and 64K; sampled at 256K), edge lengths, budgets 1-32 (both
list capacities of the kernel), group sizes 1-16, fp32 and bf16 inputs, batches, and
score orders that stress the kernel's candidate lists (scores rising with the block index,
so every block displaces the K-th; exact ties everywhere).
"""
import numpy as np
import pytest
import torch

import oracle
import parity_log
from block_selection_amd import synth
from pisa_testlib import NEAR_TIE, ParityReport, to_device

pytestmark = pytest.mark.gpu


def run_flat(q: np.ndarray, k: np.ndarray, topk: int, dtype: str) -> np.ndarray:
    from block_selection_amd import ops
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    dims = ops.make_dims(B, Hq, Hkv, topk, dtype)
    qt, kt = to_device(q, dtype), to_device(k, dtype)
    pyr = ops.alloc_pyramid(dims, N)
    out = torch.full((B, N, Hkv, topk), -7, dtype=torch.int32, device="cuda")
    ops.build_pyramid(kt, N, N, dims, pyr)
    ops.select_flat(qt, pyr, N, N, dims, out, ops.alloc_flat_workspace(dims, N))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def compare_flat(gpu_idx, ts, q, pyr, N, topk) -> ParityReport:
    """gpu_idx [len(ts), Hkv, K]; q [N, Hq, d] of one batch element; pyr its oracle pyramid."""
    full = len(ts) == N
    o_idx, o_gap = oracle.flat_select(q if full else q[ts], ts, pyr, N, topk)
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
        if oracle.flat_validate(q[t], t, int(j), pyr, N, topk, gpu_idx[i, j], NEAR_TIE) == 1:
            rep.mismatch_valid += 1
        else:
            rep.mismatch_invalid += 1
            if not rep.first_fail:
                rep.first_fail = (t, int(j), gpu_idx[i, j].tolist(), o_idx[i, j].tolist(), "invalid")
    return rep


def _case(name, q, k, topk, dtype, n_sample=None, seed=0):
    B, N = q.shape[:2]
    print(f"[case] flat {name} B={B} N={N} Hq={q.shape[2]} Hkv={k.shape[2]} K={topk} {dtype}", flush=True)
    got = run_flat(q, k, topk, dtype)
    for b in range(B):
        pyr = oracle.build_pyramid(k[b])
        if n_sample is None:
            ts = np.arange(N)
        else:
            rng = np.random.default_rng(seed)
            edges = {0, 1, 63, 64, 65, 64 * topk - 1, 64 * topk, N // 2, N - 65, N - 64, N - 1}
            ts = np.array(sorted({t for t in edges if 0 <= t < N} | set(rng.choice(N, n_sample, replace=False).tolist())))
        rep = compare_flat(got[b, ts], ts, q[b], pyr, N, topk)
        parity_log.add(rep.record(f"flat_{name}_N{N}_K{topk}" + (f"_b{b}" if B > 1 else ""),
                                  positions=int(len(ts)), all_positions=n_sample is None))
        assert rep.ok(), str(rep)
    return got


@pytest.mark.parametrize("name", ["short", "mid_planted", "long64k"])
def test_flat_benchmark_shapes_all_positions(name):
    wl = synth.WORKLOADS[name]
    inp = synth.make_prefill(wl)
    _case(name, inp.q, inp.k, wl.topk, wl.dtype)


def test_flat_256k_sampled():
    wl = synth.WORKLOADS["long256k"]
    inp = synth.make_prefill(wl)
    _case("long256k", inp.q, inp.k, wl.topk, wl.dtype, n_sample=1500)


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 127, 1000, 4001])
def test_flat_edge_lengths(N):
    inp = synth.make_prefill(synth.Workload("ragged", N=N, Hq=32, Hkv=2, topk=8, dtype="bf16", seed=N))
    _case("ragged", inp.q, inp.k, 8, "bf16")


@pytest.mark.parametrize("Hq,Hkv,K,dtype", [(8, 1, 1, "bf16"), (16, 2, 4, "bf16"), (6, 3, 16, "bf16"),
                                             (16, 1, 17, "bf16"), (32, 2, 32, "bf16"), (4, 4, 8, "f32"),
                                             (12, 3, 24, "f32")])
def test_flat_shape_variants(Hq, Hkv, K, dtype):
    inp = synth.make_prefill(synth.Workload("variant", N=9000, Hq=Hq, Hkv=Hkv, topk=K, dtype=dtype, seed=Hq + K))
    _case("variant", inp.q, inp.k, K, dtype, n_sample=2500, seed=K)


def test_flat_batched():
    inp = synth.make_prefill(synth.Workload("batched", N=3001, Hq=8, Hkv=2, topk=8, dtype="bf16", B=3, seed=4))
    _case("batched", inp.q, inp.k, 8, "bf16")


@pytest.mark.parametrize("K", [8, 32])
def test_flat_rising_scores(K):
    """Block b's keys are (b + 1) * 0.01 * e_0 and every query is e_0: each block beats every
    earlier one, so every block enters the list and the lists are cut back at every chance.
    The K latest eligible blocks are selected."""
    N = 6000
    k = np.zeros((1, N, 1, 64), np.float32)
    for b in range(-(-N // 64)):
        k[0, b * 64:(b + 1) * 64, 0, 0] = (b + 1) * 0.01
    q = np.zeros((1, N, 4, 64), np.float32)
    q[0, :, :, 0] = 1.0
    got = _case("rising", q, k, K, "f32")
    for t in (0, 100, 64 * K + 5, N - 1):
        last = t // 64
        want = list(range(max(0, last - K + 1), last + 1))
        assert got[0, t, 0].tolist() == want + [-1] * (K - len(want)), t


@pytest.mark.parametrize("K", [8, 32])
def test_flat_exact_ties_lowest_index(K):
    """All keys zero: every score is exactly 0, so the K lowest eligible blocks win, bit-exact."""
    N = 5000
    rng = np.random.default_rng(2)
    q = synth.bf16_round(rng.standard_normal((1, N, 16, 64), dtype=np.float32))
    k = np.zeros((1, N, 2, 64), np.float32)
    got = run_flat(q, k, K, "bf16")
    for t in range(N):
        m = min(K, t // 64 + 1)
        want = list(range(m)) + [-1] * (K - m)
        assert got[0, t, 0].tolist() == want and got[0, t, 1].tolist() == want, t
