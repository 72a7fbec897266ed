"""GPU parity over seeded random shapes: the prefill selection through the C ABI against the
fp64 oracle, under the same rule as the fixed workloads (bit-exact index sets, or a near-tie
whose GPU set validates as a resolution of the ties).

The shapes are drawn around the lengths where the walk's first scored level changes: N near
K * 64 * 2^j, the key count at which one more level of the pyramid holds more than K nodes
(the walk starts at the highest such level, every eligible node of it a candidate). GQA groups
of 1 to 16 heads (including groups that do not fill a 4-head lane quarter), K from 1 to 32,
bf16 and fp32 inputs and the three scores. Every position is compared up to 6000 keys,
sampled positions (block edges plus seeded random rows) above.
"""
import numpy as np
import pytest

import oracle
from block_selection_amd import synth
from pisa_testlib import check_pyramid, compare_selection, run_prefill, sample_positions

pytestmark = pytest.mark.gpu

SHAPES = [(32, 2), (16, 16), (8, 1), (24, 8), (20, 4), (6, 3), (16, 1), (64, 4)]   # (Hq, Hkv)
TOPK = [1, 2, 3, 5, 7, 8, 9, 12, 16, 24, 31, 32]
SCORES = ["lse", "lse", "lse", "mean", "mean_half_var"]


def _configs(seed: int, n: int):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        Hq, Hkv = SHAPES[rng.integers(len(SHAPES))]
        K = int(TOPK[rng.integers(len(TOPK))])
        N = int(max(1, K * 64 * (1 << int(rng.integers(0, 6))) + int(rng.integers(-65, 66))))
        dtype = "bf16" if rng.random() < 0.75 else "f32"
        score = SCORES[rng.integers(len(SCORES))]
        out.append((c, N, Hq, Hkv, K, dtype, score))
    return out


@pytest.mark.parametrize("c,N,Hq,Hkv,K,dtype,score", _configs(2024, 40))
def test_prefill_random_shape(c, N, Hq, Hkv, K, dtype, score):
    wl = synth.Workload("sweep", N=N, Hq=Hq, Hkv=Hkv, topk=K, dtype=dtype, seed=5000 + c)
    inp = synth.make_prefill(wl)
    print(f"[case] sweep {c}: N={N} Hq={Hq} Hkv={Hkv} K={K} dtype={dtype} score={score}", flush=True)
    gpu = run_prefill(inp.q, inp.k, K, dtype, score=score)
    k0 = inp.k[0]
    ref = oracle.build_pyramid(k0)
    assert check_pyramid(gpu.pyramid, ref, N, gpu.cap) <= 1e-5
    ts = np.arange(N) if N <= 6000 else sample_positions(N, 1500, K, seed=c)
    rep = compare_selection(gpu.idx[0, ts], ts, inp.q[0], k0, ref, K, score=score)
    assert rep.ok(), str(rep)
