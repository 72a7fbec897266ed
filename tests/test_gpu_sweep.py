"""GPU parity over seeded random shapes: the prefill selection through the C ABI against the
fp64 oracle, under the same rule as the fixed workloads (bit-exact index sets, or a near-tie
whose GPU set validates as a resolution of the ties); packs of documents at the same
thresholds against the oracle per document; and decoding steps crossing a threshold, bit for
bit against prefill at the same position.

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


def _threshold_length(rng, K: int, spread: int = 65) -> int:
    """A length near K * 64 * 2^j, where one more pyramid level holds more than K nodes."""
    return int(max(1, K * 64 * (1 << int(rng.integers(0, 5))) + int(rng.integers(-spread, spread + 1))))


def _packed_configs(seed: int, n: int):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        Hq, Hkv = SHAPES[rng.integers(len(SHAPES))]
        K = int(TOPK[rng.integers(len(TOPK))])
        lengths = [_threshold_length(rng, K) for _ in range(int(rng.integers(2, 6)))]
        lengths += [int(x) for x in rng.integers(0, 200, int(rng.integers(1, 4)))]   # short and empty ones
        lengths = [int(x) for x in rng.permutation(lengths)]
        out.append((c, tuple(lengths), Hq, Hkv, K))
    return out


@pytest.mark.parametrize("c,lengths,Hq,Hkv,K", _packed_configs(77, 10))
def test_packed_random_documents(c, lengths, Hq, Hkv, K):
    """Packs of documents whose lengths sit at the start-level thresholds (plus short and empty
    ones): every document against the oracle as a sequence of its own."""
    from test_gpu_packed import _check_docs, _run_packed
    v = synth.make_varlen(sum(lengths), Hq, Hkv, "bf16", lengths=list(lengths), seed=300 + c)
    print(f"[case] packed sweep {c}: lengths={list(lengths)} Hq={Hq} Hkv={Hkv} K={K}", flush=True)
    dims, pyr, idx = _run_packed(v, K)
    _check_docs(v, dims, pyr, idx, K, rows_per_doc=400, seed=c)


def _decode_configs(seed: int, n: int):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        Hq, Hkv = SHAPES[rng.integers(len(SHAPES))]
        K = int(TOPK[rng.integers(len(TOPK))])
        out.append((c, _threshold_length(rng, K, spread=8), Hq, Hkv, K))
    return out


@pytest.mark.parametrize("c,N0,Hq,Hkv,K", _decode_configs(91, 8))
def test_decode_random_shapes_equal_prefill(c, N0, Hq, Hkv, K):
    """Decoding steps from a context length at a start-level threshold, crossing it: each checked
    step selects, bit for bit, what prefill selects at that position (prefill itself being
    compared with the oracle on the same kind of shapes above)."""
    import torch

    from block_selection_amd import ops
    from pisa_testlib import to_device
    steps = 12
    wl = synth.Workload("decode_sweep", N=N0, Hq=Hq, Hkv=Hkv, topk=K, dtype="bf16", decode_steps=steps,
                        seed=700 + c)
    inp = synth.make_decode(wl)
    cap = N0 + steps
    dims = ops.make_dims(1, Hq, Hkv, K, "bf16")
    kc_host = np.zeros((1, cap, Hkv, 64), np.float32)
    kc_host[0, :N0] = inp.k_ctx[0]
    k_cache = to_device(kc_host, "bf16")
    pyr = ops.alloc_pyramid(dims, cap)
    ops.build_pyramid(k_cache, N0, cap, dims, pyr)
    k_new, q_new = to_device(inp.k_new, "bf16"), to_device(inp.q_new, "bf16")
    out = torch.full((1, Hkv, K), -7, dtype=torch.int32, device="cuda")
    ws = ops.alloc_workspace(dims, 1, cap, is_decode=True)
    k_all = np.concatenate([inp.k_ctx[0], inp.k_new[:, 0]], axis=0)
    print(f"[case] decode sweep {c}: N0={N0} Hq={Hq} Hkv={Hkv} K={K}", flush=True)
    for s in range(steps):
        n = N0 + s
        ops.decode_update_select(q_new[s].contiguous(), k_new[s].contiguous(), k_cache, pyr, n, cap, dims, out, ws)
        if s % 4 == 0 or s == steps - 1:
            torch.cuda.synchronize()
            dec = out.cpu().numpy()[0]
            q = np.zeros((1, n + 1, Hq, 64), np.float32)
            q[0, n] = inp.q_new[s, 0]
            ref = run_prefill(q, k_all[None, : n + 1], K, "bf16")
            assert np.array_equal(dec, ref.idx[0, n]), (s, dec, ref.idx[0, n])


def _flat_exact_configs(seed: int, n: int):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        Hq, Hkv = SHAPES[rng.integers(len(SHAPES))]
        K = int(TOPK[rng.integers(len(TOPK))])
        N = int(rng.integers(1, 6001))
        out.append((c, N, Hq, Hkv, K))
    return out


@pytest.mark.parametrize("c,N,Hq,Hkv,K", _flat_exact_configs(313, 12))
def test_flat_exact_random_shape(c, N, Hq, Hkv, K):
    """The exact flat selection at every position of seeded random lengths, group sizes and
    budgets, under the same rule (oracle.flat_exact_select / flat_exact_validate)."""
    from test_gpu_flat_exact import _case
    inp = synth.make_prefill(synth.Workload("sweep_flat_exact", N=N, Hq=Hq, Hkv=Hkv, topk=K, dtype="bf16",
                                            seed=9000 + c))
    _case(f"sweep{c}", inp.q, inp.k, K)
