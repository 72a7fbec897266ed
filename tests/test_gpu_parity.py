"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Pyramids are compared node by node, selections walk by walk under the rule in
pisa_testlib (bit-exact index sets; near-ties counted and validated, an
unreachable or undecided mismatch fails). The five workloads -- tiny, short,
mid_planted, long64k/128k/256k and decode128k -- are compared at every query
position and KV head (every step for decoding), in the launch configuration
the benchmark times. Deeper trees (524288 positions) and larger budgets at
262144 positions are compared at sampled positions (block edges, the at-most-K
region, the last rows, plus seeded random rows). Every compared workload adds
a record (walks, exact, near-tie walks by level, mismatches by validation
outcome) that the session prints at its end.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from block_selection_amd import synth
import parity_log
from pisa_testlib import (NEAR_TIE, ParityReport, check_pyramid, compare_selection, pyramid_levels, run_prefill,
                          sample_positions, to_device)

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _log(name, rep, extra=None):
    parity_log.add(rep.record(name, **(extra or {})))


def _prefill_case(wl, n_sample=None, N=None, cap=None, score="lse"):
    inp = synth.make_prefill(wl, N=N)
    N = inp.q.shape[1]
    print(f"[case] {wl.name} N={N} Hq={wl.Hq} Hkv={wl.Hkv} K={wl.topk} dtype={wl.dtype} cap={cap} "
          f"score={score}", flush=True)
    gpu = run_prefill(inp.q, inp.k, wl.topk, wl.dtype, cap=cap, score=score)
    k0 = inp.k[0]
    ref_pyr = oracle.build_pyramid(k0)
    worst = check_pyramid(gpu.pyramid, ref_pyr, N, gpu.cap)
    ts = np.arange(N) if n_sample is None else sample_positions(N, n_sample, wl.topk)
    rep = compare_selection(gpu.idx[0, ts], ts, inp.q[0], k0, ref_pyr, wl.topk, score=score)
    tag = "" if score == "lse" else f"_{score}"
    _log(f"prefill_{wl.name}_N{N}_K{wl.topk}{tag}", rep,
         {"pyramid_worst_rel": worst, "positions": int(len(ts)), "all_positions": n_sample is None})
    assert rep.ok(), str(rep)
    return inp, gpu, rep


def test_prefill_tiny_all_positions():
    _prefill_case(synth.WORKLOADS["tiny"])


def test_prefill_short_all_positions():
    _prefill_case(synth.WORKLOADS["short"])


def test_prefill_mid_planted_all_positions():
    _prefill_case(synth.WORKLOADS["mid_planted"])


@pytest.mark.parametrize("name", ["long64k", "long128k", "long256k"])
def test_prefill_long_all_positions(name):
    _prefill_case(synth.WORKLOADS[name])


def test_prefill_512k_sampled():
    """A tree one level deeper than the headline (524288 positions, 14 levels; one KV head of 16
    query heads): sampled positions against the oracle."""
    wl = synth.Workload("long512k", N=524288, Hq=16, Hkv=1, topk=8, dtype="bf16", seed=17)
    _prefill_case(wl, n_sample=400)


def test_prefill_1m_sliced_buckets_sampled():
    """1048640 positions at Hkv = 2: 16386 (KV head, sibling pair) groups, more than the
    16384 bins one pass of the leaf stage's bucket histogram holds, so each range is counted
    and filled in two slices; sampled positions (edges included) against the oracle."""
    wl = synth.Workload("long1m", N=1048640, Hq=32, Hkv=2, topk=8, dtype="bf16", seed=19)
    _prefill_case(wl, n_sample=300)


@pytest.mark.parametrize("topk", [16, 32])
def test_prefill_256k_larger_budgets(topk):
    """The headline shape (262144 positions, Hq=32, Hkv=2) at K = 16 and 32 (the budgets
    bench.py also times): sampled positions against the oracle."""
    wl = synth.Workload(f"long256k_k{topk}", N=262144, Hq=32, Hkv=2, topk=topk, dtype="bf16", seed=3)
    _prefill_case(wl, n_sample=300)


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 1000, 4001])
def test_prefill_ragged_lengths(N):
    wl = synth.Workload("ragged", N=N, Hq=32, Hkv=2, topk=8, dtype="bf16", seed=N)
    _prefill_case(wl)


@pytest.mark.parametrize("Hq,Hkv,K,dtype", [(8, 1, 32, "bf16"), (16, 2, 1, "bf16"), (6, 3, 5, "f32"),
                                             (16, 1, 16, "bf16"), (2, 2, 8, "f32"), (12, 3, 5, "bf16"),
                                             (32, 2, 12, "bf16")])
def test_prefill_shape_variants(Hq, Hkv, K, dtype):
    wl = synth.Workload("variant", N=8192, Hq=Hq, Hkv=Hkv, topk=K, dtype=dtype, seed=Hq * 100 + K)
    _prefill_case(wl, n_sample=1500)


# The pages' two ablation scores (first- and second-order truncations of the LSE):
# the same walk, each scored against the oracle with the same score.
@pytest.mark.parametrize("score", ["mean", "mean_half_var"])
@pytest.mark.parametrize("name", ["tiny", "short"])
def test_prefill_truncated_scores(name, score):
    _prefill_case(synth.WORKLOADS[name], score=score)


@pytest.mark.parametrize("score", ["mean", "mean_half_var"])
@pytest.mark.parametrize("N,Hq,Hkv,K,dtype", [(4001, 32, 2, 8, "bf16"), (8192, 12, 3, 5, "bf16"),
                                               (8192, 16, 1, 16, "bf16"), (3000, 6, 3, 5, "f32")])
def test_prefill_truncated_scores_shapes(N, Hq, Hkv, K, dtype, score):
    wl = synth.Workload("trunc", N=N, Hq=Hq, Hkv=Hkv, topk=K, dtype=dtype, seed=N + K)
    _prefill_case(wl, n_sample=1200, score=score)


@pytest.mark.parametrize("score", ["mean", "mean_half_var"])
def test_prefill_truncated_scores_long64k(score):
    _prefill_case(synth.WORKLOADS["long64k"], n_sample=600, score=score)


def test_prefill_capacity_layout():
    """A pyramid laid out for more keys than present (as decoding uses) selects the same."""
    wl = synth.Workload("cap", N=5000, Hq=32, Hkv=2, topk=8, dtype="bf16", seed=5)
    _prefill_case(wl, n_sample=800, cap=9000)


def test_closed_form_walk_on_gpu():
    """Hand-derived selections (tests/golden/closed_form_walk.json), including an exact tie."""
    with open(os.path.join(GOLDEN, "closed_form_walk.json")) as f:
        fx = json.load(f)
    N, C, d = fx["N"], fx["C"], fx["d"]
    k = np.zeros((1, N, 1, d), np.float32)
    for b, c in enumerate(fx["leaf_logit"]):
        k[0, b * C:(b + 1) * C, 0, 0] = c
    q = np.zeros((1, N, 1, d), np.float32)
    q[0, :, 0, 0] = fx["q_first_coord"]
    for dtype in ("f32", "bf16"):
        gpu = run_prefill(q, k, fx["topk"], dtype)
        for case in fx["cases"]:
            assert gpu.idx[0, case["t"], 0].tolist() == case["expect"], (dtype, case["t"])


def test_zero_keys_ties_lowest_index():
    """All logits 0: full blocks tie exactly; the lowest eligible indices must win, bit-exact."""
    N, K = 8192, 8
    rng = np.random.default_rng(4)
    q = synth.bf16_round(rng.standard_normal((1, N, 32, 64), dtype=np.float32))
    k = np.zeros((1, N, 2, 64), np.float32)
    gpu = run_prefill(q, k, K, "bf16")
    n_elig = np.arange(N) // 64 + 1
    want = np.full((N, K), -1, np.int32)
    for t in range(N):
        m = min(K, n_elig[t])
        want[t, :m] = np.arange(m)
    for j in range(2):
        assert np.array_equal(gpu.idx[0, :, j], want)


def test_prefill_deterministic():
    wl = synth.WORKLOADS["short"]
    inp = synth.make_prefill(wl)
    a = run_prefill(inp.q, inp.k, wl.topk, wl.dtype)
    b = run_prefill(inp.q, inp.k, wl.topk, wl.dtype)
    assert np.array_equal(a.idx, b.idx)
    assert np.array_equal(a.pyramid.view(np.uint32), b.pyramid.view(np.uint32))


def test_planted_recall_matches_oracle():
    """Planted blocks: the GPU's recall over the sampled positions equals the oracle's."""
    wl = synth.WORKLOADS["mid_planted"]
    inp = synth.make_prefill(wl)
    gpu = run_prefill(inp.q, inp.k, wl.topk, wl.dtype)
    k0 = inp.k[0]
    ref_pyr = oracle.build_pyramid(k0)
    ts = sample_positions(wl.N, 1500, wl.topk, seed=9)
    ts = ts[ts >= wl.topk * 64]
    o_idx, _, _ = oracle.walk(inp.q[0, ts], ts, k0, ref_pyr, wl.topk)
    planted = set(inp.planted.tolist())

    def recall(idx):
        vals = []
        for i, t in enumerate(ts):
            elig = {b for b in planted if b * 64 <= t}
            if not elig:
                continue
            for j in range(2):
                sel = set(idx[i, j].tolist())
                vals.append(len(sel & elig) / min(wl.topk, len(elig)))
        return float(np.mean(vals))

    r_gpu, r_ora = recall(gpu.idx[0, ts]), recall(o_idx)
    print(json.dumps({"planted_recall_gpu": r_gpu, "planted_recall_oracle": r_ora}), flush=True)
    assert abs(r_gpu - r_ora) < 0.01


# ------------------------------------------------------------------ decode ---

def _decode_run(N0, steps, check_every=1, oracle_every=1, score="lse", name=None):
    from block_selection_amd import ops
    wl = synth.Workload("decode", N=N0, Hq=32, Hkv=2, topk=32, dtype="bf16", decode_steps=steps)
    inp = synth.make_decode(wl)
    cap = N0 + steps
    dims = ops.make_dims(1, 32, 2, 32, "bf16", score=score)
    k_all = np.concatenate([inp.k_ctx[0], inp.k_new[:, 0]], axis=0)   # [cap, Hkv, d]
    kc_host = np.zeros((1, cap, 2, 64), np.float32)
    kc_host[0, :N0] = inp.k_ctx[0]
    k_cache = to_device(kc_host, "bf16")
    pyr = ops.alloc_pyramid(dims, cap)
    ops.build_pyramid(k_cache, N0, cap, dims, pyr)
    k_new = to_device(inp.k_new, "bf16")      # [steps, 1, Hkv, d]
    q_new = to_device(inp.q_new, "bf16")      # [steps, 1, Hq, d]
    out = torch.full((1, 2, 32), -7, dtype=torch.int32, device="cuda")
    ws = ops.alloc_workspace(dims, 1, cap, is_decode=True)
    ref_k = to_device(np.concatenate([kc_host[0, :N0], inp.k_new[:, 0]], 0)[None], "bf16")
    pyr_rb = ops.alloc_pyramid(dims, cap)
    rep = ParityReport()
    for s in range(steps):
        n = N0 + s
        ops.decode_update_select(q_new[s].contiguous(), k_new[s].contiguous(), k_cache, pyr, n, cap,
                                 dims, out, ws)
        torch.cuda.synchronize()
        gpu_idx = out.cpu().numpy()[0]
        if s % check_every == 0 or s == steps - 1:
            # incremental == full rebuild, bitwise, on every node that exists at n + 1 keys
            ops.build_pyramid(ref_k, n + 1, cap, dims, pyr_rb)
            a, b = pyr.cpu().numpy(), pyr_rb.cpu().numpy()
            for j in range(2):
                for la, lb in zip(pyramid_levels(a[0, j], n + 1, cap), pyramid_levels(b[0, j], n + 1, cap)):
                    assert np.array_equal(la.view(np.uint32), lb.view(np.uint32)), (s, j)
        if s % oracle_every == 0 or s == steps - 1:
            ref_pyr, o_idx, o_gap, o_lvl = oracle.decode_step(k_all, n, inp.q_new[s, 0], 32, score=score,
                                                              with_level=True)
            if s == 0 or s == steps - 1:
                check_pyramid(pyr.cpu().numpy(), ref_pyr, n + 1, cap)
            step = compare_selection(gpu_idx[None], np.array([n]), _RowView(inp.q_new[s, 0], n), k_all[: n + 1],
                                     ref_pyr, 32, ora=(o_idx[None], o_gap[None], o_lvl[None]), score=score)
            _merge(rep, step)
            assert step.ok(), (s, str(step))
    if name:
        _log(name, rep, {"steps": steps, "context": N0})
    return rep


class _RowView:
    """q[t] of a single decoding query: the one row at position n (compare_selection reads q[t])."""

    def __init__(self, row, n):
        self.row, self.n = row, n
        self.shape = (n + 1,) + row.shape

    def __getitem__(self, t):
        assert t == self.n
        return self.row


def _merge(acc: ParityReport, one: ParityReport) -> None:
    for f in ("walks", "exact", "near_tie_walks", "mismatch_near_tie", "mismatch_valid", "mismatch_invalid",
              "mismatch_unverified", "hard_fail"):
        setattr(acc, f, getattr(acc, f) + getattr(one, f))
    for lv, c in one.near_tie_by_level.items():
        acc.near_tie_by_level[lv] = acc.near_tie_by_level.get(lv, 0) + c
    acc.min_gap = min(acc.min_gap, one.min_gap)
    acc.min_gap_of_mismatches = min(acc.min_gap_of_mismatches, one.min_gap_of_mismatches)
    if not acc.first_fail and one.first_fail:
        acc.first_fail = one.first_fail


def test_decode_small_context():
    """Decode from 1000 keys: crosses leaf boundaries and two new pyramid levels."""
    _decode_run(1000, 100, name="decode_from1000_100steps_K32")


@pytest.mark.parametrize("score", ["mean", "mean_half_var"])
def test_decode_truncated_scores(score):
    """Decode from 1000 keys with the truncated scores: rebuild-equal pyramid, oracle parity."""
    _decode_run(1000, 60, score=score, name=f"decode_from1000_60steps_K32_{score}")


def test_decode_128k_256_steps():
    """The decode workload: 131072 prebuilt keys, 256 steps, K = 32; step 0 adds a root level."""
    _decode_run(131072, 256, check_every=1, oracle_every=1, name="decode128k_256steps_K32")


@pytest.mark.parametrize("topk,score", [(32, "lse"), (8, "lse"), (32, "mean"), (8, "mean_half_var")])
def test_decode_equals_prefill_at_same_position(topk, score):
    """A decode step selects, bit for bit, what prefill selects for position n over n + 1 keys
    (both paths share the scoring arithmetic); 5000 context keys, 24 steps."""
    from block_selection_amd import ops
    N0, steps = 5000, 24
    wl = synth.Workload("decode", N=N0, Hq=32, Hkv=2, topk=topk, dtype="bf16", decode_steps=steps)
    inp = synth.make_decode(wl)
    cap = N0 + steps
    dims = ops.make_dims(1, 32, 2, topk, "bf16", score=score)
    kc_host = np.zeros((1, cap, 2, 64), np.float32)
    kc_host[0, :N0] = inp.k_ctx[0]
    k_cache = to_device(kc_host, "bf16")
    pyr = ops.alloc_pyramid(dims, cap)
    ops.build_pyramid(k_cache, N0, cap, dims, pyr)
    k_new = to_device(inp.k_new, "bf16")
    q_new = to_device(inp.q_new, "bf16")
    out = torch.full((1, 2, topk), -7, dtype=torch.int32, device="cuda")
    ws = ops.alloc_workspace(dims, 1, cap, is_decode=True)
    k_all = np.concatenate([inp.k_ctx[0], inp.k_new[:, 0]], axis=0)
    checked = 0
    for s in range(steps):
        n = N0 + s
        print(f"[case] decode-vs-prefill K={topk} step={s} n={n}", flush=True)
        ops.decode_update_select(q_new[s].contiguous(), k_new[s].contiguous(), k_cache, pyr, n, cap,
                                 dims, out, ws)
        if s % 6 == 0 or s == steps - 1:
            torch.cuda.synchronize()
            dec = out.cpu().numpy()[0]
            q = np.zeros((1, n + 1, 32, 64), np.float32)
            q[0, n] = inp.q_new[s, 0]
            ref = run_prefill(q, k_all[None, : n + 1], topk, "bf16", score=score)
            assert np.array_equal(dec, ref.idx[0, n]), (s, dec, ref.idx[0, n])
            checked += 1
    assert checked == 5


def test_decode_workspace_needs_no_zeroing():
    """The decoding step's completion counters are tagged per call, so a workspace holding
    stray bytes, or counters one arrival short of "last" under a foreign tag, gives bit for bit
    the selection and pyramid of a zero-filled one (B = 2, K = 16: four workgroups per
    (batch, KV head) meet at each counter)."""
    from block_selection_amd import ops
    B, K, N0, steps = 2, 16, 3000, 6
    wl = synth.Workload("decode_ws", N=N0, Hq=16, Hkv=2, topk=K, dtype="bf16", B=B, decode_steps=steps, seed=9)
    inp = synth.make_decode(wl)
    cap = N0 + steps
    dims = ops.make_dims(B, 16, 2, K, "bf16")
    kc_host = np.zeros((B, cap, 2, 64), np.float32)
    kc_host[:, :N0] = inp.k_ctx
    k_new, q_new = to_device(inp.k_new, "bf16"), to_device(inp.q_new, "bf16")
    nbytes = ops.workspace_bytes(dims, 1, cap, True)
    gen = torch.Generator(device="cpu").manual_seed(3)

    def run(poison):
        k_cache = to_device(kc_host, "bf16")
        pyr = ops.alloc_pyramid(dims, cap)
        ops.build_pyramid(k_cache, N0, cap, dims, pyr)
        ws = ops.alloc_workspace(dims, 1, cap, is_decode=True)
        out = torch.full((B, 2, K), -7, dtype=torch.int32, device="cuda")
        sel = []
        for s in range(steps):
            if poison == "bytes":
                ws.copy_(torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=gen).cuda())
            elif poison == "one_short":
                words = torch.randint(1, 1 << 31, (B * 2,), dtype=torch.int64, generator=gen)
                ws[: 8 * B * 2].copy_(((words << 32) | 3).view(torch.uint8).cuda())
            print(f"[case] decode workspace poison={poison} step={s}", flush=True)
            ops.decode_update_select(q_new[s].contiguous(), k_new[s].contiguous(), k_cache, pyr, N0 + s, cap,
                                     dims, out, ws)
            torch.cuda.synchronize()
            sel.append(out.cpu().numpy().copy())
        return np.stack(sel), pyr.cpu().numpy()

    ref_sel, ref_pyr = run(None)
    assert (ref_sel >= 0).all()
    for poison in ("bytes", "one_short"):
        sel, pyr = run(poison)
        assert np.array_equal(sel, ref_sel), poison
        assert np.array_equal(pyr.view(np.uint32), ref_pyr.view(np.uint32)), poison


@pytest.mark.parametrize("B,dtype", [(3, "bf16"), (4, "bf16"), (3, "f32")])
def test_prefill_batched(B, dtype):
    """Several batch elements with their own keys and queries (B*Hkv = 6 or 8 walks per
    position): each element matches the oracle run on it alone."""
    wl = synth.Workload("batched", N=3001, Hq=8, Hkv=2, topk=8, dtype=dtype, B=B, seed=11)
    inp = synth.make_prefill(wl)
    N = wl.N
    print(f"[case] batched B={B} N={N} dtype={dtype}", flush=True)
    gpu = run_prefill(inp.q, inp.k, wl.topk, dtype)
    for b in range(B):
        ref_pyr = oracle.build_pyramid(inp.k[b])
        check_pyramid(gpu.pyramid[b:b + 1], ref_pyr, N, gpu.cap)
        ts = sample_positions(N, 500, wl.topk)
        rep = compare_selection(gpu.idx[b, ts], ts, inp.q[b], inp.k[b], ref_pyr, wl.topk)
        _log(f"prefill_batched_B{B}_{dtype}_b{b}", rep, {"positions": int(len(ts)), "all_positions": False})
        assert rep.ok(), (b, str(rep))


@pytest.mark.parametrize("B,K,steps", [(2, 16, 12), (20, 32, 4), (40, 8, 3)])
def test_decode_batched(B, K, steps):
    """Decode of a batch: per batch element, the refreshed pyramid equals a rebuild bitwise and
    the selection matches the oracle (near-ties validated). B=20 with K=32 and B=40 with K=8
    run one workgroup per sequence and KV head instead of the split over several."""
    from block_selection_amd import ops
    N0 = 2000
    wl = synth.Workload(f"decode_b{B}", N=N0, Hq=16, Hkv=2, topk=K, dtype="bf16", B=B, decode_steps=steps, seed=5)
    inp = synth.make_decode(wl)
    cap = N0 + steps
    dims = ops.make_dims(B, 16, 2, K, "bf16")
    kc_host = np.zeros((B, cap, 2, 64), np.float32)
    kc_host[:, :N0] = inp.k_ctx
    k_cache = to_device(kc_host, "bf16")
    pyr = ops.alloc_pyramid(dims, cap)
    ops.build_pyramid(k_cache, N0, cap, dims, pyr)
    k_new, q_new = to_device(inp.k_new, "bf16"), to_device(inp.q_new, "bf16")
    out = torch.full((B, 2, K), -7, dtype=torch.int32, device="cuda")
    ws = ops.alloc_workspace(dims, 1, cap, is_decode=True)
    pyr_rb = ops.alloc_pyramid(dims, cap)
    k_all = np.concatenate([inp.k_ctx, np.transpose(inp.k_new, (1, 0, 2, 3))], axis=1)   # [B, cap, Hkv, d]
    ref_k = to_device(k_all, "bf16")
    for s in range(steps):
        n = N0 + s
        print(f"[case] decode B={B} K={K} step={s}", flush=True)
        ops.decode_update_select(q_new[s].contiguous(), k_new[s].contiguous(), k_cache, pyr, n, cap, dims, out, ws)
        torch.cuda.synchronize()
        ops.build_pyramid(ref_k, n + 1, cap, dims, pyr_rb)
        a, r = pyr.cpu().numpy(), pyr_rb.cpu().numpy()
        got = out.cpu().numpy()
        for b in range(B):
            for j in range(2):
                for la, lb in zip(pyramid_levels(a[b, j], n + 1, cap), pyramid_levels(r[b, j], n + 1, cap)):
                    assert np.array_equal(la.view(np.uint32), lb.view(np.uint32)), (s, b, j)
            ref_pyr, o_idx, o_gap, o_lvl = oracle.decode_step(k_all[b], n, inp.q_new[s, b], K, with_level=True)
            step = compare_selection(got[b][None], np.array([n]), _RowView(inp.q_new[s, b], n), k_all[b, : n + 1],
                                     ref_pyr, K, ora=(o_idx[None], o_gap[None], o_lvl[None]))
            assert step.ok(), (s, b, str(step))
