"""GPU parity of attention over the selected blocks (stage two) against the oracle.

The oracle's attention takes the oracle's own selection; the GPU kernel is given the
same index array (or its own selection, compared on the walks where the two
selections agree). Tolerance: every output element within 1e-4 * max|v| of the fp64
oracle -- the kernel's errors are fp32 accumulation of exact bf16 products (about
1e-6 relative on a logit), the hardware exp2 (about 1 ulp) and the bf16 hi + lo
split of the probabilities (2^-17), which together stay below 4e-5 of the largest
value magnitude.
"""
import numpy as np
import pytest
import torch

import oracle
from block_selection_amd import synth
from pisa_testlib import run_prefill, to_device

pytestmark = pytest.mark.gpu

ATTN_TOL = 1e-4


def _run_attention(q, k, v, idx, topk, cap=None):
    """q [N, Hq, d], k/v [N, Hkv, d], idx [N, Hkv, K] (B = 1)."""
    from block_selection_amd import ops
    N, Hq, d = q.shape
    Hkv = k.shape[1]
    cap = N if cap is None else cap
    print(f"attention N={N} cap={cap} Hq={Hq} Hkv={Hkv} K={topk}", flush=True)
    dims = ops.make_dims(1, Hq, Hkv, topk, "bf16")
    kk = np.zeros((cap, Hkv, d), np.float32)
    vv = np.zeros((cap, Hkv, d), np.float32)
    kk[:N], vv[:N] = k, v
    kk[N:], vv[N:] = 3.0, -3.0            # rows past N must not matter
    qt, kt, vt = to_device(q[None], "bf16"), to_device(kk[None], "bf16"), to_device(vv[None], "bf16")
    it = torch.from_numpy(np.ascontiguousarray(idx[None], np.int32)).cuda()
    out = torch.full((1, N, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    ws = ops.alloc_attention_workspace(dims, N, cap)
    ops.sparse_attention(qt, kt, vt, it, N, cap, dims, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()[0]


def _check(got, ref, v, rows=None):
    scale = float(np.abs(v).max())
    err = np.abs(got.astype(np.float64) - ref)
    assert np.all(np.isfinite(got))
    worst = float(err.max()) / scale
    print(f"attention max |err| / max|v| = {worst:.3e}", flush=True)
    assert worst <= ATTN_TOL, worst
    return worst


def _inputs(N, Hq, Hkv, seed):
    rng = np.random.default_rng(seed)
    q = synth.bf16_round(rng.standard_normal((N, Hq, 64), dtype=np.float32))
    k = synth.bf16_round(rng.standard_normal((N, Hkv, 64), dtype=np.float32))
    v = synth.make_values(1, N, Hkv, seed=seed)[0]
    return q, k, v


@pytest.mark.parametrize("N,Hq,Hkv,K", [(1000, 32, 2, 8), (4096, 32, 2, 8), (130, 4, 1, 4), (3000, 12, 3, 5),
                                         (2000, 8, 8, 32), (5000, 16, 1, 16), (64, 32, 2, 8), (1, 2, 1, 1)])
def test_attention_on_the_oracle_selection(N, Hq, Hkv, K):
    q, k, v = _inputs(N, Hq, Hkv, N + K)
    pyr = oracle.build_pyramid(k)
    ts = np.arange(N)
    idx, _, _ = oracle.walk(q, ts, k, pyr, K)
    got = _run_attention(q, k, v, idx, K)
    ref = oracle.attention(q, ts, k, v, idx)
    _check(got, ref, v)


def test_attention_skips_invalid_indices():
    """Entries < 0, past t's block or past the last block add nothing (as in the oracle)."""
    N, Hq, Hkv, K = 900, 8, 2, 6
    q, k, v = _inputs(N, Hq, Hkv, 3)
    rng = np.random.default_rng(4)
    idx = rng.integers(-3, 20, (N, Hkv, K)).astype(np.int32)
    idx[:, :, 0] = 0                                     # every row keeps one visible block
    idx[5, 1, 3] = 1 << 30
    for row in range(N):                                 # distinct entries per row
        for j in range(Hkv):
            seen = set()
            for i in range(K):
                if idx[row, j, i] in seen:
                    idx[row, j, i] = -1
                seen.add(int(idx[row, j, i]))
    got = _run_attention(q, k, v, idx, K)
    ref = oracle.attention(q, np.arange(N), k, v, idx)
    _check(got, ref, v)


def test_attention_capacity_layout():
    N, cap, Hq, Hkv, K = 1500, 2048, 32, 2, 8
    q, k, v = _inputs(N, Hq, Hkv, 5)
    idx, _, _ = oracle.walk(q, np.arange(N), k, oracle.build_pyramid(k), K)
    got = _run_attention(q, k, v, idx, K, cap=cap)
    _check(got, oracle.attention(q, np.arange(N), k, v, idx), v)


def _end_to_end(wl_name, n_rows, seed=0):
    from block_selection_amd import ops
    wl = synth.WORKLOADS[wl_name]
    inp = synth.make_prefill(wl)
    q, k = inp.q[0], inp.k[0]
    N = q.shape[0]
    v = synth.make_values(1, N, wl.Hkv, seed=wl.seed)[0]
    sel = run_prefill(inp.q, inp.k, wl.topk, wl.dtype)
    got = _run_attention(q, k, v, sel.idx[0], wl.topk)
    rng = np.random.default_rng(seed)
    ts = np.arange(N) if n_rows is None else np.unique(np.concatenate(
        [[0, 63, 64, N - 1], rng.choice(N, n_rows, replace=False)])).astype(np.int64)
    o_idx, _, _ = oracle.walk(q[ts], ts, k, oracle.build_pyramid(k), wl.topk)
    same = np.all(o_idx == sel.idx[0][ts], axis=(1, 2))
    ref = oracle.attention(q[ts], ts, k, v, o_idx)
    print(f"{wl_name}: {int(same.sum())} of {len(ts)} rows with identical selections compared", flush=True)
    assert same.mean() > 0.95
    return _check(got[ts][same], ref[same], v)


def test_attention_after_gpu_selection_short():
    """Selection and attention both on the GPU (4096 positions), all rows."""
    _end_to_end("short", None)


def test_attention_after_gpu_selection_long256k():
    """The full 262144-position workload: sampled rows against the oracle."""
    _end_to_end("long256k", 400)


def test_decode_attention_on_the_oracle_selection():
    """One decoding query per (batch, KV head): positions across block boundaries, K = 32,
    the value row of the new token appended by the call."""
    from block_selection_amd import ops
    N, Hq, Hkv, K = 6000, 32, 2, 32
    q, k, v = _inputs(N, Hq, Hkv, 21)
    cap = N + 64
    dims = ops.make_dims(1, Hq, Hkv, K, "bf16")
    wsd = ops.alloc_decode_attention_workspace(dims)     # reused by every call (counters left zero)
    for t in (0, 63, 64, 2047, 4000, N - 1):
        pyr = oracle.build_pyramid(k[:t + 1])
        idx, _, _ = oracle.walk(q[t:t + 1], np.array([t]), k[:t + 1], pyr, K)
        kk = np.zeros((1, cap, Hkv, 64), np.float32)
        vv = np.zeros((1, cap, Hkv, 64), np.float32)
        kk[0, :t + 1], vv[0, :t] = k[:t + 1], v[:t]
        vv[0, t + 1:] = 7.0                               # rows after t must not matter
        kt, vt = to_device(kk, "bf16"), to_device(vv, "bf16")
        out = torch.full((1, Hq, 64), float("nan"), dtype=torch.float32, device="cuda")
        print(f"decode attention t={t}", flush=True)
        ops.decode_attention(to_device(q[t][None], "bf16"), to_device(v[t][None], "bf16"), kt, vt,
                             torch.from_numpy(idx[0][None].copy()).cuda(), t, cap, dims, out, wsd)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(vt.float().cpu().numpy()[0, t], v[t])   # the appended row
        ref = oracle.attention(q[t:t + 1], np.array([t]), k[:t + 1], v[:t + 1], idx)
        _check(out.cpu().numpy(), ref, v)


def test_decode_steps_select_then_attend():
    """24 decoding steps over a 20000-key context: pisa_decode_update_select, then
    pisa_decode_attention on its selection, against the oracle's selection and attention."""
    from block_selection_amd import ops
    N0, steps, Hq, Hkv, K = 20000, 24, 32, 2, 32
    q, k, v = _inputs(N0 + steps, Hq, Hkv, 22)
    cap = N0 + steps
    dims = ops.make_dims(1, Hq, Hkv, K, "bf16")
    kk = np.zeros((1, cap, Hkv, 64), np.float32)
    vv = np.zeros((1, cap, Hkv, 64), np.float32)
    kk[0, :N0], vv[0, :N0] = k[:N0], v[:N0]
    kc, vc = to_device(kk, "bf16"), to_device(vv, "bf16")
    pyr = ops.alloc_pyramid(dims, cap)
    ops.build_pyramid(kc, N0, cap, dims, pyr)
    ws = ops.alloc_workspace(dims, 1, cap, is_decode=True)
    sel = torch.empty((1, Hkv, K), dtype=torch.int32, device="cuda")
    out = torch.empty((1, Hq, 64), dtype=torch.float32, device="cuda")
    wsd = ops.alloc_decode_attention_workspace(dims)
    compared = 0
    for s in range(steps):
        t = N0 + s
        qn, kn, vn = to_device(q[t][None], "bf16"), to_device(k[t][None], "bf16"), to_device(v[t][None], "bf16")
        ops.decode_update_select(qn, kn, kc, pyr, t, cap, dims, sel, ws)
        ops.decode_attention(qn, vn, kc, vc, sel, t, cap, dims, out, wsd)
        torch.cuda.synchronize()
        o_idx, _, _ = oracle.walk(q[t:t + 1], np.array([t]), k[:t + 1], oracle.build_pyramid(k[:t + 1]), K)
        if not np.array_equal(o_idx[0], sel.cpu().numpy()[0]):
            continue
        ref = oracle.attention(q[t:t + 1], np.array([t]), k[:t + 1], v[:t + 1], o_idx)
        _check(out.cpu().numpy(), ref, v)
        compared += 1
    print(f"decode select + attend: {compared} of {steps} steps compared", flush=True)
    assert compared >= steps - 2


def test_attention_batched():
    """B = 3 batch elements in one call, each against the oracle on its own selection."""
    from block_selection_amd import ops
    B, N, Hq, Hkv, K = 3, 1500, 16, 2, 8
    rng = np.random.default_rng(31)
    q = synth.bf16_round(rng.standard_normal((B, N, Hq, 64), dtype=np.float32))
    k = synth.bf16_round(rng.standard_normal((B, N, Hkv, 64), dtype=np.float32))
    v = synth.make_values(B, N, Hkv, seed=31)
    idx = np.stack([oracle.walk(q[b], np.arange(N), k[b], oracle.build_pyramid(k[b]), K)[0] for b in range(B)])
    dims = ops.make_dims(B, Hq, Hkv, K, "bf16")
    print(f"attention batched B={B} N={N}", flush=True)
    out = torch.full((B, N, Hq, 64), float("nan"), dtype=torch.float32, device="cuda")
    ops.sparse_attention(to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16"),
                         torch.from_numpy(np.ascontiguousarray(idx)).cuda(), N, N, dims, out,
                         ops.alloc_attention_workspace(dims, N))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(B):
        _check(got[b], oracle.attention(q[b], np.arange(N), k[b], v[b], idx[b]), v)


@pytest.mark.parametrize("B,K", [(2, 32), (20, 32), (40, 8)])
def test_decode_attention_batched(B, K):
    """B=20 with K=32 and B=40 with K=8 (2 KV heads) run one workgroup per (batch, KV head),
    each wavefront over several blocks; B=2 splits the blocks over workgroups."""
    from block_selection_amd import ops
    N, Hq, Hkv = 3000, 32, 2
    rng = np.random.default_rng(32)
    q = synth.bf16_round(rng.standard_normal((B, Hq, 64), dtype=np.float32))
    k = synth.bf16_round(rng.standard_normal((B, N, Hkv, 64), dtype=np.float32))
    v = synth.make_values(B, N, Hkv, seed=32)
    t = N - 1
    idx = np.stack([oracle.walk(q[b][None], np.array([t]), k[b], oracle.build_pyramid(k[b]), K)[0][0]
                    for b in range(B)])
    dims = ops.make_dims(B, Hq, Hkv, K, "bf16")
    out = torch.empty((B, Hq, 64), dtype=torch.float32, device="cuda")
    print(f"decode attention batched B={B} K={K} t={t}", flush=True)
    ops.decode_attention(to_device(q, "bf16"), None, to_device(k, "bf16"), to_device(v, "bf16"),
                         torch.from_numpy(np.ascontiguousarray(idx)).cuda(), t, N, dims, out,
                         ops.alloc_decode_attention_workspace(dims))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(B):
        _check(got[b][None], oracle.attention(q[b][None], np.array([t]), k[b], v[b], idx[b][None]), v)


def test_decode_attention_workspace_needs_no_zeroing():
    """Tagged completion counters: a decode-attention workspace full of stray bytes, or whose
    counters hold a foreign tag one arrival short of the last, gives bit for bit the output of
    a zero-filled one (K = 32: eight workgroups per (batch, KV head) meet at each counter)."""
    from block_selection_amd import ops
    B, N, Hq, Hkv, K = 2, 3000, 32, 2, 32
    rng = np.random.default_rng(33)
    q = synth.bf16_round(rng.standard_normal((B, Hq, 64), dtype=np.float32))
    k = synth.bf16_round(rng.standard_normal((B, N, Hkv, 64), dtype=np.float32))
    v = synth.make_values(B, N, Hkv, seed=33)
    t = N - 1
    idx = np.stack([oracle.walk(q[b][None], np.array([t]), k[b], oracle.build_pyramid(k[b]), K)[0][0]
                    for b in range(B)])
    dims = ops.make_dims(B, Hq, Hkv, K, "bf16")
    qd, kd, vd = to_device(q, "bf16"), to_device(k, "bf16"), to_device(v, "bf16")
    idxd = torch.from_numpy(np.ascontiguousarray(idx)).cuda()
    ws = ops.alloc_decode_attention_workspace(dims)
    gen = torch.Generator(device="cpu").manual_seed(4)
    outs = []
    for poison in (None, "bytes", "one_short", None):
        if poison == "bytes":
            ws.copy_(torch.randint(0, 256, (ws.numel(),), dtype=torch.uint8, generator=gen).cuda())
        elif poison == "one_short":
            words = torch.randint(1, 1 << 31, (B * Hkv,), dtype=torch.int64, generator=gen)
            ws[: 8 * B * Hkv].copy_(((words << 32) | 7).view(torch.uint8).cuda())
        out = torch.empty((B, Hq, 64), dtype=torch.float32, device="cuda")
        print(f"decode attention workspace poison={poison}", flush=True)
        ops.decode_attention(qd, None, kd, vd, idxd, t, N, dims, out, ws)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))
    got = outs[0]
    for b in range(B):
        _check(got[b][None], oracle.attention(q[b][None], np.array([t]), k[b], v[b], idx[b][None]), v)
