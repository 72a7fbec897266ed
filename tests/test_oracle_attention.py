"""Pins of the oracle's stage-two attention over the selected blocks.

Stage two (reading note "Block Sparse Attention with Log-Linear Complexity", the
two-stage formulation it opens with) is attention limited to the raw key/value rows
of the blocks stage one picked. The oracle's reading: per query head, softmax of
q.k/sqrt(d) over the keys <= t of the blocks its KV head selected, applied to their
values. Pins:
  * every eligible block selected: dense causal attention (torch's
    scaled_dot_product_attention on the CPU in float64, a library routine);
  * value rows all equal to c inside the selected keys: output c (a convex
    combination);
  * zero query: the plain mean of the selected values up to t;
  * keys and values after t, and outside the selected blocks, do not matter;
  * the order of the indices and -1 padding do not matter;
  * GQA: query head h reads KV head h // (Hq/Hkv) and that head's selection.
"""
import numpy as np
import pytest
import torch

import oracle
from block_selection_amd import synth


def _qkv(N, Hq, Hkv, seed, d=64):
    rng = np.random.default_rng(seed)
    q = synth.bf16_round(rng.standard_normal((N, Hq, d), dtype=np.float32))
    k = synth.bf16_round(rng.standard_normal((N, Hkv, d), dtype=np.float32))
    v = synth.bf16_round(rng.standard_normal((N, Hkv, d), dtype=np.float32))
    return q, k, v


@pytest.mark.parametrize("N,Hq,Hkv", [(300, 4, 2), (640, 6, 3), (129, 2, 1)])
def test_all_blocks_is_dense_causal_attention(N, Hq, Hkv):
    q, k, v = _qkv(N, Hq, Hkv, N)
    nb = -(-N // 64)
    ts = np.arange(N)
    idx = np.full((N, Hkv, nb), -1, np.int32)
    for t in ts:
        idx[t, :, : t // 64 + 1] = np.arange(t // 64 + 1)
    got = oracle.attention(q, ts, k, v, idx)
    GQ = Hq // Hkv
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)               # [Hq, N, d]
    kt = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2).repeat_interleave(GQ, 0)
    vt = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2).repeat_interleave(GQ, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    np.testing.assert_allclose(got, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_constant_values_give_the_constant():
    N, Hq, Hkv = 512, 4, 2
    q, k, v = _qkv(N, Hq, Hkv, 2)
    c = np.random.default_rng(3).standard_normal((Hkv, 64)).astype(np.float32)
    v[128:192] = c                     # block 2 only
    ts = np.array([130, 191, 300, 511])
    idx = np.full((4, Hkv, 3), -1, np.int32)
    idx[:, :, 0] = 2
    got = oracle.attention(q[ts], ts, k, v, idx)
    for h in range(Hq):
        np.testing.assert_allclose(got[:, h], np.broadcast_to(c[h // 2], (4, 64)), rtol=0, atol=1e-12)


def test_zero_query_is_the_mean_of_the_selected_values():
    N, Hq, Hkv = 700, 2, 1
    q, k, v = _qkv(N, Hq, Hkv, 4)
    q[:] = 0
    ts = np.array([5, 64, 200, 699])
    idx = np.array([[[0, -1, -1]], [[0, 1, -1]], [[3, 0, -1]], [[10, 2, 7]]], np.int32)
    got = oracle.attention(q[ts], ts, k, v, idx)
    for i, t in enumerate(ts):
        rows = sorted(r for b in idx[i, 0] if b >= 0 for r in range(64 * b, min(64 * b + 64, N)) if r <= t)
        ref = v[rows, 0].astype(np.float64).mean(axis=0)
        for h in range(Hq):
            np.testing.assert_allclose(got[i, h], ref, rtol=0, atol=1e-12)


def test_keys_after_t_and_unselected_blocks_do_not_matter():
    N, Hq, Hkv = 640, 4, 2
    q, k, v = _qkv(N, Hq, Hkv, 5)
    ts = np.array([70, 333, 639])
    idx = np.array([[[0, 1, -1]] * 2, [[1, 5, 3]] * 2, [[9, 0, 4]] * 2], np.int32)
    a = oracle.attention(q[ts], ts, k, v, idx)
    k2, v2 = k.copy(), v.copy()
    k2[71:128], v2[71:128] = 9.0, -9.0               # after t = 70, inside its block 1
    b_ = oracle.attention(q[ts[:1]], ts[:1], k2, v2, idx[:1])
    np.testing.assert_array_equal(a[:1], b_)
    k3, v3 = k.copy(), v.copy()
    for b in (2, 6, 7, 8):                            # selected by no row
        k3[64 * b:64 * b + 64], v3[64 * b:64 * b + 64] = 5.0, 5.0
    np.testing.assert_array_equal(a, oracle.attention(q[ts], ts, k3, v3, idx))


def test_index_order_and_padding_do_not_matter():
    N, Hq, Hkv = 600, 4, 2
    q, k, v = _qkv(N, Hq, Hkv, 6)
    ts = np.array([599, 400])
    idx = np.array([[[1, 4, 8], [0, 2, 9]], [[6, 3, 0], [5, 1, 2]]], np.int32)
    perm = idx[:, :, ::-1].copy()
    pad = np.concatenate([np.full((2, 2, 2), -1, np.int32), idx], axis=2)
    a = oracle.attention(q[ts], ts, k, v, idx)
    np.testing.assert_allclose(oracle.attention(q[ts], ts, k, v, perm), a, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(oracle.attention(q[ts], ts, k, v, pad), a, rtol=1e-13, atol=1e-13)


def test_group_heads_use_their_kv_head_and_its_selection():
    """Two KV heads with different selections: each query head matches a one-head call."""
    N, Hq, Hkv = 512, 6, 2
    q, k, v = _qkv(N, Hq, Hkv, 7)
    ts = np.array([450])
    idx = np.array([[[0, 3], [5, 7]]], np.int32)
    got = oracle.attention(q[ts], ts, k, v, idx)
    for h in range(Hq):
        j = h // 3
        one = oracle.attention(q[ts][:, h:h + 1], ts, k[:, j:j + 1], v[:, j:j + 1], idx[:, j:j + 1])
        np.testing.assert_array_equal(got[:, h], one[:, 0])
