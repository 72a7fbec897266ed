"""The decoding step without allocation (pisa_decode_update_select_noalloc, for callers that
cannot allocate) against the workspace entry point (pisa_decode_update_select) through the
C ABI: on identical copies of the key cache and pyramid, every step's selection and refreshed
pyramid must be bitwise equal. Consecutive calls share the library's static scratch, so the
cases run in a row from large to small: a batch that takes the one-workgroup form, then
smaller batches that take the split form (completion counters handed over between
workgroups), then a single sequence.
"""
import numpy as np
import pytest
import torch

from block_selection_amd import synth
from pisa_testlib import pyramid_levels, to_device

pytestmark = pytest.mark.gpu


def _run(B, K, steps, N0=3000, Hq=16, Hkv=2, seed=7):
    from block_selection_amd import ops
    wl = synth.Workload(f"noalloc_b{B}", N=N0, Hq=Hq, Hkv=Hkv, topk=K, dtype="bf16", B=B, decode_steps=steps,
                        seed=seed)
    inp = synth.make_decode(wl)
    cap = N0 + steps
    dims = ops.make_dims(B, Hq, Hkv, K, "bf16")
    kc_host = np.zeros((B, cap, Hkv, 64), np.float32)
    kc_host[:, :N0] = inp.k_ctx
    kc_a, kc_b = to_device(kc_host, "bf16"), to_device(kc_host, "bf16")
    pyr_a, pyr_b = ops.alloc_pyramid(dims, cap), ops.alloc_pyramid(dims, cap)
    ops.build_pyramid(kc_a, N0, cap, dims, pyr_a)
    ops.build_pyramid(kc_b, N0, cap, dims, pyr_b)
    k_new, q_new = to_device(inp.k_new, "bf16"), to_device(inp.q_new, "bf16")
    out_a = torch.full((B, Hkv, K), -7, dtype=torch.int32, device="cuda")
    out_b = torch.full((B, Hkv, K), -9, dtype=torch.int32, device="cuda")
    ws = ops.alloc_workspace(dims, 1, cap, is_decode=True)
    for s in range(steps):
        n = N0 + s
        print(f"[case] noalloc B={B} K={K} step={s}", flush=True)
        ops.decode_update_select(q_new[s].contiguous(), k_new[s].contiguous(), kc_a, pyr_a, n, cap, dims, out_a, ws)
        ops.decode_update_select_noalloc(q_new[s].contiguous(), k_new[s].contiguous(), kc_b, pyr_b, n, cap, dims,
                                         out_b)
        torch.cuda.synchronize()
        a, b = out_a.cpu().numpy(), out_b.cpu().numpy()
        assert np.array_equal(a, b), (B, K, s)
        assert (a >= -1).all() and (a[..., 0] >= 0).all()
        pa, pb = pyr_a.cpu().numpy(), pyr_b.cpu().numpy()
        for bb in range(B):
            for j in range(Hkv):
                for la, lb in zip(pyramid_levels(pa[bb, j], n + 1, cap), pyramid_levels(pb[bb, j], n + 1, cap)):
                    assert np.array_equal(la.view(np.uint32), lb.view(np.uint32)), (B, s, bb, j)
    assert torch.equal(kc_a, kc_b)


def test_noalloc_matches_workspace_entry_point_large_then_small():
    _run(B=40, K=16, steps=3)     # 80 (batch, KV head) pairs: one workgroup each
    _run(B=3, K=32, steps=4)      # split form: 4 workgroups per pair, counters handed over
    _run(B=1, K=8, steps=5)       # one sequence, 2 workgroups per pair
