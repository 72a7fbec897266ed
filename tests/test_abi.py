"""C ABI checks that need no GPU: the library loads, exports every function
include/pisa.h declares, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "pisa.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(pisa_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    from block_selection_amd import ops
    names = _declared()
    assert set(names) == set(ops.EXPORTED)
    for n in names:
        assert hasattr(ops.lib, n), n


def test_geometry_helpers():
    from block_selection_amd import ops
    d = ops.make_dims(1, 32, 2, 8)
    assert ops.pyramid_nodes(d, 262144) == 8191
    assert ops.level_offset(d, 262144, 1) == 0
    assert ops.level_offset(d, 262144, 2) == 4096
    assert ops.level_offset(d, 262144, 13) == 8190
    assert ops.level_offset(d, 262144, 14) == -1
    assert ops.pyramid_bytes(d, 262144) == 2 * 8191 * 64 * 4
    assert ops.pyramid_nodes(d, 1) == 1
    assert ops.workspace_bytes(d, 4096) > 0
    # bf16 decode: 8-byte tagged counters per (batch, KV head), 256-byte aligned, then 64 leaf scores each
    assert ops.workspace_bytes(d, 1, 131328, is_decode=True) == 256 + 2 * 64 * 4
    assert ops.workspace_bytes(ops.make_dims(40, 32, 2, 8), 1, 4096, is_decode=True) == 768 + 80 * 64 * 4
    assert ops.workspace_bytes(d, 5000, 4000) == 0


def _call_select(ops, dims, N=64, cap=64, ws=8, ws_bytes=1 << 30, ptr=8):
    p = ctypes.c_void_p(ptr)
    return ops.lib.pisa_select_prefill(p, p, p, N, cap, ctypes.byref(dims), p,
                                       ctypes.c_void_p(ws) if ws else None, ws_bytes, None)


def test_argument_errors_return_before_launch():
    from block_selection_amd import ops
    good = ops.make_dims(1, 32, 2, 8)
    assert _call_select(ops, ops.make_dims(1, 32, 2, 8, d=32)) == ops.PISA_ERR_UNSUPPORTED
    assert _call_select(ops, ops.make_dims(1, 32, 2, 8, C=32)) == ops.PISA_ERR_UNSUPPORTED
    assert _call_select(ops, ops.make_dims(1, 32, 2, 8, g=4)) == ops.PISA_ERR_UNSUPPORTED
    assert _call_select(ops, ops.make_dims(1, 34, 1, 8)) == ops.PISA_ERR_UNSUPPORTED   # group of 34
    assert _call_select(ops, ops.make_dims(1, 32, 2, 33)) == ops.PISA_ERR_UNSUPPORTED
    assert _call_select(ops, ops.make_dims(32768, 32, 2, 8)) == ops.PISA_ERR_UNSUPPORTED   # B * Hkv > 65535
    assert _call_select(ops, ops.make_dims(1, 31, 2, 8)) == ops.PISA_ERR_INVALID_ARG
    assert _call_select(ops, ops.make_dims(1, 32, 2, 0)) == ops.PISA_ERR_INVALID_ARG
    assert _call_select(ops, ops.make_dims(0, 32, 2, 8)) == ops.PISA_ERR_INVALID_ARG
    bad_score = ops.make_dims(1, 32, 2, 8)
    bad_score.score = 3                                   # not a pisa_score
    assert _call_select(ops, bad_score) == ops.PISA_ERR_INVALID_ARG
    for sc in ("lse", "mean", "mean_half_var"):           # every score passes the dims checks
        assert _call_select(ops, ops.make_dims(1, 32, 2, 8, score=sc), ws_bytes=16) == ops.PISA_ERR_WORKSPACE
    assert _call_select(ops, good, N=65, cap=64) == ops.PISA_ERR_CAPACITY
    assert _call_select(ops, good, N=0) == ops.PISA_ERR_INVALID_ARG
    assert _call_select(ops, good, ws=0) == ops.PISA_ERR_WORKSPACE
    assert _call_select(ops, good, ws_bytes=16) == ops.PISA_ERR_WORKSPACE
    assert _call_select(ops, good, ptr=0) == ops.PISA_ERR_INVALID_ARG
    p = ctypes.c_void_p(8)
    assert ops.lib.pisa_build_pyramid(None, 64, 64, ctypes.byref(good), p, None) == ops.PISA_ERR_INVALID_ARG
    assert ops.lib.pisa_decode_update_select(p, p, p, p, 0, 64, ctypes.byref(good), p, p, 1 << 30,
                                             None) == ops.PISA_ERR_INVALID_ARG
    assert ops.lib.pisa_decode_update_select(p, p, p, p, 64, 64, ctypes.byref(good), p, p, 1 << 30,
                                             None) == ops.PISA_ERR_CAPACITY
    assert ops.status_string(ops.PISA_ERR_WORKSPACE) == "workspace too small"


def test_noalloc_decode_argument_errors_return_before_launch():
    """The decoding step without allocation rejects, before touching the GPU, batches beyond
    its static scratch (B * Hkv > 4096), fp32 inputs, bad pointers and bad lengths."""
    from block_selection_amd import ops
    p = ctypes.c_void_p(8)

    def step(dims, n_before=64, cap=128, ptr=p):
        return ops.lib.pisa_decode_update_select_noalloc(ptr, p, p, p, n_before, cap, ctypes.byref(dims), p, None)
    assert step(ops.make_dims(2049, 32, 2, 8)) == ops.PISA_ERR_WORKSPACE       # 4098 pairs
    assert step(ops.make_dims(1, 32, 2, 8, dtype="f32")) == ops.PISA_ERR_UNSUPPORTED
    assert step(ops.make_dims(1, 32, 2, 8), ptr=None) == ops.PISA_ERR_INVALID_ARG
    assert step(ops.make_dims(1, 32, 2, 8), n_before=0) == ops.PISA_ERR_INVALID_ARG
    assert step(ops.make_dims(1, 32, 2, 8), n_before=128) == ops.PISA_ERR_CAPACITY
    assert step(ops.make_dims(1, 32, 2, 33)) == ops.PISA_ERR_UNSUPPORTED


def test_bf16_prefill_limits_are_the_32_bit_entry_numbering():
    """bf16 selection numbers the leaf stage's entries in 32 bits: it needs walks * 2K < 2^32
    (B * N * Hkv walks); past it the call returns UNSUPPORTED before any launch and the
    workspace query returns 0. The bucket pass's LDS histogram sets no limit of its own
    (more groups are counted slice by slice), and fp32 selection has no such limit."""
    from block_selection_amd import ops
    d = ops.make_dims(1, 32, 2, 8)
    old_limit = 16384 * 1024 // 2 + 1             # past the 16384-bin histogram of a single pass
    assert ops.workspace_bytes(d, old_limit) > 0
    assert _call_select(ops, d, N=old_limit, cap=old_limit, ws_bytes=16) == ops.PISA_ERR_WORKSPACE
    d8 = ops.make_dims(1, 32, 8, 32)              # Hkv = 8, K = 32: N * 8 * 64 reaches 2^32 at 2^23
    assert ops.workspace_bytes(d8, (1 << 23) - 1) > 0
    assert ops.workspace_bytes(d8, 1 << 23) == 0
    assert _call_select(ops, d8, N=(1 << 23) - 1, cap=(1 << 23) - 1, ws_bytes=16) == ops.PISA_ERR_WORKSPACE
    assert _call_select(ops, d8, N=1 << 23, cap=1 << 23) == ops.PISA_ERR_UNSUPPORTED
    f32 = ops.make_dims(1, 32, 8, 32, dtype="f32")
    assert ops.workspace_bytes(f32, 1 << 23) > 0


def test_pack_geometry_helpers():
    """Packed layout: level l has (T >> (5 + l)) + D + 1 rows per KV head, levels 1 .. L(T)."""
    from block_selection_amd import ops
    d = ops.make_dims(1, 32, 2, 8)
    for T, D in [(262144, 1), (262144, 64), (16384, 7), (1, 1), (100, 5)]:
        L = 1
        m = -(-T // 64)
        while m > 1:
            m, L = -(-m // 2), L + 1
        off = 0
        for l in range(1, L + 1):
            assert ops.pack_level_offset(d, T, D, l) == off
            off += (T >> (5 + l)) + D + 1
        assert ops.pack_level_offset(d, T, D, L + 1) == -1
        assert ops.pack_pyramid_rows(d, T, D) == off
        assert ops.lib.pisa_pack_pyramid_bytes(ctypes.byref(d), T, D) == 2 * off * 64 * 4
        assert ops.pack_workspace_bytes(d, T, D) > 0
    assert ops.pack_pyramid_rows(d, 0, 1) == -1
    assert ops.pack_pyramid_rows(d, 64, 0) == -1
    assert ops.pack_pyramid_rows(ops.make_dims(2, 32, 2, 8), 64, 1) == -1   # packs have B = 1


def test_pack_argument_errors_return_before_launch():
    from block_selection_amd import ops
    p = ctypes.c_void_p(8)
    good = ops.make_dims(1, 32, 2, 8)

    def sel(dims, cu=p, D=3, T=4096, ws_bytes=1 << 34):
        return ops.lib.pisa_select_prefill_packed(p, p, p, cu, D, T, ctypes.byref(dims), p, p, ws_bytes, None)

    assert sel(good, cu=None) == ops.PISA_ERR_INVALID_ARG
    assert sel(good, D=0) == ops.PISA_ERR_INVALID_ARG
    assert sel(good, T=0) == ops.PISA_ERR_INVALID_ARG
    assert sel(ops.make_dims(2, 32, 2, 8)) == ops.PISA_ERR_INVALID_ARG
    assert sel(ops.make_dims(1, 32, 2, 8, dtype="f32")) == ops.PISA_ERR_UNSUPPORTED
    assert sel(ops.make_dims(1, 32, 2, 8, d=32)) == ops.PISA_ERR_UNSUPPORTED
    assert sel(good, T=1 << 24, ws_bytes=16) == ops.PISA_ERR_WORKSPACE   # within the limits
    assert sel(good, T=1 << 27) == ops.PISA_ERR_UNSUPPORTED   # T * Hkv * 2K entries reach 2^32
    assert sel(good, ws_bytes=16) == ops.PISA_ERR_WORKSPACE
    assert ops.lib.pisa_build_pyramid_packed(p, None, 3, 4096, ctypes.byref(good), p, None) == ops.PISA_ERR_INVALID_ARG
    assert ops.lib.pisa_build_pyramid_packed(None, p, 3, 4096, ctypes.byref(good), p, None) == ops.PISA_ERR_INVALID_ARG


def test_attention_argument_errors_return_before_launch():
    from block_selection_amd import ops
    p = ctypes.c_void_p(8)
    good = ops.make_dims(1, 32, 2, 8)

    def att(dims, N=4096, cap=4096, ws_bytes=1 << 34, ptr=p):
        return ops.lib.pisa_sparse_attention(ptr, p, p, p, N, cap, ctypes.byref(dims), p, p, ws_bytes, None)

    assert ops.attention_workspace_bytes(good, 4096) == 2 * 64 * 64 * 64 * 2
    assert ops.attention_workspace_bytes(good, 4097, 4096) == 0
    assert att(good, ptr=None) == ops.PISA_ERR_INVALID_ARG
    assert att(good, N=0) == ops.PISA_ERR_INVALID_ARG
    assert att(good, N=5000) == ops.PISA_ERR_CAPACITY
    assert att(ops.make_dims(1, 32, 2, 8, dtype="f32")) == ops.PISA_ERR_UNSUPPORTED
    assert att(ops.make_dims(1, 32, 2, 8, d=128)) == ops.PISA_ERR_UNSUPPORTED
    assert att(good, ws_bytes=16) == ops.PISA_ERR_WORKSPACE


def test_packed_attention_argument_errors_return_before_launch():
    from block_selection_amd import ops
    p = ctypes.c_void_p(8)
    good = ops.make_dims(1, 32, 2, 8)

    def att(dims, cu=p, D=3, T=4096, ws_bytes=1 << 34):
        return ops.lib.pisa_sparse_attention_packed(p, p, p, p, cu, D, T, ctypes.byref(dims), p, p, ws_bytes, None)

    assert ops.pack_attention_workspace_bytes(good, 4096, 3) == 2 * ((4096 >> 6) + 4) * 64 * 64 * 2
    assert att(good, cu=None) == ops.PISA_ERR_INVALID_ARG
    assert att(good, D=0) == ops.PISA_ERR_INVALID_ARG
    assert att(ops.make_dims(2, 32, 2, 8)) == ops.PISA_ERR_INVALID_ARG
    assert att(ops.make_dims(1, 32, 2, 8, dtype="f32")) == ops.PISA_ERR_UNSUPPORTED
    assert att(good, ws_bytes=16) == ops.PISA_ERR_WORKSPACE


def test_decode_attention_argument_errors_return_before_launch():
    from block_selection_amd import ops
    p = ctypes.c_void_p(8)
    good = ops.make_dims(1, 32, 2, 32)

    def att(dims, t=100, cap=4096, ptr=p, ws_bytes=1 << 20):
        return ops.lib.pisa_decode_attention(ptr, None, p, p, p, t, cap, ctypes.byref(dims), p, p, ws_bytes, None)

    # counters (256-byte aligned), then 8 partial states of (16 + 16 + 16 * 64) floats per KV head
    assert ops.decode_attention_workspace_bytes(good) == 256 + (2 * 8 * (32 + 1024) * 4 + 255) // 256 * 256
    assert att(good, ptr=None) == ops.PISA_ERR_INVALID_ARG
    assert att(good, t=-1) == ops.PISA_ERR_INVALID_ARG
    assert att(good, t=4096) == ops.PISA_ERR_CAPACITY
    assert att(ops.make_dims(1, 32, 2, 32, dtype="f32")) == ops.PISA_ERR_UNSUPPORTED
    assert att(good, ws_bytes=16) == ops.PISA_ERR_WORKSPACE


def test_flat_exact_argument_errors_return_before_launch():
    from block_selection_amd import ops
    p = ctypes.c_void_p(8)
    good = ops.make_dims(1, 32, 2, 8)

    def sel(dims, N=4096, cap=4096, ptr=p, ws_bytes=None):
        if ws_bytes is None:
            ws_bytes = ops.flat_exact_workspace_bytes(dims, N, cap)
        return ops.lib.pisa_select_flat_exact(ptr, p, N, cap, ctypes.byref(dims), p, p, ws_bytes, None)

    # one fp32 score per (batch, KV head, position, leaf), rounded up to 256 bytes
    assert ops.flat_exact_workspace_bytes(good, 4096) == 2 * 4096 * 64 * 4
    assert ops.flat_exact_workspace_bytes(ops.make_dims(3, 8, 1, 4), 1000, 2000) == \
        (3 * 1000 * 16 * 4 + 255) // 256 * 256
    assert ops.flat_exact_workspace_bytes(good, 0) == 0
    assert ops.flat_exact_workspace_bytes(good, 10, 5) == 0
    assert sel(good, ptr=None, ws_bytes=1 << 30) == ops.PISA_ERR_INVALID_ARG
    assert sel(good, N=0, ws_bytes=1 << 30) == ops.PISA_ERR_INVALID_ARG
    assert sel(good, N=5000, cap=4096, ws_bytes=1 << 30) == ops.PISA_ERR_CAPACITY
    assert sel(ops.make_dims(1, 32, 2, 8, dtype="f32"), ws_bytes=1 << 30) == ops.PISA_ERR_UNSUPPORTED
    assert sel(ops.make_dims(1, 32, 2, 8, score="mean"), ws_bytes=1 << 30) == ops.PISA_ERR_UNSUPPORTED
    assert sel(ops.make_dims(1, 32, 2, 40), ws_bytes=1 << 30) == ops.PISA_ERR_UNSUPPORTED   # K > 32
    assert sel(good, ws_bytes=ops.flat_exact_workspace_bytes(good, 4096) - 4) == ops.PISA_ERR_WORKSPACE
    assert ops.lib.pisa_select_flat_exact(p, p, 4096, 4096, ctypes.byref(good), p, None, 1 << 30,
                                          None) == ops.PISA_ERR_WORKSPACE
