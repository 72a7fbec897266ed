"""Thin ctypes binding over libpisa.so (C ABI in include/pisa.h).

Argument marshalling only: every step of the selection runs in the HIP
kernels of libpisa.so. Tensors are PyTorch device tensors (ROCm), used for
their memory and streams; the calls enqueue on the current torch stream
unless a stream is given. If the library is missing this module raises at
import time: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpisa.so")

PISA_OK = 0
PISA_ERR_INVALID_ARG = -1
PISA_ERR_UNSUPPORTED = -2
PISA_ERR_WORKSPACE = -3
PISA_ERR_CAPACITY = -4
PISA_ERR_HIP = -5
PISA_DTYPE_F32 = 0
PISA_DTYPE_BF16 = 1

EXPORTED = ("pisa_pyramid_nodes", "pisa_level_offset", "pisa_pyramid_bytes", "pisa_workspace_bytes",
            "pisa_build_pyramid", "pisa_select_prefill", "pisa_select_prefill_profiled",
            "pisa_decode_update_select", "pisa_status_string", "pisa_pack_pyramid_rows",
            "pisa_pack_level_offset", "pisa_pack_pyramid_bytes", "pisa_pack_workspace_bytes",
            "pisa_build_pyramid_packed", "pisa_select_prefill_packed", "pisa_attention_workspace_bytes",
            "pisa_sparse_attention", "pisa_pack_attention_workspace_bytes", "pisa_sparse_attention_packed",
            "pisa_decode_attention", "pisa_decode_attention_workspace_bytes", "pisa_flat_workspace_bytes",
            "pisa_select_flat", "pisa_decode_update_select_noalloc", "pisa_flat_exact_workspace_bytes",
            "pisa_select_flat_exact")


class Dims(ctypes.Structure):
    """Mirror of pisa_dims."""
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("C", ctypes.c_int32), ("g", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("dtype", ctypes.c_int32), ("score", ctypes.c_int32)]

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == PISA_DTYPE_BF16 else torch.float32


class PisaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libpisa.so not built ({LIB_PATH}); run `python -m block_selection_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    D = ctypes.POINTER(Dims)
    lib.pisa_pyramid_nodes.argtypes = [D, i64]
    lib.pisa_pyramid_nodes.restype = i64
    lib.pisa_level_offset.argtypes = [D, i64, i32]
    lib.pisa_level_offset.restype = i64
    lib.pisa_pyramid_bytes.argtypes = [D, i64]
    lib.pisa_pyramid_bytes.restype = sz
    lib.pisa_workspace_bytes.argtypes = [D, i64, i64, i32]
    lib.pisa_workspace_bytes.restype = sz
    lib.pisa_build_pyramid.argtypes = [P, i64, i64, D, P, P]
    lib.pisa_build_pyramid.restype = ctypes.c_int
    lib.pisa_select_prefill.argtypes = [P, P, P, i64, i64, D, P, P, sz, P]
    lib.pisa_select_prefill.restype = ctypes.c_int
    lib.pisa_select_prefill_profiled.argtypes = [P, P, P, i64, i64, D, P, P, sz, P, P]
    lib.pisa_select_prefill_profiled.restype = ctypes.c_int
    lib.pisa_decode_update_select.argtypes = [P, P, P, P, i64, i64, D, P, P, sz, P]
    lib.pisa_decode_update_select.restype = ctypes.c_int
    lib.pisa_pack_pyramid_rows.argtypes = [D, i64, i64]
    lib.pisa_pack_pyramid_rows.restype = i64
    lib.pisa_pack_level_offset.argtypes = [D, i64, i64, i32]
    lib.pisa_pack_level_offset.restype = i64
    lib.pisa_pack_pyramid_bytes.argtypes = [D, i64, i64]
    lib.pisa_pack_pyramid_bytes.restype = sz
    lib.pisa_pack_workspace_bytes.argtypes = [D, i64, i64]
    lib.pisa_pack_workspace_bytes.restype = sz
    lib.pisa_build_pyramid_packed.argtypes = [P, P, i64, i64, D, P, P]
    lib.pisa_build_pyramid_packed.restype = ctypes.c_int
    lib.pisa_select_prefill_packed.argtypes = [P, P, P, P, i64, i64, D, P, P, sz, P]
    lib.pisa_select_prefill_packed.restype = ctypes.c_int
    lib.pisa_attention_workspace_bytes.argtypes = [D, i64, i64]
    lib.pisa_attention_workspace_bytes.restype = sz
    lib.pisa_sparse_attention.argtypes = [P, P, P, P, i64, i64, D, P, P, sz, P]
    lib.pisa_sparse_attention.restype = ctypes.c_int
    lib.pisa_pack_attention_workspace_bytes.argtypes = [D, i64, i64]
    lib.pisa_pack_attention_workspace_bytes.restype = sz
    lib.pisa_sparse_attention_packed.argtypes = [P, P, P, P, P, i64, i64, D, P, P, sz, P]
    lib.pisa_sparse_attention_packed.restype = ctypes.c_int
    lib.pisa_decode_attention_workspace_bytes.argtypes = [D]
    lib.pisa_decode_attention_workspace_bytes.restype = sz
    lib.pisa_decode_attention.argtypes = [P, P, P, P, P, i64, i64, D, P, P, sz, P]
    lib.pisa_decode_attention.restype = ctypes.c_int
    lib.pisa_flat_workspace_bytes.argtypes = [D, i64, i64]
    lib.pisa_flat_workspace_bytes.restype = sz
    lib.pisa_select_flat.argtypes = [P, P, i64, i64, D, P, P, sz, P]
    lib.pisa_select_flat.restype = ctypes.c_int
    lib.pisa_flat_exact_workspace_bytes.argtypes = [D, i64, i64]
    lib.pisa_flat_exact_workspace_bytes.restype = sz
    lib.pisa_select_flat_exact.argtypes = [P, P, i64, i64, D, P, P, sz, P]
    lib.pisa_select_flat_exact.restype = ctypes.c_int
    lib.pisa_decode_update_select_noalloc.argtypes = [P, P, P, P, i64, i64, D, P, P]
    lib.pisa_decode_update_select_noalloc.restype = ctypes.c_int
    lib.pisa_status_string.argtypes = [ctypes.c_int]
    lib.pisa_status_string.restype = ctypes.c_char_p
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.pisa_status_string(status).decode()


# candidate scores (pisa_score): the LogSumExp of the method and its two truncations
SCORES = {"lse": 0, "mean": 1, "mean_half_var": 2}


def make_dims(B: int, Hq: int, Hkv: int, topk: int, dtype: str = "bf16", d: int = 64, C: int = 64,
              g: int = 2, score: str = "lse") -> Dims:
    dt = {"bf16": PISA_DTYPE_BF16, "f32": PISA_DTYPE_F32}[dtype]
    return Dims(B, Hq, Hkv, d, C, g, topk, dt, SCORES[score])


def pyramid_nodes(dims: Dims, n_capacity: int) -> int:
    return int(lib.pisa_pyramid_nodes(ctypes.byref(dims), n_capacity))


def level_offset(dims: Dims, n_capacity: int, level: int) -> int:
    return int(lib.pisa_level_offset(ctypes.byref(dims), n_capacity, level))


def pyramid_bytes(dims: Dims, n_capacity: int) -> int:
    return int(lib.pisa_pyramid_bytes(ctypes.byref(dims), n_capacity))


def workspace_bytes(dims: Dims, N: int, n_capacity: Optional[int] = None, is_decode: bool = False) -> int:
    cap = N if n_capacity is None else n_capacity
    return int(lib.pisa_workspace_bytes(ctypes.byref(dims), N, cap, int(bool(is_decode))))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(t: torch.Tensor, name: str, dtype, numel: int):
    if not t.is_cuda or not t.is_contiguous() or t.dtype != dtype or t.numel() != numel:
        raise ValueError(f"{name}: expected a contiguous device tensor of {numel} {dtype}, got "
                         f"{tuple(t.shape)} {t.dtype} on {t.device}")


def alloc_pyramid(dims: Dims, n_capacity: int, device="cuda") -> torch.Tensor:
    return torch.empty((dims.B, dims.Hkv, pyramid_nodes(dims, n_capacity), dims.d),
                       dtype=torch.float32, device=device)


def alloc_workspace(dims: Dims, N: int, n_capacity: Optional[int] = None, is_decode: bool = False,
                    device="cuda") -> Optional[torch.Tensor]:
    n = workspace_bytes(dims, N, n_capacity, is_decode)
    # zero-filled, though nothing requires it: a decode workspace's completion counters are tagged per call
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def build_pyramid(k: torch.Tensor, N: int, n_capacity: int, dims: Dims, pyramid: torch.Tensor,
                  stream=None) -> None:
    _check(k, "k", dims.torch_dtype, dims.B * n_capacity * dims.Hkv * dims.d)
    _check(pyramid, "pyramid", torch.float32, dims.B * dims.Hkv * pyramid_nodes(dims, n_capacity) * dims.d)
    rc = lib.pisa_build_pyramid(_ptr(k), N, n_capacity, ctypes.byref(dims), _ptr(pyramid), _stream(stream))
    if rc != PISA_OK:
        raise PisaError("pisa_build_pyramid", rc)


def select_prefill(q: torch.Tensor, k: torch.Tensor, pyramid: torch.Tensor, N: int, n_capacity: int,
                   dims: Dims, out_idx: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                   stream=None) -> None:
    _check(q, "q", dims.torch_dtype, dims.B * N * dims.Hq * dims.d)
    _check(k, "k", dims.torch_dtype, dims.B * n_capacity * dims.Hkv * dims.d)
    _check(pyramid, "pyramid", torch.float32, dims.B * dims.Hkv * pyramid_nodes(dims, n_capacity) * dims.d)
    _check(out_idx, "out_idx", torch.int32, dims.B * N * dims.Hkv * dims.topk)
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.pisa_select_prefill(_ptr(q), _ptr(k), _ptr(pyramid), N, n_capacity, ctypes.byref(dims),
                                 _ptr(out_idx), _ptr(workspace), ws_n, _stream(stream))
    if rc != PISA_OK:
        raise PisaError("pisa_select_prefill", rc)


def select_prefill_profiled(q: torch.Tensor, k: torch.Tensor, pyramid: torch.Tensor, N: int, n_capacity: int,
                            dims: Dims, out_idx: torch.Tensor, workspace: Optional[torch.Tensor],
                            stage_events, stream=None) -> None:
    """pisa_select_prefill recording 4 caller-created hipEvent_t handles (ints or None) at stage
    boundaries: before/after the upper-level walk, before/after the leaf-scoring kernel."""
    _check(q, "q", dims.torch_dtype, dims.B * N * dims.Hq * dims.d)
    _check(k, "k", dims.torch_dtype, dims.B * n_capacity * dims.Hkv * dims.d)
    _check(pyramid, "pyramid", torch.float32, dims.B * dims.Hkv * pyramid_nodes(dims, n_capacity) * dims.d)
    _check(out_idx, "out_idx", torch.int32, dims.B * N * dims.Hkv * dims.topk)
    ev = (ctypes.c_void_p * 4)(*[ctypes.c_void_p(e) if e else None for e in stage_events])
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.pisa_select_prefill_profiled(_ptr(q), _ptr(k), _ptr(pyramid), N, n_capacity, ctypes.byref(dims),
                                          _ptr(out_idx), _ptr(workspace), ws_n, _stream(stream), ev)
    if rc != PISA_OK:
        raise PisaError("pisa_select_prefill_profiled", rc)


def decode_update_select(q_new: torch.Tensor, k_new: torch.Tensor, k_cache: torch.Tensor,
                         pyramid: torch.Tensor, n_before: int, n_capacity: int, dims: Dims,
                         out_idx: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                         stream=None) -> None:
    _check(q_new, "q_new", dims.torch_dtype, dims.B * dims.Hq * dims.d)
    _check(k_new, "k_new", dims.torch_dtype, dims.B * dims.Hkv * dims.d)
    _check(k_cache, "k_cache", dims.torch_dtype, dims.B * n_capacity * dims.Hkv * dims.d)
    _check(pyramid, "pyramid", torch.float32, dims.B * dims.Hkv * pyramid_nodes(dims, n_capacity) * dims.d)
    _check(out_idx, "out_idx", torch.int32, dims.B * dims.Hkv * dims.topk)
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.pisa_decode_update_select(_ptr(q_new), _ptr(k_new), _ptr(k_cache), _ptr(pyramid), n_before,
                                       n_capacity, ctypes.byref(dims), _ptr(out_idx), _ptr(workspace),
                                       ws_n, _stream(stream))
    if rc != PISA_OK:
        raise PisaError("pisa_decode_update_select", rc)


def decode_update_select_noalloc(q_new: torch.Tensor, k_new: torch.Tensor, k_cache: torch.Tensor,
                                 pyramid: torch.Tensor, n_before: int, n_capacity: int, dims: Dims,
                                 out_idx: torch.Tensor, stream=None) -> None:
    """decode_update_select (bf16) without a workspace: the library's static per-GPU scratch
    serves instead (B * Hkv <= 4096; calls overlapping on one GPU race)."""
    _check(q_new, "q_new", dims.torch_dtype, dims.B * dims.Hq * dims.d)
    _check(k_new, "k_new", dims.torch_dtype, dims.B * dims.Hkv * dims.d)
    _check(k_cache, "k_cache", dims.torch_dtype, dims.B * n_capacity * dims.Hkv * dims.d)
    _check(pyramid, "pyramid", torch.float32, dims.B * dims.Hkv * pyramid_nodes(dims, n_capacity) * dims.d)
    _check(out_idx, "out_idx", torch.int32, dims.B * dims.Hkv * dims.topk)
    rc = lib.pisa_decode_update_select_noalloc(_ptr(q_new), _ptr(k_new), _ptr(k_cache), _ptr(pyramid), n_before,
                                               n_capacity, ctypes.byref(dims), _ptr(out_idx), _stream(stream))
    if rc != PISA_OK:
        raise PisaError("pisa_decode_update_select_noalloc", rc)


# ------------------------------------------------------------------ packed documents --
# D documents laid end to end in T token rows; cu_seqlens (int32 device tensor [D + 1])
# holds their first rows and T. Each document is selected as a sequence of its own
# (positions and leaf indices counted from its start). dims.B must be 1.

def pack_pyramid_rows(dims: Dims, T: int, D: int) -> int:
    return int(lib.pisa_pack_pyramid_rows(ctypes.byref(dims), T, D))


def pack_level_offset(dims: Dims, T: int, D: int, level: int) -> int:
    return int(lib.pisa_pack_level_offset(ctypes.byref(dims), T, D, level))


def pack_workspace_bytes(dims: Dims, T: int, D: int) -> int:
    return int(lib.pisa_pack_workspace_bytes(ctypes.byref(dims), T, D))


def alloc_pack_pyramid(dims: Dims, T: int, D: int, device="cuda") -> torch.Tensor:
    return torch.empty((dims.Hkv, pack_pyramid_rows(dims, T, D), dims.d), dtype=torch.float32, device=device)


def alloc_pack_workspace(dims: Dims, T: int, D: int, device="cuda") -> Optional[torch.Tensor]:
    n = pack_workspace_bytes(dims, T, D)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def build_pyramid_packed(k: torch.Tensor, cu_seqlens: torch.Tensor, dims: Dims, pyramid: torch.Tensor,
                         stream=None) -> None:
    D, T = cu_seqlens.numel() - 1, k.shape[0]
    _check(k, "k", dims.torch_dtype, T * dims.Hkv * dims.d)
    _check(cu_seqlens, "cu_seqlens", torch.int32, D + 1)
    _check(pyramid, "pyramid", torch.float32, dims.Hkv * pack_pyramid_rows(dims, T, D) * dims.d)
    rc = lib.pisa_build_pyramid_packed(_ptr(k), _ptr(cu_seqlens), D, T, ctypes.byref(dims), _ptr(pyramid),
                                       _stream(stream))
    if rc != PISA_OK:
        raise PisaError("pisa_build_pyramid_packed", rc)


def select_prefill_packed(q: torch.Tensor, k: torch.Tensor, pyramid: torch.Tensor, cu_seqlens: torch.Tensor,
                          dims: Dims, out_idx: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                          stream=None) -> None:
    D, T = cu_seqlens.numel() - 1, q.shape[0]
    _check(q, "q", dims.torch_dtype, T * dims.Hq * dims.d)
    _check(k, "k", dims.torch_dtype, T * dims.Hkv * dims.d)
    _check(cu_seqlens, "cu_seqlens", torch.int32, D + 1)
    _check(pyramid, "pyramid", torch.float32, dims.Hkv * pack_pyramid_rows(dims, T, D) * dims.d)
    _check(out_idx, "out_idx", torch.int32, T * dims.Hkv * dims.topk)
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.pisa_select_prefill_packed(_ptr(q), _ptr(k), _ptr(pyramid), _ptr(cu_seqlens), D, T,
                                        ctypes.byref(dims), _ptr(out_idx), _ptr(workspace), ws_n,
                                        _stream(stream))
    if rc != PISA_OK:
        raise PisaError("pisa_select_prefill_packed", rc)


# ------------------------------------------------------------- attention (stage two) --
# Attention over the selected blocks: per query head, softmax over the keys <= t of the
# blocks its KV head selected (idx as pisa_select_prefill writes it), applied to their
# value rows. q [B, N, Hq, d], k and v [B, n_capacity, Hkv, d] bf16; out fp32 [B, N, Hq, d].

def attention_workspace_bytes(dims: Dims, N: int, n_capacity: Optional[int] = None) -> int:
    cap = N if n_capacity is None else n_capacity
    return int(lib.pisa_attention_workspace_bytes(ctypes.byref(dims), N, cap))


def alloc_attention_workspace(dims: Dims, N: int, n_capacity: Optional[int] = None,
                              device="cuda") -> Optional[torch.Tensor]:
    n = attention_workspace_bytes(dims, N, n_capacity)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def sparse_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor, N: int,
                     n_capacity: int, dims: Dims, out: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                     stream=None) -> None:
    _check(q, "q", dims.torch_dtype, dims.B * N * dims.Hq * dims.d)
    _check(k, "k", dims.torch_dtype, dims.B * n_capacity * dims.Hkv * dims.d)
    _check(v, "v", dims.torch_dtype, dims.B * n_capacity * dims.Hkv * dims.d)
    _check(idx, "idx", torch.int32, dims.B * N * dims.Hkv * dims.topk)
    _check(out, "out", torch.float32, dims.B * N * dims.Hq * dims.d)
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.pisa_sparse_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(idx), N, n_capacity, ctypes.byref(dims),
                                   _ptr(out), _ptr(workspace), ws_n, _stream(stream))
    if rc != PISA_OK:
        raise PisaError("pisa_sparse_attention", rc)


def pack_attention_workspace_bytes(dims: Dims, T: int, D: int) -> int:
    return int(lib.pisa_pack_attention_workspace_bytes(ctypes.byref(dims), T, D))


def alloc_pack_attention_workspace(dims: Dims, T: int, D: int, device="cuda") -> Optional[torch.Tensor]:
    n = pack_attention_workspace_bytes(dims, T, D)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def sparse_attention_packed(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor,
                            cu_seqlens: torch.Tensor, dims: Dims, out: torch.Tensor,
                            workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Attention over the selected blocks of a pack: idx [T, Hkv, K] of document-local blocks (as
    select_prefill_packed writes them); each row attends inside its own document only."""
    D, T = cu_seqlens.numel() - 1, q.shape[0]
    _check(q, "q", dims.torch_dtype, T * dims.Hq * dims.d)
    _check(k, "k", dims.torch_dtype, T * dims.Hkv * dims.d)
    _check(v, "v", dims.torch_dtype, T * dims.Hkv * dims.d)
    _check(idx, "idx", torch.int32, T * dims.Hkv * dims.topk)
    _check(cu_seqlens, "cu_seqlens", torch.int32, D + 1)
    _check(out, "out", torch.float32, T * dims.Hq * dims.d)
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.pisa_sparse_attention_packed(_ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(cu_seqlens), D, T,
                                          ctypes.byref(dims), _ptr(out), _ptr(workspace), ws_n, _stream(stream))
    if rc != PISA_OK:
        raise PisaError("pisa_sparse_attention_packed", rc)


def decode_attention_workspace_bytes(dims: Dims) -> int:
    return int(lib.pisa_decode_attention_workspace_bytes(ctypes.byref(dims)))


def alloc_decode_attention_workspace(dims: Dims, device="cuda") -> torch.Tensor:
    # zero-filled, though nothing requires it: its completion counters are tagged per call
    return torch.zeros(decode_attention_workspace_bytes(dims), dtype=torch.uint8, device=device)


def decode_attention(q_new: torch.Tensor, v_new: Optional[torch.Tensor], k_cache: torch.Tensor,
                     v_cache: torch.Tensor, idx: torch.Tensor, t: int, n_capacity: int, dims: Dims,
                     out: torch.Tensor, workspace: torch.Tensor, stream=None) -> None:
    """Attention of the decoding query at position t over its selected blocks (idx as
    decode_update_select writes it); v_new, if given, is written to row t of v_cache."""
    _check(q_new, "q_new", dims.torch_dtype, dims.B * dims.Hq * dims.d)
    if v_new is not None:
        _check(v_new, "v_new", dims.torch_dtype, dims.B * dims.Hkv * dims.d)
    _check(k_cache, "k_cache", dims.torch_dtype, dims.B * n_capacity * dims.Hkv * dims.d)
    _check(v_cache, "v_cache", dims.torch_dtype, dims.B * n_capacity * dims.Hkv * dims.d)
    _check(idx, "idx", torch.int32, dims.B * dims.Hkv * dims.topk)
    _check(out, "out", torch.float32, dims.B * dims.Hq * dims.d)
    ws_n = workspace.numel() * workspace.element_size()
    rc = lib.pisa_decode_attention(_ptr(q_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(idx), t, n_capacity,
                                   ctypes.byref(dims), _ptr(out), _ptr(workspace), ws_n, _stream(stream))
    if rc != PISA_OK:
        raise PisaError("pisa_decode_attention", rc)


# ------------------------------------------------------- flat stage-one selection --
# The selection the pyramid replaces: every query scores every eligible leaf summary (the
# sum over its group's heads of q.kbar/sqrt(d)) and keeps the K best. Reads level 1 of a
# pyramid written by build_pyramid; out_idx [B, N, Hkv, K] as select_prefill writes it.

def flat_workspace_bytes(dims: Dims, N: int, n_capacity: Optional[int] = None) -> int:
    cap = N if n_capacity is None else n_capacity
    return int(lib.pisa_flat_workspace_bytes(ctypes.byref(dims), N, cap))


def alloc_flat_workspace(dims: Dims, N: int, n_capacity: Optional[int] = None,
                         device="cuda") -> Optional[torch.Tensor]:
    n = flat_workspace_bytes(dims, N, n_capacity)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def select_flat(q: torch.Tensor, pyramid: torch.Tensor, N: int, n_capacity: int, dims: Dims,
                out_idx: torch.Tensor, workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    _check(q, "q", dims.torch_dtype, dims.B * N * dims.Hq * dims.d)
    _check(pyramid, "pyramid", torch.float32, dims.B * dims.Hkv * pyramid_nodes(dims, n_capacity) * dims.d)
    _check(out_idx, "out_idx", torch.int32, dims.B * N * dims.Hkv * dims.topk)
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.pisa_select_flat(_ptr(q), _ptr(pyramid), N, n_capacity, ctypes.byref(dims), _ptr(out_idx),
                              _ptr(workspace), ws_n, _stream(stream))
    if rc != PISA_OK:
        raise PisaError("pisa_select_flat", rc)


# ------------------------------------------------------------ exact flat selection --
# Every eligible leaf block scored by the exact LSE over its raw keys up to t (summed over the
# group's heads), the K best kept: the ground truth the walk's recall is measured against.
# bf16 and the LSE score only; out_idx [B, N, Hkv, K] as select_prefill writes it.

def flat_exact_workspace_bytes(dims: Dims, N: int, n_capacity: Optional[int] = None) -> int:
    cap = N if n_capacity is None else n_capacity
    return int(lib.pisa_flat_exact_workspace_bytes(ctypes.byref(dims), N, cap))


def alloc_flat_exact_workspace(dims: Dims, N: int, n_capacity: Optional[int] = None,
                               device="cuda") -> Optional[torch.Tensor]:
    n = flat_exact_workspace_bytes(dims, N, n_capacity)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def select_flat_exact(q: torch.Tensor, k: torch.Tensor, N: int, n_capacity: int, dims: Dims,
                      out_idx: torch.Tensor, workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    _check(q, "q", dims.torch_dtype, dims.B * N * dims.Hq * dims.d)
    _check(k, "k", dims.torch_dtype, dims.B * n_capacity * dims.Hkv * dims.d)
    _check(out_idx, "out_idx", torch.int32, dims.B * N * dims.Hkv * dims.topk)
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib.pisa_select_flat_exact(_ptr(q), _ptr(k), N, n_capacity, ctypes.byref(dims), _ptr(out_idx),
                                    _ptr(workspace), ws_n, _stream(stream))
    if rc != PISA_OK:
        raise PisaError("pisa_select_flat_exact", rc)
