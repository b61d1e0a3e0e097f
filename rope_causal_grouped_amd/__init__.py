"""Causal grouped-query attention with RoPE (theta = 1e6) on MI355X.

Thin PyTorch-facing wrapper over the C ABI in include/gqa.h: it checks that
tensors live on the GPU, are contiguous and have the expected shapes, then
passes raw device pointers, sizes and the current HIP stream.  Every step
of the computation runs in the library's HIP kernels; there is no other
implementation behind these functions.
"""

from __future__ import annotations

import ctypes
import math

import torch

from ._lib import (GQA_BF16, GQA_F32, GQAError, check, lib)

__all__ = ["rope_apply", "prefill", "decode", "prefill_workspace_size",
           "decode_workspace_size", "timing_enable", "timing_read", "version",
           "GQAError", "ROPE_THETA"]

ROPE_THETA = 1.0e6

_DT = {torch.float32: GQA_F32, torch.bfloat16: GQA_BF16}


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")
    return _DT[t.dtype]


def _dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def version() -> str:
    return lib().gqa_version().decode()


def rope_apply(x: torch.Tensor, pos0: int = 0, theta: float = ROPE_THETA) -> torch.Tensor:
    """In-place RoPE on x[B, L, h, d]; row l at position pos0 + l."""
    _dev(x)
    B, L, h, d = x.shape
    check(lib().gqa_rope_apply(_ptr(x), _dt(x), B, L, h, d, pos0, theta, _stream()))
    return x


def prefill_workspace_size(dtype: torch.dtype, B: int, L: int, h_kv: int, d: int) -> int:
    return lib().gqa_prefill_workspace_size(_DT[dtype], B, L, h_kv, d)


def decode_workspace_size(B: int, h_q: int, h_kv: int, d: int, cap: int) -> int:
    return lib().gqa_decode_workspace_size(B, h_q, h_kv, d, cap)


def prefill(q, k, v, *, theta: float = ROPE_THETA, scale: float | None = None,
            causal: bool = True, out_dtype: torch.dtype = torch.float32, out=None,
            k_cache=None, v_cache=None, workspace=None):
    """Causal GQA prefill with fused RoPE.  q [B, L, h_q, d], k/v [B, L, h_kv, d]
    (float32 or bfloat16, same dtype); returns o [B, L, h_q, d] in out_dtype.
    k_cache/v_cache [B, cap, h_kv, d] (optional) receive rotated K and V."""
    _dev(q, k, v, out, k_cache, v_cache, workspace)
    B, L, h_q, d = q.shape
    h_kv = k.shape[2]
    if k.shape != (B, L, h_kv, d) or v.shape != k.shape:
        raise ValueError(f"k/v shapes {tuple(k.shape)}/{tuple(v.shape)} do not match q {tuple(q.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, L, h_q, d), dtype=out_dtype, device=q.device)
    cap = 0
    if k_cache is not None:
        cap = k_cache.shape[1]
        for c in (k_cache, v_cache):
            if c is None or c.dtype != q.dtype or c.shape != (B, cap, h_kv, d):
                raise ValueError("k_cache/v_cache must both be [B, cap, h_kv, d] of q's dtype")
    need = lib().gqa_prefill_workspace_size(_dt(q), B, L, h_kv, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    check(lib().gqa_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _dt(q), _dt(out), B, L, h_q,
                            h_kv, d, theta, scale, int(causal), _ptr(k_cache), _ptr(v_cache),
                            cap, _ptr(workspace), workspace.numel(), _stream()))
    return out


def decode(q, k_cache, v_cache, kv_len: int, q_pos: int, *, theta: float = ROPE_THETA,
           scale: float | None = None, out_dtype: torch.dtype = torch.float32, out=None,
           workspace=None):
    """One decode step.  q [B, h_q, d] (pre-RoPE), caches [B, cap, h_kv, d]
    holding rotated keys; attends to cache rows 0..kv_len-1."""
    _dev(q, k_cache, v_cache, out, workspace)
    B, h_q, d = q.shape
    cap, h_kv = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape != (B, cap, h_kv, d) or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [B, cap, h_kv, d] matching q")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("q and the caches must share one dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, h_q, d), dtype=out_dtype, device=q.device)
    if workspace is None:
        need = lib().gqa_decode_workspace_size(B, h_q, h_kv, d, cap)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    check(lib().gqa_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _dt(q), _dt(out), B,
                           h_q, h_kv, d, cap, kv_len, q_pos, theta, scale, _ptr(workspace),
                           workspace.numel(), _stream()))
    return out


def timing_enable(on: bool) -> None:
    check(lib().gqa_timing_enable(int(on)))


def timing_read(which: int):
    """(total_ms, count) of the kernels timed since the last read; which = 0
    for the prefill attention kernel, 1 for the decode streaming kernel."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    check(lib().gqa_timing_read(which, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
