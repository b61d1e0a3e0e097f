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

__all__ = ["rope_apply", "prefill", "decode", "decode_noalloc", "prefill_chunk", "decode_ragged",
           "decode_append", "qkv_epilogue", "decode_paged", "decode_paged_workspace_size",
           "set_rope_yarn", "prefill_workspace_size", "prefill_chunk_workspace_size",
           "decode_workspace_size", "timing_enable", "timing_read", "stream_read", "version",
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


def decode_noalloc(q, k_cache, v_cache, kv_len: int, q_pos: int, *, out, theta: float = ROPE_THETA,
                   scale: float | None = None):
    """decode() on the library's static per-GPU scratch: no workspace and no
    device allocation in the call (the caller passes `out`).  Calls that
    overlap on one GPU share that scratch and race."""
    _dev(q, k_cache, v_cache, out)
    B, h_q, d = q.shape
    cap, h_kv = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape != (B, cap, h_kv, d) or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [B, cap, h_kv, d] matching q")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("q and the caches must share one dtype")
    if out.shape != (B, h_q, d):
        raise ValueError("out must be [B, h_q, d]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    check(lib().gqa_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _dt(q),
                                   _dt(out), B, h_q, h_kv, d, cap, kv_len, q_pos, theta, scale,
                                   _stream()))
    return out


def _seq_array(x, B: int, device, what: str):
    """Per-sequence int64 device array of B entries (a tensor or a sequence)."""
    if x is None:
        return None
    t = x if isinstance(x, torch.Tensor) else torch.tensor(list(x), dtype=torch.int64)
    if t.dtype != torch.int64 or t.numel() != B:
        raise ValueError(f"{what} must hold B={B} int64 entries")
    if not t.is_cuda:
        t = t.to(device)
    return t.contiguous()


def _caches(k_cache, v_cache, B, h_kv, d, dtype):
    cap = k_cache.shape[1]
    for c in (k_cache, v_cache):
        if c.dtype != dtype or c.shape != (B, cap, h_kv, d):
            raise ValueError("k_cache/v_cache must both be [B, cap, h_kv, d] of the inputs' dtype")
    return cap


def prefill_chunk_workspace_size(dtype: torch.dtype, B: int, kend: int, h_kv: int, d: int) -> int:
    return lib().gqa_prefill_chunk_workspace_size(_DT[dtype], B, kend, h_kv, d)


def prefill_chunk(q, k, v, k_cache, v_cache, start, length=None, *, kend: int | None = None,
                  theta: float = ROPE_THETA, scale: float | None = None, q_rotated: bool = False,
                  out_dtype: torch.dtype = torch.float32, out=None, workspace=None):
    """Chunked causal prefill.  q [B, C, h_q, d], k/v [B, C, h_kv, d] (pre-RoPE)
    are the new rows of each sequence, at positions start[b] + i for
    i < length[b]; they are appended to the caches [B, cap, h_kv, d] and
    attend to every cached row up to their own position (k = v = None: the
    caches already hold these rows, e.g. from qkv_epilogue; q_rotated: q is
    rotated already, as qkv_epilogue returns it).  kend bounds
    start[b] + length[b] (default: cap).  Returns o [B, C, h_q, d]; rows
    i >= length[b] are left as they were in ``out`` (uninitialised if None)."""
    _dev(q, k, v, k_cache, v_cache, out, workspace)
    B, C, h_q, d = q.shape
    h_kv = k_cache.shape[2]
    if (k is None) != (v is None):
        raise ValueError("k and v must both be given or both be None")
    if k is not None:
        if k.shape != (B, C, h_kv, d) or v.shape != k.shape:
            raise ValueError("k/v must be [B, C, h_kv, d] matching q and the caches")
        if not (q.dtype == k.dtype == v.dtype):
            raise TypeError("q, k and v must share one dtype")
    cap = _caches(k_cache, v_cache, B, h_kv, d, q.dtype)
    kend = cap if kend is None else kend
    st = _seq_array(start, B, q.device, "start")
    ln = _seq_array(length, B, q.device, "length")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, C, h_q, d), dtype=out_dtype, device=q.device)
    need = lib().gqa_prefill_chunk_workspace_size(_dt(q), B, kend, h_kv, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    check(lib().gqa_prefill_chunk(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _dt(q), _dt(out), B, C,
                                  h_q, h_kv, d, _ptr(st), _ptr(ln), kend, theta, scale,
                                  int(q_rotated), _ptr(k_cache), _ptr(v_cache), cap,
                                  _ptr(workspace),
                                  workspace.numel(), _stream()))
    return out


def qkv_epilogue(qkv, bias, k_cache, v_cache, h_q: int, start, length=None, *,
                 kend: int | None = None, theta: float = ROPE_THETA, q_out=None):
    """Bias, head split and rotation of the packed projection output
    qkv [B, C, (h_q + 2 h_kv) d] (query heads, then key heads, then value
    heads); bias [(h_q + 2 h_kv) d] or None.  Writes the rotated K and the V
    of token i < length[b] into cache row start[b] + i and returns its
    rotated queries [B, C, h_q, d] (for prefill_chunk / decode_ragged with
    q_rotated=True)."""
    _dev(qkv, bias, k_cache, v_cache, q_out)
    B, C, width = qkv.shape
    h_kv, d = k_cache.shape[2], k_cache.shape[3]
    if width != (h_q + 2 * h_kv) * d:
        raise ValueError(f"qkv width {width} != (h_q + 2 h_kv) d = {(h_q + 2 * h_kv) * d}")
    if bias is not None and (bias.shape != (width,) or bias.dtype != qkv.dtype):
        raise ValueError("bias must be [(h_q + 2 h_kv) d] of qkv's dtype")
    cap = _caches(k_cache, v_cache, B, h_kv, d, qkv.dtype)
    kend = cap if kend is None else kend
    st = _seq_array(start, B, qkv.device, "start")
    ln = _seq_array(length, B, qkv.device, "length")
    if q_out is None:
        q_out = torch.empty((B, C, h_q, d), dtype=qkv.dtype, device=qkv.device)
    check(lib().gqa_qkv_epilogue(_ptr(qkv), _ptr(bias), _ptr(q_out), _ptr(k_cache),
                                 _ptr(v_cache), _dt(qkv), B, C, h_q, h_kv, d, cap, _ptr(st),
                                 _ptr(ln), kend, theta, _stream()))
    return q_out


def _decode_common(q, k_cache, v_cache, out, out_dtype, workspace, scale):
    B, h_q, d = q.shape
    h_kv = k_cache.shape[2]
    cap = _caches(k_cache, v_cache, B, h_kv, d, q.dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, h_q, d), dtype=out_dtype, device=q.device)
    if workspace is None:
        need = lib().gqa_decode_workspace_size(B, h_q, h_kv, d, cap)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    return B, h_q, h_kv, d, cap, scale, out, workspace


def decode_ragged(q, k_cache, v_cache, kv_len, q_pos, *, max_kv_len: int | None = None,
                  theta: float = ROPE_THETA, scale: float | None = None, q_rotated: bool = False,
                  out_dtype: torch.dtype = torch.float32, out=None, workspace=None):
    """Decode with per-sequence kv_len[b] and q_pos[b] (int64, B entries);
    max_kv_len bounds kv_len (default: cap); q_rotated: q is rotated already."""
    _dev(q, k_cache, v_cache, out, workspace)
    B, h_q, h_kv, d, cap, scale, out, workspace = _decode_common(
        q, k_cache, v_cache, out, out_dtype, workspace, scale)
    kl = _seq_array(kv_len, B, q.device, "kv_len")
    qp = _seq_array(q_pos, B, q.device, "q_pos")
    max_kv_len = cap if max_kv_len is None else max_kv_len
    check(lib().gqa_decode_ragged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _dt(q),
                                  _dt(out), B, h_q, h_kv, d, cap, _ptr(kl), _ptr(qp), max_kv_len,
                                  theta, scale, int(q_rotated), _ptr(workspace),
                                  workspace.numel(), _stream()))
    return out


def decode_append(q, k_new, v_new, k_cache, v_cache, pos, *, max_pos: int | None = None,
                  theta: float = ROPE_THETA, scale: float | None = None,
                  out_dtype: torch.dtype = torch.float32, out=None, workspace=None):
    """One step with KV append: k_new/v_new [B, h_kv, d] (pre-RoPE) go to cache
    row pos[b], then q [B, h_q, d] at pos[b] attends to rows 0..pos[b].
    max_pos bounds pos (default: cap - 1)."""
    _dev(q, k_new, v_new, k_cache, v_cache, out, workspace)
    B, h_q, h_kv, d, cap, scale, out, workspace = _decode_common(
        q, k_cache, v_cache, out, out_dtype, workspace, scale)
    if k_new.shape != (B, h_kv, d) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [B, h_kv, d]")
    if not (q.dtype == k_new.dtype == v_new.dtype):
        raise TypeError("q, k_new and v_new must share one dtype")
    ps = _seq_array(pos, B, q.device, "pos")
    max_pos = cap - 1 if max_pos is None else max_pos
    check(lib().gqa_decode_append(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                  _ptr(v_cache), _ptr(out), _dt(q), _dt(out), B, h_q, h_kv, d,
                                  cap, _ptr(ps), max_pos, theta, scale, _ptr(workspace),
                                  workspace.numel(), _stream()))
    return out


def decode_paged_workspace_size(B: int, h_q: int, h_kv: int, d: int, max_kv_len: int) -> int:
    return lib().gqa_decode_paged_workspace_size(B, h_q, h_kv, d, max_kv_len)


def decode_paged(q, k_pool, v_pool, block_table, q_pos, kv_len=None, *, k_new=None, v_new=None,
                 max_kv_len: int | None = None, theta: float = ROPE_THETA,
                 scale: float | None = None, q_rotated: bool = False,
                 out_dtype: torch.dtype = torch.float32, out=None, workspace=None):
    """Decode over page pools [num_pages, h_kv, page_size, d] through
    block_table [B, max_pages] (int32).  Without k_new/v_new, sequence b
    attends to positions 0..kv_len[b]-1; with them (kv_len None) the new
    token is first written at q_pos[b].  max_kv_len defaults to
    max_pages * page_size."""
    _dev(q, k_pool, v_pool, block_table, k_new, v_new, out, workspace)
    B, h_q, d = q.shape
    num_pages, h_kv, page_size = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    if k_pool.shape != (num_pages, h_kv, page_size, d) or v_pool.shape != k_pool.shape:
        raise ValueError("pools must be [num_pages, h_kv, page_size, d] matching q")
    if k_pool.dtype != q.dtype or v_pool.dtype != q.dtype:
        raise TypeError("q and the pools must share one dtype")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_pages]")
    max_pages = block_table.shape[1]
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new must both be given or both be None")
    if k_new is not None and (k_new.shape != (B, h_kv, d) or v_new.shape != k_new.shape):
        raise ValueError("k_new/v_new must be [B, h_kv, d]")
    qp = _seq_array(q_pos, B, q.device, "q_pos")
    kl = _seq_array(kv_len, B, q.device, "kv_len")
    max_kv_len = max_pages * page_size if max_kv_len is None else max_kv_len
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, h_q, d), dtype=out_dtype, device=q.device)
    if workspace is None:
        need = lib().gqa_decode_paged_workspace_size(B, h_q, h_kv, d, max_kv_len)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    check(lib().gqa_decode_paged(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool),
                                 _ptr(out), _dt(q), _dt(out), B, h_q, h_kv, d, page_size,
                                 num_pages, _ptr(block_table), max_pages, _ptr(kl), _ptr(qp),
                                 max_kv_len, theta, scale, int(q_rotated), _ptr(workspace),
                                 workspace.numel(), _stream()))
    return out


def set_rope_yarn(factor: float = 1.0, original_max_position: float = 32768.0,
                  beta_fast: float = 32.0, beta_slow: float = 1.0) -> None:
    """YaRN-scaled RoPE for every later call on this thread (factor 1: plain
    RoPE).  Qwen2's long-context setting: factor 4 over 32768 positions."""
    check(lib().gqa_set_rope_yarn(factor, original_max_position, beta_fast, beta_slow))


def timing_enable(on: bool) -> None:
    check(lib().gqa_timing_enable(int(on)))


def timing_read(which: int):
    """(total_ms, count) of the calls timed while timing was last enabled:
    which = 0 the prefill attention kernel, 1 the decode streaming kernel,
    2 whole prefill calls, 3 whole decode calls (first kernel's start to
    last kernel's end; events bound to the kernel dispatches)."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    check(lib().gqa_timing_read(which, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def stream_read(x: torch.Tensor, sink: torch.Tensor) -> None:
    """Benchmark helper: read all of the contiguous device tensor x once
    (16-byte non-temporal loads) on the current stream; sink is a device
    tensor of at least 4 bytes."""
    if not (x.is_cuda and sink.is_cuda and x.is_contiguous()) or sink.numel() * sink.element_size() < 4:
        raise ValueError("stream_read: contiguous device tensor and a device sink of >= 4 bytes")
    check(lib().gqa_stream_read(x.data_ptr(), x.numel() * x.element_size(), sink.data_ptr(),
                                torch.cuda.current_stream(x.device).cuda_stream))
