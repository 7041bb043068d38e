"""torch front end: allocate outputs/workspace with torch and call the C ABI.

Device memory and streams come from PyTorch; the computation is the HIP
library's.  Tensors must be contiguous [B][H][T][D] on one GPU, all of the
same dtype (torch.bfloat16 or torch.float32).

The C ABI sizes every buffer from its integer arguments, not from the real
allocations, so every wrapper checks here that the tensors it passes have
the shapes, dtype and device those arguments describe (a smaller ``out`` or
a k with a different batch would otherwise be read or written past its end).
Shape and dtype checks come first, then device and layout, so a mismatch is
reported (ValueError / TypeError) before anything reaches the GPU.
"""
from __future__ import annotations

import torch

from . import attn as _abi


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _abi.ATTN_BF16
    if t.dtype == torch.float32:
        return _abi.ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _on_gpu(**tensors):
    """Every tensor contiguous, on a GPU, and all on q's (the first's) device."""
    dev = None
    for name, t in tensors.items():
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, not on {dev}")


def _check_out(out, like, name="out"):
    """``out`` must be exactly like ``like``: shape, dtype (device and layout
    are checked with the inputs)."""
    if out.shape != like.shape:
        raise ValueError(f"{name} has shape {tuple(out.shape)}, expected {tuple(like.shape)}")
    if out.dtype != like.dtype:
        raise TypeError(f"{name} has dtype {out.dtype}, expected {like.dtype}")


def _check_qkv(q, k, v):
    """q [B][H_q][T_q][D], k and v [B][H_kv][T_kv][D], one dtype."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B][H][T][D], got {tuple(t.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    _dtype_code(q)
    if k.shape != v.shape:
        raise ValueError(f"k {tuple(k.shape)} and v {tuple(v.shape)} shapes differ")
    if q.shape[0] != k.shape[0]:
        raise ValueError(f"q has batch {q.shape[0]}, k and v have {k.shape[0]}")
    if q.shape[3] != k.shape[3]:
        raise ValueError(f"q has head dim {q.shape[3]}, k and v have {k.shape[3]}")
    if k.shape[1] == 0 or q.shape[1] % k.shape[1] != 0:
        raise ValueError(f"q heads ({q.shape[1]}) must be a multiple of kv heads ({k.shape[1]})")


def _stream(s, dev):
    return torch.cuda.current_stream(dev) if s is None else s


def prefill(q, k, v, causal: bool, scale: float, out=None, stream=None):
    """O = softmax(scale * Q K^T + mask) V; returns ``out`` (allocated if None)."""
    _check_qkv(q, k, v)
    if out is not None:
        _check_out(out, q)
    _on_gpu(q=q, k=k, v=v, **({} if out is None else {"out": out}))
    B, H_q, T_q, D = q.shape
    _, H_kv, T_kv, _ = k.shape
    o = torch.empty_like(q) if out is None else out
    _abi.attn_fwd_prefill(q, k, v, o, B, H_q, H_kv, T_q, T_kv, D, causal, scale, _dtype_code(q),
                          _stream(stream, q.device))
    return o


def decode_workspace(q, k, num_splits: int = 0):
    """Workspace tensor (uint8) sized for a decode call, or None if not needed."""
    B, H_q, _, D = q.shape
    _, H_kv, T_kv, _ = k.shape
    n = _abi.attn_fwd_decode_workspace_bytes(B, H_q, H_kv, T_kv, D, _dtype_code(q), num_splits)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def decode(q, k, v, scale: float, num_splits: int = 0, workspace=None, out=None, stream=None):
    """One query token per (batch, q head) against T_kv keys; q is [B][H_q][1][D]."""
    _check_qkv(q, k, v)
    if q.shape[2] != 1:
        raise ValueError(f"decode takes one query row per head, q has {q.shape[2]}")
    if out is not None:
        _check_out(out, q)
    extra = {} if out is None else {"out": out}
    if workspace is not None:
        extra["workspace"] = workspace
    _on_gpu(q=q, k=k, v=v, **extra)
    B, H_q, T_q, D = q.shape
    _, H_kv, T_kv, _ = k.shape
    o = torch.empty_like(q) if out is None else out
    ws = decode_workspace(q, k, num_splits) if workspace is None else workspace
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _abi.attn_fwd_decode(q, k, v, o, B, H_q, H_kv, T_q, T_kv, D, False, scale, _dtype_code(q),
                         num_splits, ws, ws_bytes, _stream(stream, q.device))
    return o


def decode_paged(q, k_pages, v_pages, block_table, seq_lens, scale: float, num_splits: int = 0,
                 workspace=None, out=None, stream=None):
    """Decode over a paged KV cache.

    q [B][H_q][1][D] (or [B][H_q][D]) bf16; k_pages, v_pages
    [num_pages][H_kv][page_size][D] bf16; block_table int32 [B][max_pages];
    seq_lens int32 [B].  Returns O shaped like q.
    """
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_table and seq_lens must be int32")
    if k_pages.shape != v_pages.shape or k_pages.dim() != 4:
        raise ValueError("k_pages and v_pages must both be [num_pages][H_kv][page_size][D]")
    if q.dim() == 4 and q.shape[2] != 1:
        raise ValueError(f"decode takes one query row per head, q has {q.shape[2]}")
    if q.dim() not in (3, 4):
        raise ValueError("q must be [B][H_q][1][D] or [B][H_q][D]")
    if not (q.dtype == k_pages.dtype == v_pages.dtype):
        raise TypeError("q, k_pages, v_pages must share a dtype")
    num_pages, H_kv, page_size, D = k_pages.shape
    B, H_q = q.shape[0], q.shape[1]
    if q.shape[-1] != D:
        raise ValueError(f"q has head dim {q.shape[-1]}, the pages have {D}")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be [B={B}][max_pages], got {tuple(block_table.shape)}")
    if seq_lens.dim() != 1 or seq_lens.shape[0] != B:
        raise ValueError(f"seq_lens must be [B={B}], got {tuple(seq_lens.shape)}")
    if out is not None:
        _check_out(out, q)
    extra = {} if out is None else {"out": out}
    if workspace is not None:
        extra["workspace"] = workspace
    _on_gpu(q=q, k_pages=k_pages, v_pages=v_pages, block_table=block_table, seq_lens=seq_lens,
            **extra)
    max_pages = block_table.shape[1]
    o = torch.empty_like(q) if out is None else out
    if workspace is None:
        n = _abi.attn_fwd_decode_paged_workspace_bytes(B, H_q, H_kv, D, page_size, max_pages,
                                                       num_splits)
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device) if n else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _abi.attn_fwd_decode_paged(q, k_pages, v_pages, o, block_table, seq_lens, B, H_q, H_kv, D,
                               page_size, num_pages, max_pages, scale, _dtype_code(q), num_splits,
                               workspace, ws_bytes, _stream(stream, q.device))
    return o


def prefill_window(q, k, v, window: int, scale: float, out=None, stream=None):
    """Causal sliding-window attention: row i (position i + T_kv - T_q) sees
    its last ``window`` keys.  bf16 [B][H][T][D] tensors."""
    _check_qkv(q, k, v)
    if out is not None:
        _check_out(out, q)
    _on_gpu(q=q, k=k, v=v, **({} if out is None else {"out": out}))
    B, H_q, T_q, D = q.shape
    _, H_kv, T_kv, _ = k.shape
    o = torch.empty_like(q) if out is None else out
    _abi.attn_fwd_prefill_window(q, k, v, o, B, H_q, H_kv, T_q, T_kv, D, window, scale,
                                 _dtype_code(q), _stream(stream, q.device))
    return o


def prefill_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                   causal: bool, scale: float, window: int = 0, out=None, stream=None):
    """Packed batch: q [total_q][H_q][D], k and v [total_k][H_kv][D] (bf16,
    token-major); int32 cu_seqlens [B + 1] on the GPU give each sequence's
    rows.  Returns O shaped like q."""
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape:
        raise ValueError("q must be [total_q][H_q][D], k and v [total_k][H_kv][D]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    if q.shape[2] != k.shape[2]:
        raise ValueError(f"q has head dim {q.shape[2]}, k and v have {k.shape[2]}")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if cu_seqlens_q.dim() != 1 or cu_seqlens_q.shape != cu_seqlens_k.shape or cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both be 1-D [B + 1]")
    if out is not None:
        _check_out(out, q)
    _on_gpu(q=q, k=k, v=v, cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k,
            **({} if out is None else {"out": out}))
    total_q, H_q, D = q.shape
    total_k, H_kv, _ = k.shape
    B = cu_seqlens_q.numel() - 1
    o = torch.empty_like(q) if out is None else out
    _abi.attn_fwd_prefill_varlen(q, k, v, o, cu_seqlens_q, cu_seqlens_k, B, H_q, H_kv, D, total_q,
                                 total_k, max_seqlen_q, max_seqlen_k, causal, window, scale,
                                 _dtype_code(q), _stream(stream, q.device))
    return o


def qkv_project(x, w, B: int, T: int, H_q: int, H_kv: int, D: int, stream=None):
    """Fused projection: x [B*T][d_model] and w [(H_q + 2 H_kv) D][d_model]
    (rows W_Q, then W_K, then W_V) in bf16; returns (q, k, v) head-major,
    [B][H_q][T][D] and [B][H_kv][T][D]."""
    for name, t in (("x", x), ("w", w)):
        if t.dim() != 2:
            raise ValueError(f"{name} must be 2-D, got {tuple(t.shape)}")
    if x.dtype != w.dtype:
        raise TypeError("x and w must share a dtype")
    d_model = x.shape[1]
    if x.shape[0] != B * T:
        raise ValueError(f"x has {x.shape[0]} rows, expected B*T = {B * T}")
    if tuple(w.shape) != ((H_q + 2 * H_kv) * D, d_model):
        raise ValueError(f"w has shape {tuple(w.shape)}, expected ({(H_q + 2 * H_kv) * D}, {d_model})")
    _on_gpu(x=x, w=w)
    q = torch.empty((B, H_q, T, D), dtype=x.dtype, device=x.device)
    k = torch.empty((B, H_kv, T, D), dtype=x.dtype, device=x.device)
    v = torch.empty_like(k)
    _abi.attn_qkv_project(x, w, q, k, v, B, T, d_model, H_q, H_kv, D, _dtype_code(x),
                          _stream(stream, x.device))
    return q, k, v
