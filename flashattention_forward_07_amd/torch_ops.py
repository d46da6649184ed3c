"""libfa355 as PyTorch operators (forward only).

    import flashattention_forward_07_amd.torch_ops      # registers the ops
    o, lse = torch.ops.fa355.fwd(q, k, v, causal, scale)
    o, lse = torch.ops.fa355.fwd_varlen(q, k, v, cu_seqlens, max_seqlen, causal, scale)
    o, lse = torch.ops.fa355.decode(q, k_cache, v_cache, causal, scale, num_splits)

The operators allocate the outputs with torch and enqueue the library's
kernel on the current stream of the inputs' device through the C ABI (the
same call as ``fa_fwd`` / ``fa_fwd_varlen``); they compute nothing
themselves.  Each has a fake (meta) implementation, so shape propagation,
``torch.compile`` graphs and ``torch.library.opcheck`` see correct output
shapes without running the kernel.  No backward is registered: the
library is a forward pass.

``scale`` None means 1/sqrt(d).  Shapes and dtypes follow the C ABI:
q, k, v contiguous [B, H, N, d] (or packed [T, H, d] with int32
``cu_seqlens`` [nseq + 1] on the device), bf16 or fp32, d in {64, 128}.
``decode`` takes q [B, H, Nq, d] (the newest Nq positions, Nq <= 64) and
k, v [B, H, Nk, d]; it allocates the split workspace with torch as well.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import torch

from . import (FA_DTYPE_BF16, FA_DTYPE_F32, fa_decode_fwd, fa_decode_workspace_bytes, fa_fwd,
               fa_fwd_varlen)

__all__ = ["fwd", "fwd_varlen", "decode"]


def _code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FA_DTYPE_BF16
    if t.dtype == torch.float32:
        return FA_DTYPE_F32
    raise ValueError(f"fa355: unsupported dtype {t.dtype} (bfloat16 or float32)")


def _check(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, rank: int) -> None:
    if q.dim() != rank:
        raise ValueError(f"fa355: q must have {rank} dimensions, got {tuple(q.shape)}")
    for t in (k, v):
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("fa355: q, k and v must share shape, dtype and device")
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("fa355: q, k and v must be contiguous")


def _check_varlen(q, k, v, cu_seqlens) -> None:
    _check(q, k, v, 3)
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
        raise ValueError("fa355: cu_seqlens must be a 1-d int32 tensor")


@torch.library.custom_op("fa355::fwd", mutates_args=())
def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
        scale: Optional[float] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Attention forward over [B, H, N, d]; returns (o [B, H, N, d], lse [B, H, N] fp32)."""
    _check(q, k, v, 4)
    B, H, N, d = q.shape
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa_fwd(q, k, v, o, lse, B, H, N, d, sc, causal, _code(q),
           torch.cuda.current_stream(q.device))
    return o, lse


@fwd.register_fake
def _fwd_fake(q, k, v, causal=False, scale=None):
    _check(q, k, v, 4)
    B, H, N, _ = q.shape
    return torch.empty_like(q), q.new_empty((B, H, N), dtype=torch.float32)


@torch.library.custom_op("fa355::fwd_varlen", mutates_args=())
def fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
               max_seqlen: int, causal: bool = False,
               scale: Optional[float] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Attention forward over a packed batch [T, H, d]; returns (o [T, H, d], lse [T, H])."""
    _check_varlen(q, k, v, cu_seqlens)
    T, H, d = q.shape
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q)
    lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, cu_seqlens.numel() - 1, int(max_seqlen), H, d,
                  sc, causal, _code(q), torch.cuda.current_stream(q.device))
    return o, lse


@fwd_varlen.register_fake
def _fwd_varlen_fake(q, k, v, cu_seqlens, max_seqlen, causal=False, scale=None):
    _check_varlen(q, k, v, cu_seqlens)
    T, H, _ = q.shape
    return torch.empty_like(q), q.new_empty((T, H), dtype=torch.float32)


def _check_decode(q, k, v) -> None:
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("fa355: decode takes q [B, H, Nq, d] and k, v [B, H, Nk, d]")
    if k.shape[0] != q.shape[0] or k.shape[1] != q.shape[1] or k.shape[3] != q.shape[3]:
        raise ValueError("fa355: q, k and v must share B, H and d")
    for t in (k, v):
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError("fa355: q, k and v must share dtype and device")
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("fa355: q, k and v must be contiguous")


@torch.library.custom_op("fa355::decode", mutates_args=())
def decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
           scale: Optional[float] = None, num_splits: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """Split-KV decode: q [B, H, Nq, d] against k, v [B, H, Nk, d]; returns
    (o [B, H, Nq, d], lse [B, H, Nq] fp32)."""
    _check_decode(q, k, v)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    need = fa_decode_workspace_bytes(B, H, Nq, Nk, d, num_splits)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device) if need > 0 else None
    fa_decode_fwd(q, k, v, o, lse, ws, need, B, H, Nq, Nk, d, sc, causal, _code(q), num_splits,
                  torch.cuda.current_stream(q.device))
    return o, lse


@decode.register_fake
def _decode_fake(q, k, v, causal=False, scale=None, num_splits=0):
    _check_decode(q, k, v)
    B, H, Nq, _ = q.shape
    return torch.empty_like(q), q.new_empty((B, H, Nq), dtype=torch.float32)
