"""Python binding of libfa355 -- the attention forward pass on MI355X.

Argument marshalling only: every entry point passes device pointers and
sizes straight to the C ABI of ``include/fa355.h`` (same names, same
arguments), and all computation runs in the HIP kernels of the library.
PyTorch supplies device memory and the current stream.  There is no
fallback: if ``libfa355.so`` has not been built, loading fails loudly.

    o, lse = attention(q, k, v, causal=True)             # [B, H, N, d]
    o, lse = attention_varlen(q, k, v, cu_seqlens, max_seqlen, causal=True)
    o, lse = naive_attention(q, k, v, causal=True)       # unfused baseline
    o, lse = decode_attention(q, k_cache, v_cache)        # q [B, H, Nq, d], split-KV
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "FA_DTYPE_F32", "FA_DTYPE_BF16", "FAError", "fa_fwd", "fa_fwd_varlen",
    "fa_status_string", "fa_last_hip_error", "fa_version", "attention",
    "attention_varlen", "library_path", "load", "fa_naive_fwd", "fa_naive_workspace_bytes",
    "naive_attention", "fa_decode_fwd", "fa_decode_workspace_bytes", "fa_decode_num_splits",
    "fa_decode_fwd_noalloc", "FA_DECODE_SCRATCH_BYTES",
    "decode_attention",
]

FA_DTYPE_F32 = 0
FA_DTYPE_BF16 = 1
FA_OK = 0

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa355.so")
_lib = None


class FAError(RuntimeError):
    """A nonzero status returned by libfa355."""

    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {fa_status_string(status)}"
        if status == 8:
            msg += f" (hipError {fa_last_hip_error()})"
        super().__init__(msg)


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libfa355.so (built in-tree by ``build.py``); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with "
            "`python -m flashattention_forward_07_amd.build` (there is no fallback path)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_fwd.argtypes = [P, P, P, P, P, i32, i32, i32, i32, f32, i32, i32, P]
    lib.fa_fwd.restype = i32
    lib.fa_fwd_varlen.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, f32, i32, i32, P]
    lib.fa_fwd_varlen.restype = i32
    lib.fa_naive_fwd.argtypes = [P, P, P, P, P, P, ctypes.c_size_t, i32, i32, i32, i32, f32,
                                 i32, i32, P]
    lib.fa_naive_fwd.restype = i32
    lib.fa_naive_workspace_bytes.argtypes = [i32, i32, i32]
    lib.fa_naive_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_decode_fwd.argtypes = [P, P, P, P, P, P, ctypes.c_size_t, i32, i32, i32, i32, i32,
                                  f32, i32, i32, i32, P]
    lib.fa_decode_fwd.restype = i32
    lib.fa_decode_fwd_noalloc.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, f32, i32, i32,
                                          i32, P]
    lib.fa_decode_fwd_noalloc.restype = i32
    lib.fa_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.fa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_decode_num_splits.argtypes = [i32, i32, i32, i32, i32]
    lib.fa_decode_num_splits.restype = i32
    lib.fa_status_string.argtypes = [i32]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_last_hip_error.argtypes = []
    lib.fa_last_hip_error.restype = i32
    lib.fa_version.argtypes = []
    lib.fa_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _ptr(x):
    """Device address of a tensor, an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError("libfa355 takes device tensors")
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, stream=None) -> None:
    """Enqueue attention forward over a fixed-length batch ([B, H, N, d])."""
    st = load().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H),
                       int(N), int(d), float(scale), int(bool(causal)), int(dtype),
                       _stream(stream))
    if st != FA_OK:
        raise FAError(st, "fa_fwd")


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, nseq, max_seqlen, H, d, scale, causal,
                  dtype, stream=None) -> None:
    """Enqueue attention forward over a packed batch ([T, H, d])."""
    st = load().fa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                              _ptr(cu_seqlens), int(nseq), int(max_seqlen), int(H), int(d),
                              float(scale), int(bool(causal)), int(dtype), _stream(stream))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_varlen")


def fa_naive_workspace_bytes(B, H, N) -> int:
    """Workspace bytes fa_naive_fwd needs (0 for sizes out of range)."""
    return int(load().fa_naive_workspace_bytes(int(B), int(H), int(N)))


def fa_naive_fwd(q, k, v, o, lse, workspace, workspace_bytes, B, H, N, d, scale, causal, dtype,
                 stream=None) -> None:
    """Enqueue the unfused three-step forward (scores in the workspace)."""
    st = load().fa_naive_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(workspace),
                             int(workspace_bytes), int(B), int(H), int(N), int(d), float(scale),
                             int(bool(causal)), int(dtype), _stream(stream))
    if st != FA_OK:
        raise FAError(st, "fa_naive_fwd")


def fa_decode_workspace_bytes(B, H, Nq, Nk, d, num_splits=0) -> int:
    """Workspace bytes fa_decode_fwd needs (0 when the keys are not split or
    the sizes are out of range)."""
    return int(load().fa_decode_workspace_bytes(int(B), int(H), int(Nq), int(Nk), int(d),
                                                int(num_splits)))


def fa_decode_num_splits(B, H, Nq, Nk, num_splits=0) -> int:
    """Key ranges per (b, h) that fa_decode_fwd uses (0 for sizes out of range)."""
    return int(load().fa_decode_num_splits(int(B), int(H), int(Nq), int(Nk), int(num_splits)))


def fa_decode_fwd(q, k, v, o, lse, workspace, workspace_bytes, B, H, Nq, Nk, d, scale, causal,
                  dtype, num_splits=0, stream=None) -> None:
    """Enqueue the split-KV decode forward (partials in the workspace)."""
    st = load().fa_decode_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(workspace),
                              int(workspace_bytes), int(B), int(H), int(Nq), int(Nk), int(d),
                              float(scale), int(bool(causal)), int(dtype), int(num_splits),
                              _stream(stream))
    if st != FA_OK:
        raise FAError(st, "fa_decode_fwd")


# Size of the library's static decode scratch (FA_DECODE_SCRATCH_BYTES).
FA_DECODE_SCRATCH_BYTES = 16 << 20


def fa_decode_fwd_noalloc(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, dtype, num_splits=0,
                          stream=None) -> None:
    """Enqueue the split-KV decode forward with its partial results in the
    library's static per-GPU scratch (no workspace, no allocation)."""
    st = load().fa_decode_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B),
                                      int(H), int(Nq), int(Nk), int(d), float(scale),
                                      int(bool(causal)), int(dtype), int(num_splits),
                                      _stream(stream))
    if st != FA_OK:
        raise FAError(st, "fa_decode_fwd_noalloc")


def fa_status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


def fa_last_hip_error() -> int:
    return int(load().fa_last_hip_error())


def fa_version() -> str:
    return load().fa_version().decode()


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return FA_DTYPE_BF16
    if t.dtype == torch.float32:
        return FA_DTYPE_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def attention(q, k, v, causal=False, scale=None, with_lse=True, stream=None):
    """softmax(q k^T * scale) v for q, k, v of shape [B, H, N, d] on the GPU.
    Returns (o, lse) with lse [B, H, N] fp32 (None if with_lse is False)."""
    import torch
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    for t in (q, k, v):
        if tuple(t.shape) != (B, H, N, d) or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous tensors of one [B, H, N, d] shape")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if with_lse else None
    fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, _dtype_code(q), stream)
    return o, lse


def attention_varlen(q, k, v, cu_seqlens, max_seqlen, causal=False, scale=None,
                     with_lse=True, stream=None):
    """Packed variable-length attention: q, k, v [T, H, d], cu_seqlens int32
    [nseq + 1] on the device.  Returns (o [T, H, d], lse [T, H])."""
    import torch
    T, H, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    for t in (q, k, v):
        if tuple(t.shape) != (T, H, d) or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous tensors of one [T, H, d] shape")
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda:
        raise ValueError("cu_seqlens must be an int32 device tensor")
    o = torch.empty_like(q)
    lse = torch.empty((T, H), dtype=torch.float32, device=q.device) if with_lse else None
    fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, cu_seqlens.numel() - 1, max_seqlen, H, d,
                  scale, causal, _dtype_code(q), stream)
    return o, lse


def naive_attention(q, k, v, causal=False, scale=None, with_lse=True, workspace=None,
                    stream=None):
    """The unfused three-step forward for q, k, v [B, H, N, d]; allocates the
    N x N workspace with torch unless one (uint8, large enough) is given."""
    import torch
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    for t in (q, k, v):
        if tuple(t.shape) != (B, H, N, d) or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous tensors of one [B, H, N, d] shape")
    need = fa_naive_workspace_bytes(B, H, N)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if with_lse else None
    fa_naive_fwd(q, k, v, o, lse, workspace, workspace.numel() * workspace.element_size(), B, H,
                 N, d, scale, causal, _dtype_code(q), stream)
    return o, lse


def decode_attention(q, k, v, causal=False, scale=None, with_lse=True, num_splits=0,
                     workspace=None, stream=None):
    """Decode-shaped attention: q [B, H, Nq, d] (the newest Nq positions)
    against k, v [B, H, Nk, d].  Allocates the split workspace with torch
    unless one (uint8, large enough) is given."""
    import torch
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if tuple(k.shape) != (B, H, Nk, d) or tuple(v.shape) != (B, H, Nk, d):
        raise ValueError("k and v must be [B, H, Nk, d] with q's B, H and d")
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous")
    need = fa_decode_workspace_bytes(B, H, Nq, Nk, d, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if with_lse else None
    fa_decode_fwd(q, k, v, o, lse, workspace, wbytes, B, H, Nq, Nk, d, scale, causal,
                  _dtype_code(q), num_splits, stream)
    return o, lse
