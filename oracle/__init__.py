"""fp64 CPU oracle for the attention forward pass -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (``flashattention_forward_07_amd``)
never imports it, and the two share no code: the oracle is plain C
(``fa_ref.c``, fp64, OpenMP over rows) plus this ctypes wrapper.

What it computes is the definition of attention on the page "Mini
FlashAttention", section 1 ("What attention is"): S = Q K^T * scale,
row softmax, O = P V, optionally with the causal mask S[i, j] = -inf for
j > i; plus lse_i = ln sum_j exp(S[i, j]) over the allowed keys.  The
algorithm is the plain three-pass softmax per row described on the page
"How Did I Write My First FlashAttention Kernel in CUDA?" (max, then sum of
exponentials, then normalisation).  ``online`` is the chunked running-state
recurrence of "Mini FlashAttention", section 4, kept only so the tests can
check it against the three-pass result.

Inputs are float32 numpy arrays holding the exact values the GPU sees
(bf16 inputs widened exactly); outputs are float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa_ref.c")
_LIB_PATH = os.path.join(_HERE, "libfa355_ref.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile fa_ref.c into libfa355_ref.so (gcc, -O2, OpenMP)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", _SRC,
           "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _bind(lib):
    """Declare the C signatures on a loaded oracle library."""
    P = ctypes.c_void_p
    i32 = ctypes.c_int
    f64 = ctypes.c_double
    lib.fa_ref_fwd.argtypes = [P, P, P, P, P, i32, i32, i32, i32, f64, i32]
    lib.fa_ref_fwd_rows.argtypes = [P, P, P, i32, i32, i32, i32, f64, i32,
                                    P, i32, P, P]
    lib.fa_ref_fwd_varlen.argtypes = [P, P, P, P, P, P, i32, i32, i32, f64,
                                      i32]
    lib.fa_ref_fwd_varlen_rows.argtypes = [P, P, P, P, i32, i32, i32, f64,
                                           i32, P, i32, P, P]
    lib.fa_ref_online.argtypes = [P, P, P, P, P, i32, i32, f64, i32, i32]
    lib.fa_ref_fwd_decode.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32,
                                      f64, i32]
    lib.fa_ref_set_threads.argtypes = [i32]
    lib.fa_ref_set_threads.restype = None
    lib.fa_ref_threads.restype = i32
    for name in ("fa_ref_fwd", "fa_ref_fwd_rows", "fa_ref_fwd_varlen",
                 "fa_ref_fwd_varlen_rows", "fa_ref_online", "fa_ref_fwd_decode"):
        getattr(lib, name).restype = i32
    return lib


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"oracle {name} failed with code {rc}")


def set_threads(n: int) -> None:
    _load().fa_ref_set_threads(int(n))


def threads() -> int:
    return int(_load().fa_ref_threads())


def attention(q, k, v, scale, causal=False):
    """Fixed-length batch.  q, k, v: [B, H, N, d] (or [N, d] for one head).
    Returns (o [.., N, d] float64, lse [.., N] float64)."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    squeeze = q.ndim == 2
    if squeeze:
        q, k, v = q[None, None], k[None, None], v[None, None]
    if q.shape != k.shape or q.shape != v.shape or q.ndim != 4:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    B, H, N, d = q.shape
    o = np.empty((B, H, N, d), np.float64)
    lse = np.empty((B, H, N), np.float64)
    rc = _load().fa_ref_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                            B, H, N, d, float(scale), int(bool(causal)))
    _check(rc, "fa_ref_fwd")
    if squeeze:
        return o[0, 0], lse[0, 0]
    return o, lse


def attention_rows(q, k, v, scale, causal, rows):
    """Selected rows of a fixed-length batch; rows are flat indices into
    [B, H, N].  Returns (o [len(rows), d], lse [len(rows)])."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, N, d = q.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    o = np.empty((rows.size, d), np.float64)
    lse = np.empty(rows.size, np.float64)
    rc = _load().fa_ref_fwd_rows(_ptr(q), _ptr(k), _ptr(v), B, H, N, d,
                                 float(scale), int(bool(causal)), _ptr(rows),
                                 rows.size, _ptr(o), _ptr(lse))
    _check(rc, "fa_ref_fwd_rows")
    return o, lse


def attention_decode(q, k, v, scale, causal=False):
    """Decode-shaped batch: q [B, H, Nq, d] against k, v [B, H, Nk, d] (or
    [Nq, d] / [Nk, d] for one head).  The queries are the newest Nq
    positions of the Nk-long sequence: with the causal mask query i sees
    keys 0 .. Nk - Nq + i.  Returns (o [.., Nq, d], lse [.., Nq]) float64."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    squeeze = q.ndim == 2
    if squeeze:
        q, k, v = q[None, None], k[None, None], v[None, None]
    if q.ndim != 4 or k.shape != v.shape or k.ndim != 4 or q.shape[:2] != k.shape[:2] \
            or q.shape[3] != k.shape[3]:
        raise ValueError("q [B, H, Nq, d] and k, v [B, H, Nk, d] expected")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    o = np.empty((B, H, Nq, d), np.float64)
    lse = np.empty((B, H, Nq), np.float64)
    rc = _load().fa_ref_fwd_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                   B, H, Nq, Nk, d, float(scale), int(bool(causal)))
    _check(rc, "fa_ref_fwd_decode")
    if squeeze:
        return o[0, 0], lse[0, 0]
    return o, lse


def attention_varlen(q, k, v, cu_seqlens, scale, causal=False):
    """Packed batch: q, k, v [T, H, d], cu_seqlens [nseq + 1] int32.
    Returns (o [T, H, d], lse [T, H]) in float64."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    T, H, d = q.shape
    o = np.empty((T, H, d), np.float64)
    lse = np.empty((T, H), np.float64)
    rc = _load().fa_ref_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                   _ptr(lse), _ptr(cu), cu.size - 1, H, d,
                                   float(scale), int(bool(causal)))
    _check(rc, "fa_ref_fwd_varlen")
    return o, lse


def attention_varlen_rows(q, k, v, cu_seqlens, scale, causal, rows):
    """Selected rows of a packed batch; rows are flat indices token*H + head."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    T, H, d = q.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    o = np.empty((rows.size, d), np.float64)
    lse = np.empty(rows.size, np.float64)
    rc = _load().fa_ref_fwd_varlen_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(cu),
                                        cu.size - 1, H, d, float(scale),
                                        int(bool(causal)), _ptr(rows),
                                        rows.size, _ptr(o), _ptr(lse))
    _check(rc, "fa_ref_fwd_varlen_rows")
    return o, lse


def online(q, k, v, scale, causal, chunk):
    """The chunked recurrence of "Mini FlashAttention", section 4, one head
    [N, d].  Returns (o [N, d], lse [N]) in float64."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    N, d = q.shape
    o = np.empty((N, d), np.float64)
    lse = np.empty(N, np.float64)
    rc = _load().fa_ref_online(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                               N, d, float(scale), int(bool(causal)),
                               int(chunk))
    _check(rc, "fa_ref_online")
    return o, lse
