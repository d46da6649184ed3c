"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no attention arithmetic: it only draws random numbers,
rounds them to bf16 and describes the workloads.  Both the fp64 oracle and
the GPU library receive arrays produced here, so both see bit-identical
inputs.

Recipe (the pages only say "random Q, K and V tensors", grasp.study lesson,
section "Verification: Does It Actually Work?"; the distribution is fixed
here): numpy ``default_rng(seed)`` (PCG64), ``standard_normal`` drawn as
float32 in the order Q, K, V.  The packed variable-length workload first
draws its sequence lengths with ``integers(1, max_len, endpoint=True)``,
then Q, K, V, and multiplies Q and K by 8 (exact in fp32 and in bf16, so it
commutes with rounding).  Decode-shaped inputs draw Q [B, H, Nq, d], then
K and V [B, H, Nk, d], the same way.  bf16 tensors are the
round-to-nearest-even rounding of the float32 draws.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

DTYPE_F32 = 0
DTYPE_BF16 = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16"
    H: int
    d: int
    causal: bool
    seed: int
    B: int = 1
    N: int = 0            # fixed-length workloads
    nseq: int = 0         # packed variable-length workloads
    max_len: int = 0
    qk_mult: float = 1.0

    @property
    def varlen(self) -> bool:
        return self.nseq > 0

    @property
    def scale(self) -> float:
        # the fp32 value handed to both sides
        return float(np.float32(1.0 / math.sqrt(self.d)))


# The five workloads: a one-tile fp32 head, a ragged causal bf16 case, the
# LLM-prefill shape, a long non-causal sequence, and a packed batch of 16
# sequences of random length with widened score range.
WORKLOADS = [
    Workload("b1h1n128d64_f32", "f32", H=1, d=64, causal=False, seed=7001, B=1, N=128),
    Workload("b1h8n1000d64_causal", "bf16", H=8, d=64, causal=True, seed=7002, B=1, N=1000),
    Workload("b4h32n4096d128_causal", "bf16", H=32, d=128, causal=True, seed=7003, B=4, N=4096),
    Workload("b1h16n16384d64", "bf16", H=16, d=64, causal=False, seed=7004, B=1, N=16384),
    Workload("varlen16x8192_h32d128_causal", "bf16", H=32, d=128, causal=True, seed=7005,
             nseq=16, max_len=8192, qk_mult=8.0),
]
HEADLINE = WORKLOADS[2]


def by_name(name: str) -> Workload:
    for w in WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns the
    16-bit patterns as uint16.  NaN stays a quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value, returned as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


@dataclasses.dataclass
class Inputs:
    """One batch of inputs.  ``q``, ``k``, ``v`` are float32 arrays holding
    exactly the values the GPU receives; ``bits`` (bf16 only) are the uint16
    patterns to upload.  Fixed-length layout [B, H, N, d]; packed layout
    [T, H, d] with ``cu_seqlens`` [nseq + 1]."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    dtype: str
    cu_seqlens: Optional[np.ndarray] = None
    q_bits: Optional[np.ndarray] = None
    k_bits: Optional[np.ndarray] = None
    v_bits: Optional[np.ndarray] = None

    def device_arrays(self):
        """Arrays to upload: uint16 bf16 patterns, or float32."""
        if self.dtype == "bf16":
            return self.q_bits, self.k_bits, self.v_bits
        return self.q, self.k, self.v


def _finish(q, k, v, dtype, cu=None) -> Inputs:
    if dtype == "bf16":
        qb, kb, vb = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
        return Inputs(bf16_bits_to_f32(qb), bf16_bits_to_f32(kb),
                      bf16_bits_to_f32(vb), dtype, cu, qb, kb, vb)
    if dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return Inputs(q, k, v, dtype, cu)


def draw_lengths(rng: np.random.Generator, nseq: int, max_len: int) -> np.ndarray:
    return rng.integers(1, max_len, size=nseq, endpoint=True).astype(np.int64)


def make_fixed(B: int, H: int, N: int, d: int, dtype: str, seed: int,
               qk_mult: float = 1.0) -> Inputs:
    """i.i.d. N(0, 1) Q, K, V of shape [B, H, N, d]."""
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if qk_mult != 1.0:
        q *= np.float32(qk_mult)
        k *= np.float32(qk_mult)
    return _finish(q, k, v, dtype)


def make_varlen(lengths, H: int, d: int, dtype: str, rng: np.random.Generator,
                qk_mult: float = 1.0) -> Inputs:
    """Packed [T, H, d] Q, K, V for the given sequence lengths."""
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(lengths.size + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    shape = (T, H, d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if qk_mult != 1.0:
        q *= np.float32(qk_mult)
        k *= np.float32(qk_mult)
    return _finish(q, k, v, dtype, cu)


def make(w: Workload) -> Inputs:
    """Inputs of a named workload, from its fixed seed."""
    if w.varlen:
        rng = np.random.default_rng(w.seed)
        lengths = draw_lengths(rng, w.nseq, w.max_len)
        return make_varlen(lengths, w.H, w.d, w.dtype, rng, w.qk_mult)
    return make_fixed(w.B, w.H, w.N, w.d, w.dtype, w.seed, w.qk_mult)


def workload_lengths(w: Workload) -> np.ndarray:
    """Sequence lengths of a workload without drawing the tensors."""
    if w.varlen:
        return draw_lengths(np.random.default_rng(w.seed), w.nseq, w.max_len)
    return np.full(w.B, w.N, dtype=np.int64)


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """A decode step: Nq new queries per (batch, head) against Nk cached keys."""
    name: str
    dtype: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    seed: int

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))


# Decode shapes: one new token for a batch of 16 sequences of 8K context;
# one sequence of 128K context (32 heads only, so the key range must be
# split to fill the GPU); 4 new tokens (a short causal block, as in
# speculative decoding) for 8 sequences of 16K context.
DECODE_WORKLOADS = [
    DecodeWorkload("decode_b16h32q1k8192d128", "bf16", 16, 32, 1, 8192, 128, False, 7101),
    DecodeWorkload("decode_b1h32q1k131072d128", "bf16", 1, 32, 1, 131072, 128, False, 7102),
    DecodeWorkload("decode_b8h32q4k16384d128_causal", "bf16", 8, 32, 4, 16384, 128, True, 7103),
]


def decode_by_name(name: str) -> DecodeWorkload:
    for w in DECODE_WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


def make_decode(B: int, H: int, Nq: int, Nk: int, d: int, dtype: str, seed: int) -> Inputs:
    """i.i.d. N(0, 1) Q [B, H, Nq, d], then K, V [B, H, Nk, d]."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, Nq, d), dtype=np.float32)
    k = rng.standard_normal((B, H, Nk, d), dtype=np.float32)
    v = rng.standard_normal((B, H, Nk, d), dtype=np.float32)
    return _finish(q, k, v, dtype)


def make_decode_workload(w: DecodeWorkload) -> Inputs:
    return make_decode(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.seed)
