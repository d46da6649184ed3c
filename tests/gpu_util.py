"""Helpers for the GPU tests: upload seeded inputs, run libfa355 through its
C ABI binding, and compare with the fp64 oracle."""
import numpy as np
import torch

import flashattention_forward_07_amd as fa

# Tolerances against the fp64 oracle on identical inputs.
#   fp32 inputs: max abs error of O <= 1e-5.
#   bf16 inputs (fp32 accumulation, bf16 P and bf16 output): max abs <= 2e-2,
#   mean abs <= 2e-3.
# lse is computed from fp32 scores of the exact inputs in either dtype, so its
# error is fp32 rounding of the score sums: <= 2e-5 * max(1, |lse|) (the
# scores reach |s| ~ 1e3 in the widened-range workload; one fp32 ulp there is
# 6e-5 relative to 1, i.e. 6e-8 relative to |lse|).
TOL = {"f32": (1e-5, None), "bf16": (2e-2, 2e-3)}
LSE_RTOL = 2e-5


def to_device(x_np, dtype):
    """float32 numpy (or uint16 bf16 bits) -> device tensor."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x_np).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x_np, dtype=np.float32))
    return t.to("cuda")


def upload(inp):
    q, k, v = inp.device_arrays()
    return to_device(q, inp.dtype), to_device(k, inp.dtype), to_device(v, inp.dtype)


def run_fixed(inp, scale, causal, with_lse=True, stream=None):
    q, k, v = upload(inp)
    B, H, N, d = inp.q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda") if with_lse else None
    code = fa.FA_DTYPE_BF16 if inp.dtype == "bf16" else fa.FA_DTYPE_F32
    fa.fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, code, stream)
    torch.cuda.synchronize()
    return o, lse


def run_varlen(inp, scale, causal, max_seqlen=None, with_lse=True):
    q, k, v = upload(inp)
    T, H, d = inp.q.shape
    cu_np = inp.cu_seqlens
    cu = torch.from_numpy(cu_np).to("cuda")
    if max_seqlen is None:
        max_seqlen = int(np.max(np.diff(cu_np))) if cu_np.size > 1 else 0
    o = torch.empty_like(q)
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda") if with_lse else None
    code = fa.FA_DTYPE_BF16 if inp.dtype == "bf16" else fa.FA_DTYPE_F32
    fa.fa_fwd_varlen(q, k, v, o, lse, cu, cu_np.size - 1, max_seqlen, H, d, scale, causal, code)
    torch.cuda.synchronize()
    return o, lse


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def fp32_score_tol(q, k, v, scale):
    """Max-abs bound on O for fp32 inputs whose scores are far from O(1).

    An fp32 dot product of length d is off by about sqrt(d) * 2^-24 *
    sum_c |q_c k_c| (random-rounding model), so every softmax weight is off
    by a relative e <= scale * that; a relative weight error e moves a convex
    combination of V rows by at most 2 e max|v|.  Never below the 1e-5 bound
    that holds for unit-variance inputs."""
    q64 = np.abs(q.astype(np.float64)).reshape(-1, q.shape[-2], q.shape[-1])
    k64 = np.abs(k.astype(np.float64)).reshape(-1, k.shape[-2], k.shape[-1])
    d = q.shape[-1]
    dot_abs = max(float((qh @ kh.T).max()) for qh, kh in zip(q64, k64))
    e = scale * np.sqrt(d) * 2.0 ** -24 * dot_abs
    return max(1e-5, 2.0 * e * float(np.abs(v).max()))


def compare(o_gpu, o_ref, lse_gpu, lse_ref, dtype, what="", max_tol=None):
    """Element-wise comparison against the oracle; returns the error stats."""
    o = o_gpu if isinstance(o_gpu, np.ndarray) else host(o_gpu)
    assert o.shape == o_ref.shape, (o.shape, o_ref.shape)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    err = np.abs(o - o_ref)
    default_max, mean_tol = TOL[dtype]
    max_tol = default_max if max_tol is None else max_tol
    stats = {"max_abs": float(err.max()), "mean_abs": float(err.mean())}
    assert stats["max_abs"] <= max_tol, f"{what}: max abs err {stats['max_abs']:.3e} > {max_tol}"
    if mean_tol is not None:
        assert stats["mean_abs"] <= mean_tol, f"{what}: mean abs err {stats['mean_abs']:.3e}"
    if lse_gpu is not None:
        l = lse_gpu if isinstance(lse_gpu, np.ndarray) else host(lse_gpu)
        assert l.shape == lse_ref.shape
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(l), fin), f"{what}: lse finiteness differs"
        lerr = np.abs(l[fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin]))
        stats["lse_rel"] = float(lerr.max()) if lerr.size else 0.0
        assert stats["lse_rel"] <= LSE_RTOL, f"{what}: lse rel err {stats['lse_rel']:.3e}"
    return stats


class WholeOutput:
    """Error statistics of a whole output compared chunk by chunk (so that the
    fp64 reference of a large workload never has to be held at once).  Every
    element counts: max abs and mean abs of O over the whole output, and the
    largest relative lse error, against the same bounds as compare()."""

    def __init__(self, dtype, what=""):
        self.dtype, self.what = dtype, what
        self.max_abs = 0.0
        self.sum_abs = 0.0
        self.count = 0
        self.lse_rel = 0.0
        self.rows = 0

    def add(self, o_gpu, o_ref, lse_gpu, lse_ref):
        o = o_gpu if isinstance(o_gpu, np.ndarray) else host(o_gpu)
        assert o.shape == o_ref.shape, (o.shape, o_ref.shape)
        assert np.all(np.isfinite(o)), f"{self.what}: non-finite output (unwritten or NaN)"
        err = np.abs(o - o_ref)
        self.max_abs = max(self.max_abs, float(err.max()) if err.size else 0.0)
        self.sum_abs += float(err.sum())
        self.count += err.size
        l = lse_gpu if isinstance(lse_gpu, np.ndarray) else host(lse_gpu)
        assert l.shape == lse_ref.shape
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(l), fin), f"{self.what}: lse finiteness differs"
        lerr = np.abs(l[fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin]))
        if lerr.size:
            self.lse_rel = max(self.lse_rel, float(lerr.max()))
        self.rows += l.size

    def finish(self, max_tol=None):
        default_max, mean_tol = TOL[self.dtype]
        max_tol = default_max if max_tol is None else max_tol
        mean = self.sum_abs / max(1, self.count)
        stats = {"rows": self.rows, "elements": self.count, "max_abs": self.max_abs,
                 "mean_abs": mean, "lse_rel": self.lse_rel}
        print(f"{self.what}: whole output, {self.rows} rows: max abs {self.max_abs:.3e} "
              f"mean abs {mean:.3e} lse rel {self.lse_rel:.3e}", flush=True)
        assert self.max_abs <= max_tol, f"{self.what}: max abs err {self.max_abs:.3e} > {max_tol}"
        if mean_tol is not None:
            assert mean <= mean_tol, f"{self.what}: mean abs err {mean:.3e} > {mean_tol}"
        assert self.lse_rel <= LSE_RTOL, f"{self.what}: lse rel err {self.lse_rel:.3e}"
        return stats


def sample_rows(B, H, N, count, seed, block_m=128, block_n=64):
    """Flat [B, H, N] row indices: every tile edge of a few heads plus random rows."""
    rng = np.random.default_rng(seed)
    rows = set()
    heads = [(0, 0), (B - 1, H - 1)] + [(int(rng.integers(B)), int(rng.integers(H)))
                                        for _ in range(4)]
    edges = {0, 1, N - 1, N - 2}
    step = min(block_m, block_n)
    starts = list(range(0, N, step))
    picked = starts[:3] + starts[-3:] + list(rng.choice(starts, size=min(8, len(starts)),
                                                          replace=False))
    for t in picked:
        edges.update({t - 1, t, t + 1})
    edges = {e for e in edges if 0 <= e < N}
    for b, h in heads:
        for e in edges:
            rows.add((b * H + h) * N + e)
    while len(rows) < count + len(edges) * len(heads):
        rows.add(int(rng.integers(B * H * N)))
    return np.array(sorted(rows), dtype=np.int64)
