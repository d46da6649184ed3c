"""GPU parity of libfa355 (through its C ABI) against the fp64 oracle.

Small shapes are compared element by element in full: they span several
query and key tiles and end in a ragged tail.  The five named workloads run
at their full sizes in the launch configuration the benchmark times, into
NaN-filled outputs, and every element is compared with the oracle run on the
whole workload; properties that hold at any size (finite output, output
inside the convex hull of V, finite lse) are checked as well.
"""
import math

import numpy as np
import pytest

import fa_inputs
import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import flashattention_forward_07_amd as fa  # noqa: E402
from tests import gpu_util as gu  # noqa: E402


def _scale(d):
    return float(np.float32(1.0 / math.sqrt(d)))


# --- small shapes, full comparison ------------------------------------------

# (N = 255 and 256 sit on either side of the length from which d = 64 takes
# 128-key tiles)
SHAPES = [(2, 3, 300), (1, 2, 64), (1, 1, 1), (1, 1, 129), (1, 2, 127), (2, 1, 65),
          (1, 1, 513), (1, 2, 255), (1, 1, 256)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b%dh%dn%d" % s)
def test_small_shapes_full(dtype, d, causal, shape):
    B, H, N = shape
    print(f"case dtype={dtype} d={d} causal={causal} B={B} H={H} N={N}", flush=True)
    inp = fa_inputs.make_fixed(B, H, N, d, dtype, seed=1000 + N + d)
    scale = _scale(d)
    o, lse = gu.run_fixed(inp, scale, causal)
    o_ref, lse_ref = oracle.attention(inp.q, inp.k, inp.v, scale, causal)
    gu.compare(o, o_ref, lse, lse_ref, dtype, what=f"{shape}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [333, 1000])
def test_wide_score_range(dtype, d, N):
    # Q and K x8: scores spread over hundreds, the max moves across tiles and
    # the running reference is rebased on many of them, with rows of one
    # wave rebasing by very different factors.
    inp = fa_inputs.make_fixed(1, 4, N, d, dtype, seed=77 + N, qk_mult=8.0)
    for causal in (False, True):
        o, lse = gu.run_fixed(inp, _scale(d), causal)
        o_ref, lse_ref = oracle.attention(inp.q, inp.k, inp.v, _scale(d), causal)
        # fp32: scores of |q.k| ~ 1e3 carry fp32 rounding far above 1e-5
        tol = gu.fp32_score_tol(inp.q, inp.k, inp.v, _scale(d)) if dtype == "f32" else None
        gu.compare(o, o_ref, lse, lse_ref, dtype, what=f"x8 d={d} N={N} causal={causal}",
                   max_tol=tol)


# --- the five named workloads at full size ----------------------------------
#
# Each runs in the launch configuration the benchmark times, into outputs
# filled with NaN beforehand (a tile the schedule skipped would stay NaN),
# and every element of O and lse is compared with the fp64 oracle run on the
# whole workload, a few heads at a time so the host holds one chunk of the
# fp64 reference at once.

def _hull_check(o, v_dev, dtype):
    # Every output row is a convex combination of value rows.
    vmax = v_dev.float().abs().max().item()
    slack = 1e-5 if dtype == "f32" else vmax * 2.0 ** -8
    assert torch.isfinite(o.float()).all().item()
    assert o.float().abs().max().item() <= vmax + slack


HEAD_CHUNK = 4  # heads per oracle call on the large workloads


@pytest.mark.parametrize("w", fa_inputs.WORKLOADS[:4], ids=lambda w: w.name)
def test_workload_fixed(w):
    print(f"workload {w.name}", flush=True)
    inp = fa_inputs.make(w)
    B, H, N, d = inp.q.shape
    q, k, v = gu.upload(inp)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    code = fa.FA_DTYPE_BF16 if w.dtype == "bf16" else fa.FA_DTYPE_F32
    fa.fa_fwd(q, k, v, o, lse, B, H, N, d, w.scale, w.causal, code)
    torch.cuda.synchronize()
    _hull_check(o, v, w.dtype)
    assert torch.isfinite(lse).all().item()
    acc = gu.WholeOutput(w.dtype, what=w.name)
    for b in range(B):
        for h0 in range(0, H, HEAD_CHUNK):
            h1 = min(H, h0 + HEAD_CHUNK)
            o_ref, lse_ref = oracle.attention(inp.q[b:b + 1, h0:h1], inp.k[b:b + 1, h0:h1],
                                              inp.v[b:b + 1, h0:h1], w.scale, w.causal)
            acc.add(o[b:b + 1, h0:h1], o_ref, lse[b:b + 1, h0:h1], lse_ref)
    stats = acc.finish()
    assert stats["rows"] == B * H * N


def test_workload_varlen():
    w = fa_inputs.WORKLOADS[4]
    print(f"workload {w.name}", flush=True)
    inp = fa_inputs.make(w)
    T, H, d = inp.q.shape
    q, k, v = gu.upload(inp)
    cu = torch.from_numpy(inp.cu_seqlens).to("cuda")
    o = torch.full_like(q, float("nan"))
    lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    fa.fa_fwd_varlen(q, k, v, o, lse, cu, inp.cu_seqlens.size - 1, w.max_len, H, d, w.scale,
                     w.causal, fa.FA_DTYPE_BF16)
    torch.cuda.synchronize()
    _hull_check(o, v, w.dtype)
    assert torch.isfinite(lse).all().item()
    acc = gu.WholeOutput(w.dtype, what=w.name)
    for h0 in range(0, H, HEAD_CHUNK):
        h1 = min(H, h0 + HEAD_CHUNK)
        o_ref, lse_ref = oracle.attention_varlen(inp.q[:, h0:h1], inp.k[:, h0:h1],
                                                 inp.v[:, h0:h1], inp.cu_seqlens, w.scale,
                                                 w.causal)
        acc.add(o[:, h0:h1], o_ref, lse[:, h0:h1], lse_ref)
    stats = acc.finish()
    assert stats["rows"] == T * H


# --- packed batches, full comparison ----------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lengths", [[1, 0, 127, 128, 129, 300, 2, 64],  # an empty sequence
                                     [200, 17, 0, 129, 65, 255]],  # longest below 256
                         ids=["max300", "max255"])
def test_varlen_small_full(dtype, d, causal, lengths):
    rng = np.random.default_rng((5 if len(lengths) == 8 else 7) + d)
    inp = fa_inputs.make_varlen(lengths, 3, d, dtype, rng)
    o, lse = gu.run_varlen(inp, _scale(d), causal)
    o_ref, lse_ref = oracle.attention_varlen(inp.q, inp.k, inp.v, inp.cu_seqlens, _scale(d),
                                             causal)
    gu.compare(o, o_ref, lse, lse_ref, dtype, what=f"varlen {lengths}")


def test_varlen_writes_nothing_outside_the_batch():
    lengths = [5, 130, 17]
    rng = np.random.default_rng(3)
    inp = fa_inputs.make_varlen(lengths, 2, 128, "bf16", rng)
    q, k, v = gu.upload(inp)
    T, H, d = inp.q.shape
    pad = 4096
    o_buf = torch.full((T * H * d + 2 * pad,), 7.0, dtype=torch.bfloat16, device="cuda")
    l_buf = torch.full((T * H + 2 * pad,), 7.0, dtype=torch.float32, device="cuda")
    o = o_buf[pad:pad + T * H * d]
    lse = l_buf[pad:pad + T * H]
    cu = torch.from_numpy(inp.cu_seqlens).cuda()
    fa.fa_fwd_varlen(q, k, v, o, lse, cu, len(lengths), 130, H, d, _scale(d), True,
                     fa.FA_DTYPE_BF16)
    torch.cuda.synchronize()
    assert (o_buf[:pad] == 7).all().item() and (o_buf[-pad:] == 7).all().item()
    assert (l_buf[:pad] == 7).all().item() and (l_buf[-pad:] == 7).all().item()
    o_ref, lse_ref = oracle.attention_varlen(inp.q, inp.k, inp.v, inp.cu_seqlens, _scale(d), True)
    gu.compare(o.reshape(T, H, d), o_ref, lse.reshape(T, H), lse_ref, "bf16")


# --- closed forms and behaviour -----------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_give_prefix_means(causal):
    N, d = 200, 128
    inp = fa_inputs.make_fixed(1, 1, N, d, "f32", seed=11)
    inp.q[:] = 0.0
    o, lse = gu.run_fixed(inp, 0.1, causal)
    v = inp.v[0, 0].astype(np.float64)
    want = np.cumsum(v, axis=0) / np.arange(1, N + 1)[:, None] if causal else \
        np.broadcast_to(v.mean(axis=0), v.shape)
    assert np.max(np.abs(gu.host(o)[0, 0] - want)) <= 1e-5
    n_allowed = np.arange(1, N + 1) if causal else np.full(N, N)
    assert np.max(np.abs(gu.host(lse)[0, 0] - np.log(n_allowed))) <= 1e-5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_token_gives_v(dtype):
    inp = fa_inputs.make_fixed(3, 2, 1, 64, dtype, seed=12)
    for causal in (False, True):
        o, lse = gu.run_fixed(inp, 0.125, causal)
        if dtype == "bf16":  # the bf16 store rounds the last-ulp wobble away
            assert np.array_equal(gu.host(o), inp.v.astype(np.float64))
        else:
            # the weight of the only key is exp2(fma(s, c, -fl(s c))): 1 to
            # within one fp32 rounding, so O = V to within two ulps
            np.testing.assert_allclose(gu.host(o), inp.v, rtol=2.0 ** -21, atol=0)


@pytest.mark.parametrize("dtype,N", [("bf16", 257), ("bf16", 100), ("f32", 100), ("f32", 300)])
def test_lse_is_optional_and_output_unchanged(dtype, N):
    """With and without lse, on the streaming kernels (N > 128) and on the
    one-tile kernels (N <= 128)."""
    inp = fa_inputs.make_fixed(1, 4, N, 128, dtype, seed=13)
    o1, _ = gu.run_fixed(inp, 0.09, True, with_lse=True)
    o2, lse2 = gu.run_fixed(inp, 0.09, True, with_lse=False)
    assert lse2 is None
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("dtype,N", [("bf16", 1000), ("bf16", 64), ("f32", 100)])
def test_run_to_run_bitwise_determinism(dtype, N):
    inp = fa_inputs.make_fixed(2, 8, N, 128, dtype, seed=14)
    outs = [gu.run_fixed(inp, 0.088, True) for _ in range(3)]
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])


def test_side_stream_launch():
    inp = fa_inputs.make_fixed(1, 2, 300, 64, "bf16", seed=15)
    s = torch.cuda.Stream()
    q, k, v = gu.upload(inp)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        o, lse = fa.attention(q, k, v, causal=True)
    s.synchronize()
    o_ref, lse_ref = oracle.attention(inp.q, inp.k, inp.v, 0.125, True)
    gu.compare(o, o_ref, lse, lse_ref, "bf16")


def test_empty_problem_enqueues_nothing():
    q = torch.zeros((0, 2, 16, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = fa.attention(q, q, q)
    assert o.shape == q.shape and lse.shape == (0, 2, 16)


# --- head grouping per XCD: every (head, query tile) computed exactly once ----

def _run_nan_filled(inp, scale, causal, varlen):
    """Launch with O and lse filled with NaN, so that a tile the schedule
    skipped shows up as NaN rather than as stale memory."""
    q, k, v = gu.upload(inp)
    o = torch.full_like(q, float("nan"))
    code = fa.FA_DTYPE_BF16 if inp.dtype == "bf16" else fa.FA_DTYPE_F32
    if varlen:
        T, H, d = inp.q.shape
        lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
        cu = torch.from_numpy(inp.cu_seqlens).to("cuda")
        max_len = int(np.max(np.diff(inp.cu_seqlens)))
        fa.fa_fwd_varlen(q, k, v, o, lse, cu, inp.cu_seqlens.size - 1, max_len, H, d, scale,
                         causal, code)
    else:
        B, H, N, d = inp.q.shape
        lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
        fa.fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, code)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("B,H,N", [(2, 64, 300), (1, 88, 260)],
                         ids=["16_heads_per_xcd", "11_heads_per_xcd"])
def test_many_heads_full(B, H, N):
    """128 (sequence, head) pairs give each XCD 16 heads, scheduled in groups
    of 8; 88 give it 11, which has no divisor up to 8 but 1.  Compared in
    full against the oracle."""
    d = 128
    inp = fa_inputs.make_fixed(B, H, N, d, "bf16", seed=7100 + H)
    o, lse = _run_nan_filled(inp, _scale(d), True, False)
    o_ref, lse_ref = oracle.attention(inp.q, inp.k, inp.v, _scale(d), True)
    gu.compare(o, o_ref, lse, lse_ref, "bf16", what=f"B{B} H{H} N{N}")


def test_many_heads_varlen_full():
    """8 packed sequences x 24 heads: 24 (sequence, head) pairs per XCD in
    groups of 8, ragged lengths, compared in full."""
    rng = np.random.default_rng(7200)
    lengths = [300, 1, 257, 64, 511, 129, 0, 200]
    inp = fa_inputs.make_varlen(lengths, 24, 64, "bf16", rng)
    o, lse = _run_nan_filled(inp, _scale(64), True, True)
    o_ref, lse_ref = oracle.attention_varlen(inp.q, inp.k, inp.v, inp.cu_seqlens, _scale(64), True)
    gu.compare(o, o_ref, lse, lse_ref, "bf16", what="varlen 8 x 24 heads")


def test_varlen_wide_token_rows():
    """512 heads of d = 128: a packed token row is 128 KB, so the staging
    offsets of a K/V tile reach ~16 MB (they are 32-bit byte offsets from the
    tile's base); 1024 (sequence, head) pairs put 128 on each XCD."""
    rng = np.random.default_rng(7300)
    lengths = [300, 70]
    inp = fa_inputs.make_varlen(lengths, 512, 128, "bf16", rng)
    o, lse = _run_nan_filled(inp, _scale(128), True, True)
    o_ref, lse_ref = oracle.attention_varlen(inp.q, inp.k, inp.v, inp.cu_seqlens, _scale(128), True)
    gu.compare(o, o_ref, lse, lse_ref, "bf16", what="varlen 2 x 512 heads")


# --- four-way key split over the waves of a 32-row block (small grids) -------

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N", [(1, 16, 1000), (1, 1, 129), (3, 1, 2049), (1, 2, 5000)],
                         ids=["b1h16n1000", "b1h1n129", "b3h1n2049", "b1h2n5000"])
def test_ksplit_fixed_full(B, H, N, causal, d):
    """Problems of at most 512 blocks of 32 query rows: the four waves of a
    block take every fourth key chunk and merge their partial softmax states
    at the end.  512 blocks exactly (B1 H16 N1000), a ragged last chunk, a
    one-row last block (N = 129, past the one-tile path) and 20 chunks per
    wave (N = 5000); compared in full, outputs NaN-filled beforehand."""
    inp = fa_inputs.make_fixed(B, H, N, d, "bf16", seed=7700 + N + H + d)
    o, lse = _run_nan_filled(inp, _scale(d), causal, False)
    o_ref, lse_ref = oracle.attention(inp.q, inp.k, inp.v, _scale(d), causal)
    gu.compare(o, o_ref, lse, lse_ref, "bf16", what=f"ksplit B{B} H{H} N{N} d{d}")


@pytest.mark.parametrize("d", [64, 128])
def test_ksplit_wide_scores(d):
    """Q and K x8 through the four-way split: the running maxima of the four
    waves differ by hundreds of log2 units when they are merged."""
    inp = fa_inputs.make_fixed(1, 3, 1500, d, "bf16", seed=7800 + d, qk_mult=8.0)
    for causal in (False, True):
        o, lse = _run_nan_filled(inp, _scale(d), causal, False)
        o_ref, lse_ref = oracle.attention(inp.q, inp.k, inp.v, _scale(d), causal)
        gu.compare(o, o_ref, lse, lse_ref, "bf16", what=f"ksplit x8 d{d} causal={causal}")


# --- key range split inside a workgroup (small grids at d = 64) ---------------

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N", [(1, 1, 4097), (2, 3, 777), (1, 2, 512), (1, 48, 1000)],
                         ids=["b1h1n4097", "b2h3n777", "b1h2n512", "b1h48n1000"])
def test_split_keys_fixed_full(B, H, N, causal, d):
    """Grids of at most 128 workgroups of 256 rows at d = 64 (256 when
    causal; N >= 512) split each workgroup's key range between its two wave
    groups and merge the halves (192 workgroups: split only when causal);
    compared in full, outputs NaN-filled beforehand.  (At d = 128 the split
    streams 32-key tiles.)"""
    inp = fa_inputs.make_fixed(B, H, N, d, "bf16", seed=7400 + N + H + d)
    o, lse = _run_nan_filled(inp, _scale(d), causal, False)
    o_ref, lse_ref = oracle.attention(inp.q, inp.k, inp.v, _scale(d), causal)
    gu.compare(o, o_ref, lse, lse_ref, "bf16", what=f"split B{B} H{H} N{N}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_split_keys_varlen_full(causal, d):
    """A packed batch small enough for the key split: ragged lengths, an
    empty sequence and a one-token one."""
    rng = np.random.default_rng(7500 + d)
    lengths = [1000, 3, 600, 0, 513, 1]
    inp = fa_inputs.make_varlen(lengths, 2, d, "bf16", rng)
    o, lse = _run_nan_filled(inp, _scale(d), causal, True)
    o_ref, lse_ref = oracle.attention_varlen(inp.q, inp.k, inp.v, inp.cu_seqlens, _scale(d),
                                             causal)
    gu.compare(o, o_ref, lse, lse_ref, "bf16", what="split varlen")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_one_tile_full(causal, d):
    """Packed bf16 batches whose sequences all fit one key tile (at most 128
    tokens) take the one-tile kernel: ragged lengths, an empty and a
    one-token sequence, compared in full."""
    rng = np.random.default_rng(7600 + d)
    lengths = [1, 0, 127, 128, 64, 33, 100, 17, 96]
    inp = fa_inputs.make_varlen(lengths, 3, d, "bf16", rng)
    o, lse = _run_nan_filled(inp, _scale(d), causal, True)
    o_ref, lse_ref = oracle.attention_varlen(inp.q, inp.k, inp.v, inp.cu_seqlens, _scale(d),
                                             causal)
    gu.compare(o, o_ref, lse, lse_ref, "bf16", what="varlen one-tile")


def test_varlen_max_seqlen_above_lengths():
    """max_seqlen is an upper bound: a looser one (here above the one-tile
    limit, so the streaming kernel runs) gives the same result."""
    rng = np.random.default_rng(7700)
    lengths = [50, 128, 7]
    inp = fa_inputs.make_varlen(lengths, 2, 64, "bf16", rng)
    o1, l1 = gu.run_varlen(inp, _scale(64), True)
    o2, l2 = gu.run_varlen(inp, _scale(64), True, max_seqlen=300)
    o_ref, lse_ref = oracle.attention_varlen(inp.q, inp.k, inp.v, inp.cu_seqlens, _scale(64), True)
    gu.compare(o1, o_ref, l1, lse_ref, "bf16", what="one-tile")
    gu.compare(o2, o_ref, l2, lse_ref, "bf16", what="streaming")
