"""GPU parity of the one-tile paths that fa_fwd takes for sequences of
N <= 128 (a whole sequence in one key tile; bf16: 4 heads per workgroup when
N <= 32, 2 when N <= 64; fp32: 16 queries per workgroup): every length
around the block edges, head counts that leave the last workgroup partly
filled, both dtypes and head dimensions, with and without the causal mask,
compared in full with the fp64 oracle.
The outputs start as NaN so a row the kernel misses shows.
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

LENGTHS = [1, 2, 7, 16, 31, 32, 33, 63, 64, 65, 96, 100, 127, 128]


def _run(inp, scale, causal):
    q, k, v = gu.upload(inp)
    B, H, N, d = inp.q.shape
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    code = fa.FA_DTYPE_BF16 if inp.dtype == "bf16" else fa.FA_DTYPE_F32
    fa.fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, code)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", LENGTHS)
def test_one_tile_lengths(dtype, d, causal, N):
    B, H = 3, 3  # 9 heads: the last bf16 workgroup holds 1 of 4 (N <= 32) or 1 of 2 (N <= 64)
    print(f"case one-tile {dtype} d={d} causal={causal} B={B} H={H} N={N}", flush=True)
    inp = fa_inputs.make_fixed(B, H, N, d, dtype, seed=5000 + N + d)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = _run(inp, scale, causal)
    o_ref, lse_ref = oracle.attention(inp.q, inp.k, inp.v, scale, causal)
    gu.compare(o, o_ref, lse, lse_ref, dtype, what=f"one-tile {dtype} N={N}")


@pytest.mark.parametrize("N", [16, 64, 128])
def test_one_tile_many_heads(N):
    """Many short sequences: 4099 heads (not a multiple of the heads per
    workgroup), sampled heads compared in full."""
    B, H, d = 4099, 1, 64
    print(f"case one-tile many heads N={N}", flush=True)
    inp = fa_inputs.make_fixed(B, H, N, d, "bf16", seed=5100 + N)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = _run(inp, scale, True)
    pick = np.array([0, 1, 2, 3, 4, 5, 1024, 2047, 4096, 4097, 4098])
    o_ref, lse_ref = oracle.attention(inp.q[pick], inp.k[pick], inp.v[pick], scale, True)
    idx = torch.from_numpy(pick).cuda()
    gu.compare(gu.host(o[idx]), o_ref, gu.host(lse[idx]), lse_ref, "bf16", what=f"heads N={N}")
    assert torch.isfinite(o.float()).all().item() and torch.isfinite(lse).all().item()


def test_one_tile_and_general_kernel_meet_at_128():
    """N = 128 runs the one-tile kernel and N = 129 the general one; both
    match the oracle on the same data (the first 128 keys' problem is a
    prefix of the second under the causal mask)."""
    d = 128
    inp = fa_inputs.make_fixed(2, 2, 129, d, "bf16", seed=5200)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o129, l129 = _run(inp, scale, True)
    sub = fa_inputs.Inputs(inp.q[:, :, :128].copy(), inp.k[:, :, :128].copy(),
                           inp.v[:, :, :128].copy(), "bf16", None,
                           inp.q_bits[:, :, :128].copy(), inp.k_bits[:, :, :128].copy(),
                           inp.v_bits[:, :, :128].copy())
    o128, l128 = _run(sub, scale, True)
    o_ref, lse_ref = oracle.attention(inp.q, inp.k, inp.v, scale, True)
    gu.compare(o129, o_ref, l129, lse_ref, "bf16", what="N=129")
    gu.compare(o128, o_ref[:, :, :128], l128, lse_ref[:, :, :128], "bf16", what="N=128")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [97, 100, 128])
def test_one_tile_staged_ahead_full(d, causal, N):
    """Heads of 97..128 rows, more of them than the GPU holds workgroups at
    once (605 > 2 per compute unit at d = 64, 1 at d = 128): the one-tile
    kernel that stages the next heads while it computes. Every head is
    compared in full; the outputs start as NaN."""
    B, H = 5, 121
    print(f"case one-tile staged d={d} causal={causal} B={B} H={H} N={N}", flush=True)
    inp = fa_inputs.make_fixed(B, H, N, d, "bf16", seed=5300 + N + d + int(causal))
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = _run(inp, scale, causal)
    o_ref, lse_ref = oracle.attention(inp.q, inp.k, inp.v, scale, causal)
    gu.compare(o, o_ref, lse, lse_ref, "bf16", what=f"staged N={N}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_one_tile_staged_ahead_varlen_full(d, causal):
    """A packed batch of 700 sequences x 2 heads, lengths 0..128 with the
    longest 128 (so the staged one-tile kernel runs), every row compared."""
    rng = np.random.default_rng(5400 + d + int(causal))
    lengths = [int(x) for x in rng.integers(0, 129, size=700)]
    lengths[0], lengths[1], lengths[2] = 128, 0, 1
    print(f"case one-tile staged varlen d={d} causal={causal}", flush=True)
    inp = fa_inputs.make_varlen(lengths, 2, d, "bf16", rng)
    q, k, v = gu.upload(inp)
    T = q.shape[0]
    o = torch.full_like(q, float("nan"))
    lse = torch.full((T, 2), float("nan"), dtype=torch.float32, device="cuda")
    scale = float(np.float32(1.0 / math.sqrt(d)))
    cu = torch.from_numpy(inp.cu_seqlens).cuda()
    fa.fa_fwd_varlen(q, k, v, o, lse, cu, len(lengths), max(lengths), 2, d, scale, causal,
                     fa.FA_DTYPE_BF16)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_varlen(inp.q, inp.k, inp.v, inp.cu_seqlens, scale, causal)
    gu.compare(o, o_ref, lse, lse_ref, "bf16", what="staged varlen")


@pytest.mark.parametrize("d", [64, 128])
def test_one_tile_staged_ahead_without_lse(d):
    """The staged one-tile kernel with lse = NULL: O still matches in full."""
    B, H, N = 3, 200, 120
    inp = fa_inputs.make_fixed(B, H, N, d, "bf16", seed=5500 + d)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    q, k, v = gu.upload(inp)
    o = torch.full_like(q, float("nan"))
    fa.fa_fwd(q, k, v, o, None, B, H, N, d, scale, True, fa.FA_DTYPE_BF16)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(inp.q, inp.k, inp.v, scale, True)
    gu.compare(o, o_ref, None, None, "bf16", what="staged, no lse")
