"""GPU parity at the largest sizes the tests afford: one very long sequence
for the fused kernel (a power of two and a ragged length, bf16, causal and
not), a million-key decode step, and a packed batch
of many short sequences.  The oracle computes sampled rows one by one
(every tile edge of the sequence plus random rows), which it does in
seconds at any length.
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


@pytest.mark.parametrize("N", [65536, 100003])
@pytest.mark.parametrize("causal", [False, True])
def test_long_sequence(N, causal):
    """One head of 64K / 100K tokens, d = 128, bf16: the key loop runs
    1000+ tiles, so a drift in the running max or sum would show."""
    B, H, d = 1, 2, 128
    print(f"case long N={N} causal={causal}", flush=True)
    inp = fa_inputs.make_fixed(B, H, N, d, "bf16", seed=6000 + N % 1000)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o, lse = gu.run_fixed(inp, scale, causal)
    rows = gu.sample_rows(B, H, N, count=256, seed=6100)
    o_ref, lse_ref = oracle.attention_rows(inp.q, inp.k, inp.v, scale, causal, rows)
    idx = torch.from_numpy(rows).cuda()
    gu.compare(gu.host(o.reshape(-1, d)[idx]), o_ref, gu.host(lse.reshape(-1)[idx]), lse_ref,
               "bf16", what=f"long N={N}")


def test_decode_million_keys():
    """A decode step against 2^20 cached keys (64 key ranges of 16K keys),
    4 causal queries."""
    B, H, Nq, Nk, d = 1, 2, 4, 1 << 20, 128
    print("case decode 1M keys", flush=True)
    inp = fa_inputs.make_decode(B, H, Nq, Nk, d, "bf16", seed=6200)
    q, k, v = gu.upload(inp)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    o = torch.full_like(q, float("nan"))
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    need = fa.fa_decode_workspace_bytes(B, H, Nq, Nk, d, 64)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    fa.fa_decode_fwd(q, k, v, o, lse, ws, need, B, H, Nq, Nk, d, scale, True, fa.FA_DTYPE_BF16, 64)
    torch.cuda.synchronize()
    assert fa.fa_decode_num_splits(B, H, Nq, Nk, 64) == 64
    o_ref, lse_ref = oracle.attention_decode(inp.q, inp.k, inp.v, scale, True)
    gu.compare(o, o_ref, lse, lse_ref, "bf16", what="decode 1M")


def test_varlen_many_short_sequences():
    """2000 packed sequences of 1..40 tokens (most shorter than one query
    tile), causal, compared in full."""
    rng = np.random.default_rng(6300)
    lengths = rng.integers(1, 40, size=2000, endpoint=True)
    inp = fa_inputs.make_varlen(lengths, 4, 64, "bf16", rng)
    scale = float(np.float32(1.0 / math.sqrt(64)))
    print(f"case varlen {lengths.size} seqs, {int(lengths.sum())} tokens", flush=True)
    o, lse = gu.run_varlen(inp, scale, True)
    o_ref, lse_ref = oracle.attention_varlen(inp.q, inp.k, inp.v, inp.cu_seqlens, scale, True)
    gu.compare(o, o_ref, lse, lse_ref, "bf16", what="varlen many short")
