"""fa_decode_fwd_noalloc, the decode entry point that allocates nothing (its
split partial results live in the library's static per-GPU scratch), called
through the C ABI and checked against fa_decode_fwd with a caller workspace:
the same plan and kernels, so the outputs must be bitwise equal; both are
also checked against the fp64 oracle.  Two calls in a row, the second on a
smaller problem, so the second reads a scratch array that still holds the
first call's partials.  The ABI-level rejection of oversized problems is in
test_abi.py (no GPU needed)."""
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


def _with_workspace(q, k, v, B, H, Nq, Nk, d, scale, causal, code, splits):
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device="cuda")
    need = fa.fa_decode_workspace_bytes(B, H, Nq, Nk, d, splits)
    ws = torch.full((max(need, 16),), 0xFF, dtype=torch.uint8, device="cuda")
    fa.fa_decode_fwd(q, k, v, o, lse, ws, need, B, H, Nq, Nk, d, scale, causal, code, splits)
    return o, lse


def _noalloc(q, k, v, B, H, Nq, Nk, d, scale, causal, code, splits):
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device="cuda")
    fa.fa_decode_fwd_noalloc(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, code, splits)
    return o, lse


# (B, H, Nq, Nk, d, dtype, causal, num_splits): the first call fills much of
# the scratch (4 MiB of partials), the second is smaller
CALLS = [(4, 32, 4, 16384, 128, "bf16", True, 0),
         (2, 8, 1, 3000, 64, "f32", False, 5)]


def test_noalloc_matches_workspace_entry_point_twice():
    for B, H, Nq, Nk, d, dtype, causal, splits in CALLS:
        print(f"case noalloc B={B} H={H} Nq={Nq} Nk={Nk} d={d} {dtype} causal={causal} "
              f"splits={splits}", flush=True)
        need = fa.fa_decode_workspace_bytes(B, H, Nq, Nk, d, splits)
        assert 0 < need <= fa.FA_DECODE_SCRATCH_BYTES
        inp = fa_inputs.make_decode(B, H, Nq, Nk, d, dtype, seed=4100 + Nk + d)
        scale = float(np.float32(1.0 / math.sqrt(d)))
        q, k, v = gu.upload(inp)
        code = fa.FA_DTYPE_BF16 if dtype == "bf16" else fa.FA_DTYPE_F32
        o1, l1 = _noalloc(q, k, v, B, H, Nq, Nk, d, scale, causal, code, splits)
        o2, l2 = _with_workspace(q, k, v, B, H, Nq, Nk, d, scale, causal, code, splits)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), "noalloc output differs from the workspace entry point"
        assert torch.equal(l1, l2), "noalloc lse differs from the workspace entry point"
        o_ref, lse_ref = oracle.attention_decode(inp.q, inp.k, inp.v, scale, causal)
        gu.compare(o1, o_ref, l1, lse_ref, dtype, what=f"noalloc B{B} H{H} Nq{Nq} Nk{Nk}")
