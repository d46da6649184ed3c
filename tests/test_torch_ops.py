"""The PyTorch operators torch.ops.fa355.fwd / fwd_varlen / decode.

CPU: registration, the fake (meta) implementations' output shapes and
dtypes, and argument validation.  GPU: the operators return exactly what
the direct C-ABI call returns (they only allocate and enqueue), also inside
a torch.compile graph, pass torch.library.opcheck, and agree with the fp64
oracle.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import flashattention_forward_07_amd as fa  # noqa: E402
import flashattention_forward_07_amd.torch_ops  # noqa: E402,F401  (registers the ops)


def test_ops_are_registered():
    assert hasattr(torch.ops.fa355, "fwd")
    assert hasattr(torch.ops.fa355, "fwd_varlen")
    assert hasattr(torch.ops.fa355, "decode")


def test_fake_shapes_decode():
    q = torch.empty(2, 3, 4, 128, dtype=torch.bfloat16, device="meta")
    k = torch.empty(2, 3, 1000, 128, dtype=torch.bfloat16, device="meta")
    o, lse = torch.ops.fa355.decode(q, k, k, True, None, 0)
    assert o.shape == q.shape and lse.shape == (2, 3, 4) and lse.dtype == torch.float32
    with pytest.raises(ValueError):  # d differs
        torch.ops.fa355.decode(q, k[..., :64], k[..., :64], False, None, 0)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_fake_shapes_fixed(dtype):
    q = torch.empty(2, 3, 100, 64, dtype=dtype, device="meta")
    o, lse = torch.ops.fa355.fwd(q, q, q, True, None)
    assert o.shape == q.shape and o.dtype == dtype
    assert lse.shape == (2, 3, 100) and lse.dtype == torch.float32


def test_fake_shapes_varlen():
    from torch._subclasses.fake_tensor import FakeTensorMode
    with FakeTensorMode():
        q = torch.empty(50, 4, 128, dtype=torch.bfloat16)
        cu = torch.empty(3, dtype=torch.int32)
        o, lse = torch.ops.fa355.fwd_varlen(q, q, q, cu, 30, True, None)
        assert o.shape == (50, 4, 128) and lse.shape == (50, 4)


def test_validation_in_fake_mode():
    q = torch.empty(1, 2, 16, 64, dtype=torch.bfloat16, device="meta")
    k = torch.empty(1, 2, 17, 64, dtype=torch.bfloat16, device="meta")
    with pytest.raises(ValueError):
        torch.ops.fa355.fwd(q, k, q, False, None)
    with pytest.raises(ValueError):
        torch.ops.fa355.fwd(q[0], q[0], q[0], False, None)
    cu = torch.empty(3, dtype=torch.int64, device="meta")
    qv = torch.empty(8, 2, 64, dtype=torch.bfloat16, device="meta")
    with pytest.raises(ValueError):
        torch.ops.fa355.fwd_varlen(qv, qv, qv, cu, 8, False, None)


gpu = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():  # pragma: no cover
        pytest.skip("needs a GPU")


@gpu
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("causal", [False, True])
def test_op_equals_direct_call(dtype, causal):
    _need_gpu()
    print(f"case dtype={dtype} causal={causal}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(11)
    q, k, v = (torch.randn(2, 3, 257, 128, generator=g).to(dtype).cuda() for _ in range(3))
    o, lse = torch.ops.fa355.fwd(q, k, v, causal, None)
    o2 = torch.empty_like(q)
    lse2 = torch.empty(2, 3, 257, dtype=torch.float32, device="cuda")
    fa.fa_fwd(q, k, v, o2, lse2, 2, 3, 257, 128, 1.0 / math.sqrt(128), causal,
              fa.FA_DTYPE_BF16 if dtype == torch.bfloat16 else fa.FA_DTYPE_F32)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


@gpu
def test_op_in_compiled_graph():
    _need_gpu()
    g = torch.Generator(device="cpu").manual_seed(12)
    q, k, v = (torch.randn(1, 4, 300, 64, generator=g).to(torch.bfloat16).cuda() for _ in range(3))

    def f(q, k, v):  # exact elementwise ops around the operator
        o, lse = torch.ops.fa355.fwd(q * 1.0, k, v, True, 0.125)
        return o * 2.0, lse + 0.0

    ref = f(q, k, v)
    got = torch.compile(f, fullgraph=True)(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])


@gpu
def test_opcheck():
    _need_gpu()
    g = torch.Generator(device="cpu").manual_seed(13)
    q, k, v = (torch.randn(1, 2, 130, 64, generator=g).to(torch.bfloat16).cuda() for _ in range(3))
    torch.library.opcheck(torch.ops.fa355.fwd.default, (q, k, v, True, None),
                          test_utils=("test_schema", "test_faketensor"))
    T = 70
    qv, kv, vv = (torch.randn(T, 2, 64, generator=g).to(torch.bfloat16).cuda() for _ in range(3))
    cu = torch.tensor([0, 30, 70], dtype=torch.int32, device="cuda")
    torch.library.opcheck(torch.ops.fa355.fwd_varlen.default, (qv, kv, vv, cu, 40, True, None),
                          test_utils=("test_schema", "test_faketensor"))


@gpu
def test_op_matches_oracle():
    _need_gpu()
    import fa_inputs
    import oracle
    from tests import gpu_util as gu
    inp = fa_inputs.make_fixed(1, 2, 190, 64, "bf16", seed=1234)
    q, k, v = gu.upload(inp)
    o, lse = torch.ops.fa355.fwd(q, k, v, True, None)
    torch.cuda.synchronize()
    scale = float(np.float32(1 / math.sqrt(64)))
    o_ref, lse_ref = oracle.attention(inp.q, inp.k, inp.v, scale, True)
    gu.compare(o, o_ref, lse, lse_ref, "bf16", what="op")


@gpu
def test_decode_op_equals_direct_call_and_oracle():
    _need_gpu()
    import fa_inputs
    import oracle
    from tests import gpu_util as gu
    inp = fa_inputs.make_decode(2, 2, 3, 700, 128, "bf16", seed=4321)
    q, k, v = gu.upload(inp)
    o, lse = torch.ops.fa355.decode(q, k, v, True, None, 3)
    o2 = torch.empty_like(q)
    lse2 = torch.empty(2, 2, 3, dtype=torch.float32, device="cuda")
    need = fa.fa_decode_workspace_bytes(2, 2, 3, 700, 128, 3)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    scale = float(np.float32(1 / math.sqrt(128)))
    fa.fa_decode_fwd(q, k, v, o2, lse2, ws, need, 2, 2, 3, 700, 128, 1 / math.sqrt(128), True,
                     fa.FA_DTYPE_BF16, 3)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    o_ref, lse_ref = oracle.attention_decode(inp.q, inp.k, inp.v, scale, True)
    gu.compare(o, o_ref, lse, lse_ref, "bf16", what="decode op")
    torch.library.opcheck(torch.ops.fa355.decode.default, (q, k, v, True, None, 0),
                          test_utils=("test_schema", "test_faketensor"))
