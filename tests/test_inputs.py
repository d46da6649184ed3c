"""The seeded input generator: determinism, shapes and bf16 rounding."""
import numpy as np
import torch

import fa_inputs


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 10,
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40, -1e-40,
                  np.inf, -np.inf], np.float32),
        # exact ties: halfway between two bf16 values
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
    ])
    bits = fa_inputs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    back = fa_inputs.bf16_bits_to_f32(bits)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generator_is_deterministic_and_shaped():
    a = fa_inputs.make_fixed(1, 2, 33, 64, "bf16", 123)
    b = fa_inputs.make_fixed(1, 2, 33, 64, "bf16", 123)
    assert a.q.shape == (1, 2, 33, 64)
    for x, y in zip((a.q, a.k, a.v, a.q_bits), (b.q, b.k, b.v, b.q_bits)):
        assert np.array_equal(x, y)
    assert np.array_equal(fa_inputs.bf16_bits_to_f32(a.q_bits), a.q)
    c = fa_inputs.make_fixed(1, 2, 33, 64, "bf16", 124)
    assert not np.array_equal(a.q, c.q)


def test_workloads():
    w = fa_inputs.WORKLOADS
    assert [x.dtype for x in w] == ["f32", "bf16", "bf16", "bf16", "bf16"]
    assert fa_inputs.HEADLINE.B == 4 and fa_inputs.HEADLINE.H == 32
    assert fa_inputs.HEADLINE.N == 4096 and fa_inputs.HEADLINE.d == 128
    assert fa_inputs.HEADLINE.causal
    vl = w[4]
    lengths = fa_inputs.workload_lengths(vl)
    assert lengths.size == 16 and lengths.min() >= 1 and lengths.max() <= 8192
    assert w[0].scale == np.float32(0.125)


def test_varlen_generator_small():
    rng = np.random.default_rng(9)
    inp = fa_inputs.make_varlen([3, 1, 5], 2, 8, "bf16", rng, qk_mult=8.0)
    assert inp.q.shape == (9, 2, 8)
    assert list(inp.cu_seqlens) == [0, 3, 4, 9]
    assert inp.cu_seqlens.dtype == np.int32
    # x8 is exact: the rounded values are multiples of 8 times bf16 values
    assert np.array_equal(fa_inputs.round_bf16(inp.q / 8), inp.q / 8)
