"""Pins of the oracle's decode-shaped entry (Nq queries against Nk keys).

The queries are read as the newest Nq positions of an Nk-long sequence, so
with the causal mask query i (0-based among the Nq) sees keys
0 .. Nk - Nq + i ("Mini FlashAttention", section 1: the mask hides later
tokens, and it is what autoregressive decoding uses).  Each pin ties that
reading to something computed another way: the already-pinned square entry,
a closed form over the visible keys, or a property of the definition.
"""
import math

import numpy as np
import pytest

import oracle


def _rand(shape, seed, mult=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape) * mult).astype(np.float32)


@pytest.mark.parametrize("causal", [False, True])
def test_decode_square_equals_fwd(causal):
    """Nq = Nk is the square problem."""
    B, H, N, d = 2, 3, 45, 16
    q, k, v = _rand((B, H, N, d), 1), _rand((B, H, N, d), 2), _rand((B, H, N, d), 3)
    o1, l1 = oracle.attention(q, k, v, 0.25, causal)
    o2, l2 = oracle.attention_decode(q, k, v, 0.25, causal)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


@pytest.mark.parametrize("nq", [1, 3, 17])
def test_decode_is_the_last_rows_of_the_square_problem(nq):
    """Causal decode of the newest nq queries equals the last nq rows of the
    square causal problem over the whole sequence."""
    nk, d = 50, 8
    qf, k, v = _rand((nk, d), 11), _rand((nk, d), 12), _rand((nk, d), 13)
    o_sq, l_sq = oracle.attention(qf, k, v, 0.3, causal=True)
    o, lse = oracle.attention_decode(qf[nk - nq:], k, v, 0.3, causal=True)
    np.testing.assert_allclose(o, o_sq[nk - nq:], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, l_sq[nk - nq:], rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(1, 9), (4, 9), (9, 9), (12, 9)])
def test_decode_zero_queries_give_visible_means(causal, nq, nk):
    """With q = 0 every visible score is 0: O is the mean of the visible V
    rows and lse = ln(count); a query that sees no key gets O = 0 and
    lse = -inf.  The count is Nk, or Nk - Nq + i + 1 under the mask."""
    d = 5
    k, v = _rand((nk, d), 21), _rand((nk, d), 22)
    q = np.zeros((nq, d), np.float32)
    o, lse = oracle.attention_decode(q, k, v, 0.7, causal)
    v64 = v.astype(np.float64)
    for i in range(nq):
        m = min(nk, max(0, nk - nq + i + 1)) if causal else nk
        if m == 0:
            assert np.all(o[i] == 0.0) and lse[i] == -math.inf
        else:
            np.testing.assert_allclose(o[i], v64[:m].mean(axis=0), rtol=0, atol=1e-14)
            assert abs(lse[i] - math.log(m)) <= 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_decode_batch_is_independent_heads(causal):
    """Each (batch, head) of a batched call equals that head alone, whose
    causal rows are in turn the last rows of its square problem."""
    B, H, nq, nk, d = 2, 3, 4, 11, 8
    q, k, v = _rand((B, H, nq, d), 61), _rand((B, H, nk, d), 62), _rand((B, H, nk, d), 63)
    o, lse = oracle.attention_decode(q, k, v, 0.4, causal)
    for b in range(B):
        for h in range(H):
            qf = np.concatenate([np.zeros((nk - nq, d), np.float32), q[b, h]])
            o1, l1 = oracle.attention(qf, k[b, h], v[b, h], 0.4, causal)
            np.testing.assert_allclose(o[b, h], o1[nk - nq:], rtol=0, atol=1e-14)
            np.testing.assert_allclose(lse[b, h], l1[nk - nq:], rtol=0, atol=1e-14)


def test_decode_single_query_sees_everything():
    """One query is the newest position: the mask hides nothing."""
    q, k, v = _rand((1, 16), 31), _rand((70, 16), 32), _rand((70, 16), 33)
    o1, l1 = oracle.attention_decode(q, k, v, 0.25, causal=False)
    o2, l2 = oracle.attention_decode(q, k, v, 0.25, causal=True)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_decode_split_keys_merge_exactly():
    """Attention over the union of two disjoint key sets is the lse-weighted
    mix of the attention over each set (the identity split-KV decoding rests
    on): lse = ln(e^lse1 + e^lse2), O = (e^lse1 O1 + e^lse2 O2) / e^lse."""
    q, k, v = _rand((3, 8), 41, 2.0), _rand((40, 8), 42, 2.0), _rand((40, 8), 43)
    o, lse = oracle.attention_decode(q, k, v, 0.5)
    o1, l1 = oracle.attention_decode(q, k[:13], v[:13], 0.5)
    o2, l2 = oracle.attention_decode(q, k[13:], v[13:], 0.5)
    mx = np.maximum(l1, l2)
    w1, w2 = np.exp(l1 - mx), np.exp(l2 - mx)
    np.testing.assert_allclose(lse, mx + np.log(w1 + w2), rtol=0, atol=1e-13)
    np.testing.assert_allclose(o, (w1[:, None] * o1 + w2[:, None] * o2) / (w1 + w2)[:, None],
                               rtol=0, atol=1e-13)


def test_decode_bad_arguments_are_rejected():
    q, k = _rand((1, 2, 3, 8), 51), _rand((1, 2, 5, 8), 52)
    with pytest.raises(ValueError):
        oracle.attention_decode(q, k, k[..., :4], 0.5)
    with pytest.raises(ValueError):
        oracle.attention_decode(q, k[:, :1], k[:, :1], 0.5)
