"""Pins of the fp64 oracle to facts fixed outside the oracle itself.

Each test ties the oracle to something it does not compute the same way:
hand-derived worked examples, closed forms, a library routine for a special
case, 50-digit brute force, invariants of the definition, and the chunked
online recurrence of the page "Mini FlashAttention", section 4, which must
equal the three-pass result for every chunk size.  A dropped term, a wrong
sign or index, a missing max-shift or a transposed operand fails at least
one of them.
"""
import decimal
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _rand(shape, seed, mult=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape) * mult).astype(np.float32)


def _qkv(n, d, seed, mult=1.0):
    return (_rand((n, d), seed, mult), _rand((n, d), seed + 1, mult),
            _rand((n, d), seed + 2))


def _eval_closed_form(expr):
    # Expressions over e, exp and ln only (see the fixture's "about").
    return float(eval(expr, {"__builtins__": {}},
                      {"e": math.e, "exp": math.exp, "ln": math.log}))


# --- hand-derived worked examples (definition: "Mini FlashAttention" s.1) --

@pytest.mark.parametrize("causal", [False, True])
def test_hand_worked_examples(causal):
    spec = json.load(open(GOLDEN))
    for ex in spec["examples"]:
        q = np.array(ex["q"], np.float32)
        k = np.array(ex["k"], np.float32)
        v = np.array(ex["v"], np.float32)
        want = ex["causal" if causal else "noncausal"]
        o, lse = oracle.attention(q, k, v, ex["scale"], causal)
        o_ref = np.array([[_eval_closed_form(x) for x in row] for row in want["o"]])
        lse_ref = np.array([_eval_closed_form(x) for x in want["lse"]])
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-14, err_msg=ex["name"])
        np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-14, err_msg=ex["name"])


# --- the chunked online recurrence equals three-pass for every chunk -------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d,seed", [(37, 8, 11), (50, 16, 12), (64, 4, 13)])
def test_online_recurrence_equals_three_pass(causal, n, d, seed):
    q, k, v = _qkv(n, d, seed, mult=2.0)
    scale = 1.0 / math.sqrt(d)
    o3, l3 = oracle.attention(q, k, v, scale, causal)
    for chunk in list(range(1, n + 1)) + [n + 5]:
        oc, lc = oracle.online(q, k, v, scale, causal, chunk)
        assert np.max(np.abs(oc - o3)) <= 1e-12, chunk
        assert np.max(np.abs(lc - l3)) <= 1e-12, chunk


# --- softmax special case against a library routine ------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_identity_values_give_softmax_rows(causal):
    # With V[j] = e_j (N == d) each output row is the row of softmax weights.
    n = d = 24
    q, k, _ = _qkv(n, d, 21, mult=1.5)
    v = np.eye(n, dtype=np.float32)
    scale = 0.3
    o, lse = oracle.attention(q, k, v, scale, causal)
    s = scale * (q.astype(np.float64) @ k.astype(np.float64).T)
    if causal:
        s = np.where(np.tril(np.ones((n, n), bool)), s, -np.inf)
    np.testing.assert_allclose(o, scipy.special.softmax(s, axis=1), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(s, axis=1), rtol=0, atol=1e-13)
    # softmax rows are probabilities ("Mini FlashAttention" s.1)
    assert np.max(np.abs(o.sum(axis=1) - 1.0)) <= 1e-13
    assert np.all(o >= 0)
    if causal:
        assert np.all(o[np.triu_indices(n, 1)] == 0.0)


# --- closed forms ------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_single_token_gives_v(causal):
    q, k, v = _qkv(1, 64, 31)
    o, lse = oracle.attention(q, k, v, 0.125, causal)
    assert np.array_equal(o, v.astype(np.float64))
    assert abs(lse[0] - 0.125 * float(q[0].astype(np.float64) @ k[0].astype(np.float64))) <= 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_give_constant_output(causal):
    n, d = 45, 16
    q, k, _ = _qkv(n, d, 41, mult=3.0)
    c = _rand((d,), 44)
    v = np.tile(c, (n, 1))
    o, _ = oracle.attention(q, k, v, 0.25, causal)
    assert np.max(np.abs(o - c.astype(np.float64))) <= 1e-14 * max(1.0, np.abs(c).max()) * 4


def test_causal_row_zero():
    q, k, v = _qkv(33, 32, 51)
    o, lse = oracle.attention(q, k, v, 0.2, causal=True)
    assert np.array_equal(o[0], v[0].astype(np.float64))
    assert abs(lse[0] - 0.2 * float(q[0].astype(np.float64) @ k[0].astype(np.float64))) <= 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_give_prefix_means(causal):
    n, d = 77, 8
    _, k, v = _qkv(n, d, 61)
    q = np.zeros((n, d), np.float32)
    o, lse = oracle.attention(q, k, v, 0.5, causal)
    v64 = v.astype(np.float64)
    for i in range(n):
        m = i + 1 if causal else n
        np.testing.assert_allclose(o[i], v64[:m].mean(axis=0), rtol=0, atol=1e-14)
        assert abs(lse[i] - math.log(m)) <= 1e-14


def test_permutation_equivariance_noncausal():
    n, d = 40, 16
    q, k, v = _qkv(n, d, 71)
    o, lse = oracle.attention(q, k, v, 0.25, False)
    perm = np.random.default_rng(72).permutation(n)
    o2, lse2 = oracle.attention(q, k[perm], v[perm], 0.25, False)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-14)
    o3, lse3 = oracle.attention(q[perm], k, v, 0.25, False)
    assert np.array_equal(o3, o[perm]) and np.array_equal(lse3, lse[perm])


def test_large_margin_rows_pick_the_argmax_value():
    # Scores far apart: the softmax is one-hot to within exp(-margin).
    n, d = 20, 16
    rng = np.random.default_rng(81)
    k = rng.standard_normal((n, d)).astype(np.float32)
    target = rng.permutation(n)
    q = (24.0 * k[target]).astype(np.float32)
    v = rng.standard_normal((n, d)).astype(np.float32)
    scale = 0.5
    o, lse = oracle.attention(q, k, v, scale, False)
    s = scale * (q.astype(np.float64) @ k.astype(np.float64).T)
    top = np.argmax(s, axis=1)
    srt = np.sort(s, axis=1)
    margin = srt[:, -1] - srt[:, -2]
    assert margin.min() > 20
    for i in range(n):
        bound = n * math.exp(-margin[i]) * np.abs(v).max() * 2
        assert np.max(np.abs(o[i] - v[top[i]])) <= bound + 1e-15
        assert abs(lse[i] - srt[i, -1]) <= n * math.exp(-margin[i]) + 1e-13


# --- 50-digit brute force, no max subtraction -----------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_4x4_decimal(causal):
    decimal.getcontext().prec = 50
    D = decimal.Decimal
    n = d = 4
    q, k, v = _qkv(n, d, 91, mult=2.0)
    scale = float(np.float32(0.5))
    o, lse = oracle.attention(q, k, v, scale, causal)
    for i in range(n):
        keys = range(i + 1) if causal else range(n)
        w = []
        for j in keys:
            s = sum(D(float(q[i, c])) * D(float(k[j, c])) for c in range(d)) * D(scale)
            w.append(s.exp())
        tot = sum(w)
        for c in range(d):
            want = sum(wj * D(float(v[j, c])) for wj, j in zip(w, keys)) / tot
            assert abs(o[i, c] - float(want)) <= 1e-14
        assert abs(lse[i] - float(tot.ln())) <= 1e-14


# --- internal consistency of the oracle's entry points ---------------------

def test_rows_entry_matches_full():
    B, H, N, d = 2, 3, 29, 8
    rng = np.random.default_rng(101)
    q, k, v = (rng.standard_normal((B, H, N, d)).astype(np.float32) for _ in range(3))
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, 0.3, causal)
        rows = np.array([0, 5, N - 1, N, 2 * N + 7, B * H * N - 1])
        orr, lr = oracle.attention_rows(q, k, v, 0.3, causal, rows)
        assert np.array_equal(orr, o.reshape(-1, d)[rows])
        assert np.array_equal(lr, lse.reshape(-1)[rows])


def test_varlen_equals_per_sequence_heads():
    H, d = 3, 8
    lengths = [5, 1, 17, 9]
    rng = np.random.default_rng(111)
    T = sum(lengths)
    q, k, v = (rng.standard_normal((T, H, d)).astype(np.float32) for _ in range(3))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    for causal in (False, True):
        o, lse = oracle.attention_varlen(q, k, v, cu, 0.4, causal)
        for s in range(len(lengths)):
            a, b = cu[s], cu[s + 1]
            for h in range(H):
                oh, lh = oracle.attention(q[a:b, h], k[a:b, h], v[a:b, h], 0.4, causal)
                assert np.array_equal(o[a:b, h], oh)
                assert np.array_equal(lse[a:b, h], lh)
        rows = np.array([0, 3 * H + 1, (T - 1) * H + 2, 6 * H])
        orr, lr = oracle.attention_varlen_rows(q, k, v, cu, 0.4, causal, rows)
        assert np.array_equal(orr, o.reshape(-1, d)[rows])
        assert np.array_equal(lr, lse.reshape(-1)[rows])


def test_bad_arguments_are_rejected():
    q = np.zeros((4, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.attention_varlen(q[:, None], q[:, None], q[:, None],
                                np.array([0, 3, 2], np.int32), 1.0)
    with pytest.raises(ValueError):
        oracle.attention_rows(q[None, None], q[None, None], q[None, None], 1.0,
                              False, [4])
