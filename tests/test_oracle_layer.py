"""Pins for the oracle's layer prologue: the safe decay gate (EDA paper Eqs.
(14)-(15); slides frame on the safe decay parameterization), the L2
normalisation of q, k, e (paper Fig. 1) and the grouping of value heads over
key heads (paper appendix model table: 8/16 and 16/32 heads).

Each test checks oracle.eda_ref_safe_gate / eda_ref_l2norm /
eda_ref_fwd_layer against a hand-computed value, a limit or bound the pages
state, or an explicit per-head brute force, not against a retyped copy of
the same formula.
"""
import math

import numpy as np
import pytest

import oracle
from eda_inputs import make_layer_inputs


def test_softplus_identities():
    x = np.linspace(-30.0, 30.0, 121)
    sp = oracle.softplus(x)
    assert np.allclose(sp - oracle.softplus(-x), x, rtol=0, atol=1e-12)   # softplus(x) - softplus(-x) = x
    assert oracle.softplus(0.0) == pytest.approx(math.log(2.0), abs=1e-15)
    assert np.all(sp > 0) and np.all(np.diff(sp) > 0)


@pytest.mark.parametrize("a,b,A,want", [
    # a + b = 0: Delta = ln 2; A = 5: g = -5 + 5 * 2^-1 = -2.5
    (0.0, 0.0, 5.0, math.exp(-2.5)),
    # A = 5 ln 2 / ln 2 ... Delta = ln 2 again with a + b = 0 split as 1 + (-1); A = 10: g = -5 + 5/4
    (1.0, -1.0, 10.0, math.exp(-3.75)),
    # Delta = ln(1 + e^{ln 3}) = ln 4 = 2 ln 2 with a + b = ln 3; A = 5: g = -5 + 5/4
    (math.log(3.0), 0.0, 5.0, math.exp(-3.75)),
])
def test_safe_gate_hand_values(a, b, A, want):
    got = oracle.eda_ref_safe_gate(np.array([[a]]), np.array([[math.log(A)]]), np.array([[b]]))
    assert got.shape == (1, 1)
    assert got[0, 0] == pytest.approx(want, rel=1e-14)


def test_safe_gate_bounds_and_limits():
    # the pages: with l = -5, e^-5 < alpha <= 1; large inputs saturate at the floor
    rng = np.random.default_rng(0)
    a = rng.uniform(-40, 40, (64, 3, 16))
    A_log = np.log(rng.uniform(0.1, 50.0, (3, 16)))
    b = rng.uniform(-8, 2, (3, 16))
    al = oracle.eda_ref_safe_gate(a, A_log, b)
    # (strictly above the floor in exact arithmetic; in fp64 the correction
    # term e^{-A Delta / 5} underflows once A Delta is in the hundreds)
    assert np.all(al >= math.exp(-5.0)) and np.all(al <= 1.0)
    # A Delta / 5 <= 16 * softplus(3) / 5 < 10: representably above the floor
    mid = oracle.eda_ref_safe_gate(np.clip(a, -3, 3), np.minimum(A_log, math.log(16.0)), np.minimum(b, 0.0))
    assert np.all(mid > math.exp(-5.0)) and np.all(mid < 1.0)
    hi = oracle.eda_ref_safe_gate(np.full((1, 1), 700.0), np.zeros((1, 1)), np.zeros((1, 1)))
    assert hi[0, 0] == pytest.approx(math.exp(-5.0), rel=1e-12)
    lo = oracle.eda_ref_safe_gate(np.full((1, 1), -700.0), np.zeros((1, 1)), np.zeros((1, 1)))
    assert lo[0, 0] == 1.0


def test_safe_gate_small_input_is_minus_A_delta():
    # the pages: near zero, g ~ -A Delta.  The series of -5 (1 - e^{-u/5}) in
    # u = A Delta alternates: g = -u + u^2/10 - u^3/150 + ..., so the error of
    # the two-term form is below u^3 / 150
    for A in (0.5, 3.0):
        for x in (-6.0, -4.0, -2.0):
            u = A * math.log1p(math.exp(x))
            g = math.log(oracle.eda_ref_safe_gate(np.array([[x]]), np.array([[math.log(A)]]),
                                                  np.zeros((1, 1)))[0, 0])
            assert abs(g - (-u + u * u / 10.0)) <= u ** 3 / 150.0 * 1.001 + 1e-15
            assert abs(g + u) > u ** 3 / 150.0     # ... and the second-order term is there


def test_safe_gate_monotone_in_a_and_A():
    a = np.linspace(-10, 10, 201)[:, None]
    al = oracle.eda_ref_safe_gate(a, np.zeros((1, 1)), np.zeros((1, 1)))[:, 0]
    assert np.all(np.diff(al) < 0)                     # more decay input, less retention
    A = np.linspace(0.1, 20, 50)[None, :]
    al = oracle.eda_ref_safe_gate(np.zeros((1, 50)), np.log(A), np.zeros((1, 50)))[0]
    assert np.all(np.diff(al) < 0)


def test_l2norm():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 5, 2, 7)) * rng.uniform(0.01, 100, (3, 5, 2, 1))
    y = oracle.eda_ref_l2norm(x)
    assert np.allclose(np.linalg.norm(y, axis=-1), 1.0, atol=1e-14)
    # same direction: y = x / |x| component-wise with a positive scale
    ratio = y / x
    assert np.allclose(ratio, ratio[..., :1], rtol=1e-13) and np.all(ratio > 0)
    assert np.all(oracle.eda_ref_l2norm(np.zeros((2, 4))) == 0.0)
    tiny = np.array([[3e-7, 4e-7]])                    # |x| = 5e-7 < eps: divided by eps
    assert np.allclose(oracle.eda_ref_l2norm(tiny), tiny / 1e-6, rtol=1e-15)


def test_expand_key_heads():
    x = np.arange(2 * 3 * 2 * 4, dtype=np.float64).reshape(2, 3, 2, 4)
    y = oracle.expand_key_heads(x, 6)
    assert y.shape == (2, 3, 6, 4)
    for h in range(6):
        assert np.array_equal(y[:, :, h], x[:, :, h // 3])
    with pytest.raises(ValueError):
        oracle.expand_key_heads(x, 5)


def brute_layer(x):
    """Per value head, per token, the three stages on explicit matrices with
    the normalised vectors and the gate computed here from scratch."""
    q, k, e, a = (np.asarray(x[n], dtype=np.float64) for n in ("q", "k", "e", "a"))
    v = np.asarray(x["v"], dtype=np.float64)
    A_log, b = np.asarray(x["A_log"], np.float64), np.asarray(x["dt_bias"], np.float64)
    beta, gamma = np.asarray(x["beta"], np.float64), np.asarray(x["gamma"], np.float64)
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    o = np.zeros((B, T, Hv, dv))
    Sf = np.zeros((B, Hv, dk, dv))
    for bb in range(B):
        for h in range(Hv):
            hk = h // (Hv // Hk)
            S = np.zeros((dk, dv))
            for t in range(T):
                qt, kt, et = (w[bb, t, hk] / max(np.sqrt(w[bb, t, hk] @ w[bb, t, hk]), 1e-6)
                              for w in (q, k, e))
                delta = np.log(1.0 + np.exp(a[bb, t, hk] + b[hk]))
                g = -5.0 + 5.0 * np.exp(-np.exp(A_log[hk]) / 5.0 * delta)
                S = np.diag(np.exp(g)) @ S
                S = (np.eye(dk) - gamma[bb, t, h] * np.outer(et, et)) @ S
                S = (np.eye(dk) - beta[bb, t, h] * np.outer(kt, kt)) @ S + beta[bb, t, h] * np.outer(kt, v[bb, t, h])
                o[bb, t, h] = S.T @ qt
            Sf[bb, h] = S
    return o, Sf


@pytest.mark.parametrize("Hk,Hv", [(1, 1), (1, 2), (2, 4), (3, 3)])
def test_layer_matches_explicit_brute_force(Hk, Hv):
    x = make_layer_inputs(2, 7, Hk, Hv, 5, 3, "f32", seed=10 + Hv)
    o, S = oracle.eda_ref_fwd_layer(x["q"], x["k"], x["e"], x["v"], x["a"], x["A_log"], x["dt_bias"],
                                    x["beta"], x["gamma"])
    ro, rS = brute_layer(x)
    assert np.allclose(o, ro, rtol=1e-12, atol=1e-12)
    assert np.allclose(S, rS, rtol=1e-12, atol=1e-12)


def test_layer_with_unit_inputs_and_no_decay_is_the_plain_recurrence():
    # q, k, e already unit and a -> -inf (alpha = 1): the layer form adds nothing
    x = {n: (None if t is None else t.double().numpy())
         for n, t in make_layer_inputs(1, 6, 2, 2, 4, 3, "f32", seed=3).items()}
    for n in ("q", "k", "e"):
        x[n] = x[n] / np.linalg.norm(x[n], axis=-1, keepdims=True)
    x["a"] = np.full_like(x["a"], -1e4)
    o, S = oracle.eda_ref_fwd_layer(x["q"], x["k"], x["e"], x["v"], x["a"], x["A_log"], x["dt_bias"],
                                    x["beta"], x["gamma"])
    ones = np.ones(x["q"].shape)
    po, pS = oracle.eda_ref_fwd(x["q"], x["k"], x["e"], x["v"], ones, x["beta"], x["gamma"])
    assert np.allclose(o, po, rtol=1e-13, atol=1e-13) and np.allclose(S, pS, rtol=1e-13, atol=1e-13)
