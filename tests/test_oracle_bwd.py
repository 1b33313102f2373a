"""Pins for the backward oracle (oracle.eda_ref_bwd): central finite
differences of the C forward oracle (a separate implementation) for every
input, and closed forms of one token from a zero state."""
import numpy as np
import pytest

import oracle


def case(seed, B=1, T=5, H=2, dk=4, dv=3):
    rng = np.random.default_rng(seed)
    unit = lambda s: (lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True))(rng.standard_normal(s))
    return dict(q=unit((B, T, H, dk)), k=unit((B, T, H, dk)), e=unit((B, T, H, dk)),
                v=rng.standard_normal((B, T, H, dv)), alpha=rng.uniform(0.4, 1.0, (B, T, H, dk)),
                beta=rng.uniform(0.1, 0.9, (B, T, H)), gamma=rng.uniform(0.1, 0.9, (B, T, H)),
                S0=rng.standard_normal((B, H, dk, dv))), rng.standard_normal((B, T, H, dv)), \
        rng.standard_normal((B, H, dk, dv))


def loss(x, dO, dS):
    o, S = oracle.eda_ref_fwd(x["q"], x["k"], x["e"], x["v"], x["alpha"], x["beta"], x["gamma"], x["S0"])
    return float((o * dO).sum() + (S * dS).sum())


@pytest.mark.parametrize("name", ["q", "k", "e", "v", "alpha", "beta", "gamma", "S0"])
def test_gradients_match_finite_differences(name):
    x, dO, dS = case(11)
    g = oracle.eda_ref_bwd(x["q"], x["k"], x["e"], x["v"], x["alpha"], x["beta"], x["gamma"], x["S0"], dO, dS)
    grad = g["d" + name]
    rng = np.random.default_rng(3)
    for _ in range(6):
        idx = tuple(int(rng.integers(n)) for n in x[name].shape)
        h = 1e-5
        xp = {n: a.copy() for n, a in x.items()}
        xm = {n: a.copy() for n, a in x.items()}
        xp[name][idx] += h
        xm[name][idx] -= h
        fd = (loss(xp, dO, dS) - loss(xm, dO, dS)) / (2 * h)
        assert grad[idx] == pytest.approx(fd, rel=1e-6, abs=1e-8), (name, idx)


def test_one_token_from_zero_state_closed_forms():
    # S0 = 0: the decay and the erase act on zero, S1 = beta k v^T, o = beta (k.q) v
    x, dO, dS = case(12, T=1, H=1, dk=5, dv=4)
    S0 = np.zeros_like(x["S0"])
    g = oracle.eda_ref_bwd(x["q"], x["k"], x["e"], x["v"], x["alpha"], x["beta"], x["gamma"], S0, dO, dS)
    q, k, e, v = (x[n][0, 0, 0] for n in ("q", "k", "e", "v"))
    a, b, gm = x["alpha"][0, 0, 0], x["beta"][0, 0, 0], x["gamma"][0, 0, 0]
    do, G = dO[0, 0, 0], dS[0, 0]
    assert np.allclose(g["dv"][0, 0, 0], b * (k @ q) * do + b * G.T @ k, atol=1e-13)
    assert np.allclose(g["dq"][0, 0, 0], b * k * (v @ do), atol=1e-13)
    assert g["dbeta"][0, 0, 0] == pytest.approx((k @ q) * (v @ do) + k @ G @ v, abs=1e-13)
    assert np.allclose(g["de"], 0.0) and np.allclose(g["dgamma"], 0.0) and np.allclose(g["dalpha"], 0.0)
    # the state gradient: transpose of the one-step operator applied to q dO^T + G
    M = (np.eye(5) - b * np.outer(k, k)) @ (np.eye(5) - gm * np.outer(e, e)) @ np.diag(a)
    assert np.allclose(g["dS0"][0, 0], M.T @ (np.outer(q, do) + G), atol=1e-13)


def test_backward_is_linear_in_the_output_gradients():
    x, dO, dS = case(13)
    args = [x[n] for n in ("q", "k", "e", "v", "alpha", "beta", "gamma", "S0")]
    g1 = oracle.eda_ref_bwd(*args, dO, dS)
    g2 = oracle.eda_ref_bwd(*args, 2.0 * dO, None)
    g3 = oracle.eda_ref_bwd(*args, 0.0 * dO, 3.0 * dS)
    for n in g1:
        assert np.allclose(g1[n], 0.5 * g2[n] + g3[n] / 3.0, atol=1e-12)
