"""Pins for the oracle of the second workload, the rank-1 DPLR update of
GDN-2 and QED (QED slides, frames on GDN-2's decay/erase/write split and on
QED's erase vector): S_t = Sbar_t + k_t (v_t - Sbar_t^T a_t)^T with
Sbar_t = Diag(alpha_t) S_{t-1}, o_t = S_t^T q_t.

Checked against the slides' worked two-dimensional examples
(tests/golden/qed_example.txt), against the EDA oracle (a different
implementation, in C) through the exact reduction gamma = 0, a = beta k,
v -> beta v, and against explicit matrices and invariants the slides state.
"""
import numpy as np
import pytest

import oracle
from conftest import read_golden


def col(x):
    return np.asarray(x, dtype=np.float64).reshape(1, 1, 1, -1)


def test_qed_two_dimensional_example():
    g = read_golden("qed_example.txt")
    k, q, b = (np.array(g[n]) for n in ("k", "q", "b"))
    S0 = np.array(g["Sbar"]).reshape(1, 1, 2, 1)
    v = col(g["wv"])
    lam = g["lambda"][0]
    alpha = col([1.0, 1.0])
    # GDN-2: a = b o k
    a_base = oracle.gdn2_erase_vector(k, b)
    o_b, S_b = oracle.eda_ref_dplr_fwd(col(q), col(k), col(a_base), v, alpha, S0)
    assert float(v[0, 0, 0, 0] - S0[0, 0, :, 0] @ a_base) == pytest.approx(g["r_base"][0], abs=1e-15)
    assert o_b[0, 0, 0, 0] == pytest.approx(g["o_base"][0], abs=1e-14)
    # QED: the projected gated query and its measurement
    d = oracle.qed_erase_vector(q, k, b, lam) - oracle.gdn2_erase_vector(k, b)
    assert np.allclose(d / lam, g["d"], atol=1e-15)
    assert float(S0[0, 0, :, 0] @ (d / lam)) == pytest.approx(g["Sbar_dot_d"][0], abs=1e-14)
    a_qed = oracle.qed_erase_vector(q, k, b, lam)
    o_q, S_q = oracle.eda_ref_dplr_fwd(col(q), col(k), col(a_qed), v, alpha, S0)
    assert np.allclose(S_q[0, 0, :, 0] - S_b[0, 0, :, 0], g["delta_S"], atol=1e-14)
    assert o_q[0, 0, 0, 0] - o_b[0, 0, 0, 0] == pytest.approx(g["delta_o"][0], abs=1e-14)
    assert o_q[0, 0, 0, 0] == pytest.approx(g["o_qed"][0], abs=1e-14)


def test_non_normal_erase_factor_example():
    g = read_golden("qed_example.txt")
    k, q, b, lam = np.array([1.0, 0.0]), np.array([0.0, 1.0]), np.array(g["b"]), g["lambda"][0]
    a = oracle.qed_erase_vector(q, k, b, lam)
    assert np.allclose(a, g["a_frame2"], atol=1e-15)
    # one step with v = 0 and alpha = 1 applies M = I - k a^T to the state
    S0 = np.array([0.0, 1.0]).reshape(1, 1, 2, 1)
    _, S = oracle.eda_ref_dplr_fwd(col(q), col(k), col(a), col([0.0]), col([1.0, 1.0]), S0)
    M = np.array(g["M_frame2"]).reshape(2, 2)
    assert np.allclose(S[0, 0, :, 0], M @ np.array([0.0, 1.0]), atol=1e-15)
    assert float(S[0, 0, :, 0] @ S[0, 0, :, 0]) == pytest.approx(g["M_times_e2_norm_sq"][0], abs=1e-14)
    assert sorted(np.linalg.eigvals(M).real) == pytest.approx([1.0 - a @ k, 1.0])


def test_gamma_zero_eda_is_dplr_with_gated_key():
    # EDA with gamma = 0: S = (I - beta k k^T) Diag(alpha) S + beta k v^T
    #                     = Sbar + k (beta v - Sbar^T (beta k))^T
    rng = np.random.default_rng(5)
    B, T, H, dk, dv = 2, 9, 3, 6, 4
    unit = lambda s: (lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True))(rng.standard_normal(s))
    q, k, e = unit((B, T, H, dk)), unit((B, T, H, dk)), unit((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    alpha = rng.uniform(0.3, 1.0, (B, T, H, dk))
    beta = rng.uniform(0, 1, (B, T, H))
    S0 = rng.standard_normal((B, H, dk, dv))
    eo, eS = oracle.eda_ref_fwd(q, k, e, v, alpha, beta, np.zeros((B, T, H)), S0)
    do, dS = oracle.eda_ref_dplr_fwd(q, k, beta[..., None] * k, beta[..., None] * v, alpha, S0)
    assert np.allclose(do, eo, rtol=1e-12, atol=1e-12) and np.allclose(dS, eS, rtol=1e-12, atol=1e-12)


def test_explicit_matrix_brute_force():
    rng = np.random.default_rng(6)
    B, T, H, dk, dv = 1, 5, 2, 4, 3
    q, k, a = (rng.standard_normal((B, T, H, dk)) for _ in range(3))
    v = rng.standard_normal((B, T, H, dv))
    alpha = rng.uniform(0.2, 1.0, (B, T, H, dk))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S = oracle.eda_ref_dplr_fwd(q, k, a, v, alpha, S0)
    for h in range(H):
        X = S0[0, h].copy()
        for t in range(T):
            X = (np.eye(dk) - np.outer(k[0, t, h], a[0, t, h])) @ np.diag(alpha[0, t, h]) @ X \
                + np.outer(k[0, t, h], v[0, t, h])
            assert np.allclose(o[0, t, h], X.T @ q[0, t, h], rtol=1e-12, atol=1e-12)
        assert np.allclose(S[0, h], X, rtol=1e-12, atol=1e-12)


def test_orthogonal_probe_unchanged_and_projection():
    # slides: for x orthogonal to k_t the edit cannot change x's response; d is orthogonal to a unit k
    rng = np.random.default_rng(7)
    dk, dv = 6, 3
    k = rng.standard_normal(dk); k /= np.linalg.norm(k)
    q, b = rng.standard_normal(dk), rng.uniform(0, 1, dk)
    a = oracle.qed_erase_vector(q, k, b, 0.3)
    d = (a - b * k) / 0.3
    assert abs(d @ k) < 1e-14
    S0 = rng.standard_normal((1, 1, dk, dv))
    alpha = rng.uniform(0.5, 1, dk)
    _, S = oracle.eda_ref_dplr_fwd(col(q), col(k), col(a), rng.standard_normal((1, 1, 1, dv)), col(alpha), S0)
    x = rng.standard_normal(dk); x -= (x @ k) * k
    Sbar = alpha[:, None] * S0[0, 0]
    assert np.allclose(S[0, 0].T @ x, Sbar.T @ x, atol=1e-13)
