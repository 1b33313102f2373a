"""The chunk algebra of the GPU chunked forward, re-derived in fp64 NumPy
(`tests/chunk_ref.py`) and checked against the fp64 token-recurrence oracle.

These run on the CPU (`-m "not gpu"`): a mistake in the factorisation the
kernels evaluate (split exponent, UT inverse, WY factors, the Phi/Psi state
map, the query-side products, the wide-chunk fallback, tail padding) shows
here without a GPU.  Sources: sub-step form, EDA paper Sec. 3.4, Eqs.
(17)-(18) and the slides' frame "Two virtual steps recover a standard delta
recurrence"; the recurrence itself, paper Sec. 3.3, Eq. (8).
"""
import numpy as np
import pytest

import eda_inputs
import oracle
from tests import chunk_ref
from tests._helpers import to64

# The kernels switch a chunk to the element-wise path when some channel
# decays by more than e^-150 inside it.
WIDE_LOG = -150.0
CHUNKS = (16, 32, 64)


def _head(x, b=0, h=0):
    g = lambda n: to64(x[n])[b, :, h]
    S0 = None if x["S0"] is None else to64(x["S0"])[b, h]
    return dict(q=g("q"), k=g("k"), e=g("e"), v=g("v"), alpha=g("alpha"), beta=g("beta"),
                gamma=g("gamma"), S0=S0)


def _oracle_head(x, b=0, h=0):
    sl = lambda t: t[b:b + 1, :, h:h + 1]
    S0 = None if x["S0"] is None else x["S0"][b:b + 1, h:h + 1]
    o, S = oracle.eda_ref_fwd(sl(x["q"]), sl(x["k"]), sl(x["e"]), sl(x["v"]), sl(x["alpha"]),
                              sl(x["beta"]), sl(x["gamma"]), S0)
    return o[0, :, 0], S[0, 0]


def _chunked(hd, C, form, wide_log=WIDE_LOG):
    sub = chunk_ref.substeps_eda(hd["q"], hd["k"], hd["e"], hd["v"], hd["alpha"], hd["beta"], hd["gamma"])
    return chunk_ref.chunk_forward(sub, hd["S0"], C, form=form, wide_log=wide_log)


def _assert_close(got, ref, tol, what):
    err = float(np.max(np.abs(got - ref)))
    scale = max(1.0, float(np.max(np.abs(ref))))
    assert err <= tol * scale, f"{what}: max-abs {err:.3e} (scale {scale:.2e})"


@pytest.mark.parametrize("C", CHUNKS)
@pytest.mark.parametrize("T", [1, 63, 64, 65, 127, 129])
@pytest.mark.parametrize("form", ["u", "phi"])
def test_chunk_forward_matches_oracle(C, T, form):
    """Both state-pass forms, every chunk size, ragged tails (T = 1 is a
    single padded chunk), random S0, d = 16."""
    x = eda_inputs.make_inputs(1, T, 1, 16, 12, "f32", seed=100 + T, s0_std=0.5)
    hd = _head(x)
    o, S, _ = _chunked(hd, C, form)
    ro, rS = _oracle_head(x)
    _assert_close(o, ro, 1e-12, f"o C={C} T={T} {form}")
    _assert_close(S, rS, 1e-12, f"S C={C} T={T} {form}")


@pytest.mark.parametrize("C", CHUNKS)
def test_full_head_dim(C):
    """d_k = d_v = 128 (the configurations' head size), three chunks and a
    tail, bf16-rounded unit inputs as the GPU reads them."""
    x = eda_inputs.make_inputs(1, 3 * C + 5, 1, 128, 128, "bf16", seed=7, s0_std=0.02)
    hd = _head(x)
    ro, rS = _oracle_head(x)
    for form in ("u", "phi"):
        o, S, _ = _chunked(hd, C, form)
        _assert_close(o, ro, 1e-12, f"o {form}")
        _assert_close(S, rS, 1e-12, f"S {form}")


@pytest.mark.parametrize("kind", eda_inputs.OVERLAP_KINDS)
@pytest.mark.parametrize("C", CHUNKS)
def test_address_overlap(kind, C):
    """e and k overlapping (Eq. (16)'s cross term at full strength), gates
    at their limits: the chunk algebra still equals the token recurrence."""
    x = eda_inputs.make_overlap_inputs(kind, 1, 3 * C + 3, 1, 32, 16, "f32", seed=21)
    hd = _head(x)
    ro, rS = _oracle_head(x)
    o, S, facs = _chunked(hd, C, "phi")
    _assert_close(o, ro, 1e-12, f"o {kind}")
    _assert_close(S, rS, 1e-12, f"S {kind}")
    if kind == "e_eq_k":
        # the cross-term entry of the Gram: A[2t+1, 2t] = beta_t (k_t . e_t) = beta_t |k_t|^2
        f = facs[0]
        t = np.arange(C)
        kk = np.sum(hd["k"][:C] * hd["k"][:C], axis=1)
        np.testing.assert_allclose(f["A"][2 * t + 1, 2 * t], hd["beta"][:C] * kk, rtol=1e-12, atol=1e-14)


def test_chunk_size_independence():
    """The chunk size is an implementation parameter: 16, 32 and 64 give the
    same result (to fp64 rounding)."""
    x = eda_inputs.make_inputs(1, 200, 1, 24, 8, "f32", seed=5, s0_std=0.3)
    hd = _head(x)
    res = [_chunked(hd, C, "phi")[:2] for C in CHUNKS]
    for o, S in res[1:]:
        _assert_close(o, res[0][0], 1e-12, "o across chunk sizes")
        _assert_close(S, res[0][1], 1e-12, "S across chunk sizes")


@pytest.mark.parametrize("C", CHUNKS)
def test_split_exponent_equals_elementwise(C):
    """A and P from the split operands (Kl = lam e^{G - r}, Kr = kap e^{r - G},
    r = G_C / 2) equal their element-wise definitions with e^{G_j - G_i}, and
    the exported factors agree, for a strongly decaying chunk that is still
    below the wide threshold."""
    rng = np.random.default_rng(3)
    dk = 16
    x = eda_inputs.make_inputs(1, C, 1, dk, 4, "f32", seed=9)
    hd = _head(x)
    hd["alpha"] = np.exp(-rng.uniform(0.0, 90.0 / C, size=hd["alpha"].shape))   # G_C down to ~e^-90
    sub = chunk_ref.substeps_eda(hd["q"], hd["k"], hd["e"], hd["v"], hd["alpha"], hd["beta"], hd["gamma"])
    args = (sub["lam"], sub["kap"], sub["bp"], sub["logdec"], sub["q"])
    fs = chunk_ref.chunk_factors(*args, wide_log=WIDE_LOG)
    fe = chunk_ref.chunk_factors(*args, wide_log=0.0)   # forces the element-wise path
    assert not fs["wide"] and fe["wide"]
    for n in ("A", "P", "W", "Tp", "Kh", "Qh", "Ph", "Phi", "Psi", "dec"):
        np.testing.assert_allclose(fs[n], fe[n], rtol=1e-9, atol=1e-12, err_msg=n)


@pytest.mark.parametrize("C", CHUNKS)
def test_wide_chunk_fallback(C):
    """Every retention at the safe gate's floor alpha = e^-5 (EDA paper Eqs.
    (14)-(15); slides frame on the safe decay): a chunk decays by e^{-5C}, past
    the e^-150 threshold at C >= 32, so those chunks take the element-wise
    path; the result still equals the recurrence."""
    x = eda_inputs.make_inputs(1, 2 * C + 7, 1, 16, 8, "f32", seed=31, s0_std=0.5)
    x["alpha"][:] = float(np.exp(-5.0))
    hd = _head(x)
    ro, rS = _oracle_head(x)
    o, S, facs = _chunked(hd, C, "phi")
    assert any(f["wide"] for f in facs) == (5.0 * C > 150.0)
    _assert_close(o, ro, 1e-12, "o floor")
    _assert_close(S, rS, 1e-12, "S floor")


@pytest.mark.parametrize("C", CHUNKS)
def test_ut_inverse_and_factor_identities(C):
    """(I + A) M = I with M unit lower triangular; U = T'V - W S reproduces
    the sub-step recurrence's pseudo-values; o = (q o Gam) S + P U equals
    Qhat S + Phat V; S_next from U equals S_next from (Phi, Psi)."""
    x = eda_inputs.make_inputs(1, C, 1, 16, 8, "f32", seed=41, s0_std=0.5)
    hd = _head(x)
    sub = chunk_ref.substeps_eda(hd["q"], hd["k"], hd["e"], hd["v"], hd["alpha"], hd["beta"], hd["gamma"])
    f = chunk_ref.chunk_factors(sub["lam"], sub["kap"], sub["bp"], sub["logdec"], sub["q"], wide_log=WIDE_LOG)
    L = 2 * C
    M = f["M"]
    np.testing.assert_allclose((np.eye(L) + f["A"]) @ M, np.eye(L), atol=1e-12)
    assert np.all(np.triu(M, 1) == 0.0) and np.allclose(np.diag(M), 1.0)
    S = hd["S0"]
    V = hd["v"]
    U = f["Tp"] @ V - f["W"] @ S
    # pseudo-values of the sub-step recurrence, token by token
    St = S.copy()
    Gam = np.exp(np.cumsum(sub["logdec"], axis=0))
    u_ref = np.empty((L, V.shape[1]))
    for j in range(L):
        if j % 2 == 0:
            St = hd["alpha"][j // 2][:, None] * St
        u_ref[j] = sub["bp"][j] * (sub["nu"][j] - St.T @ sub["lam"][j])
        St = St + np.outer(sub["kap"][j], u_ref[j])
    np.testing.assert_allclose(U, u_ref, atol=1e-12)
    O1 = (sub["q"] * Gam) @ S + f["P"] @ U
    O2 = f["Qh"] @ S + f["Ph"] @ V
    np.testing.assert_allclose(O1, O2, atol=1e-12)
    S1 = f["dec"][:, None] * S + f["Kh"].T @ U
    S2 = f["dec"][:, None] * S + f["Phi"] @ S + f["Psi"] @ V
    np.testing.assert_allclose(S1, St, atol=1e-12)
    np.testing.assert_allclose(S2, St, atol=1e-12)


@pytest.mark.parametrize("C", CHUNKS)
def test_dplr_chunk_form(C):
    """The rank-1 DPLR update (QED slides, GDN-2 and QED frames) in the same
    chunk algebra with read keys a and write keys k, against the DPLR
    oracle."""
    x = eda_inputs.make_dplr_inputs(1, 2 * C + 9, 1, 16, 8, "f32", seed=51, s0_std=0.3)
    q, k, v, alpha = (to64(x[n])[0, :, 0] for n in ("q", "k", "v", "alpha"))
    b = to64(x["b"])[0, :, 0]
    a = b * k
    S0 = to64(x["S0"])[0, 0]
    sub = chunk_ref.substeps_dplr(q, k, a, v, alpha)
    o, S, _ = chunk_ref.chunk_forward(sub, S0, C, form="phi", wide_log=WIDE_LOG)
    ro, rS = oracle.eda_ref_dplr_fwd(q[None, :, None], k[None, :, None], a[None, :, None],
                                     v[None, :, None], alpha[None, :, None], S0[None, None])
    _assert_close(o, ro[0, :, 0], 1e-12, "dplr o")
    _assert_close(S, rS[0, 0], 1e-12, "dplr S")


def test_planted_mistakes_are_caught():
    """The comparison bites: dropping the cross-term row pairing (A made
    block-diagonal per token), or the decay in the state map, breaks the
    agreement with the oracle by far more than the tolerance."""
    x = eda_inputs.make_overlap_inputs("cos09", 1, 40, 1, 16, 8, "f32", seed=61)
    hd = _head(x)
    ro, rS = _oracle_head(x)
    sub = chunk_ref.substeps_eda(hd["q"], hd["k"], hd["e"], hd["v"], hd["alpha"], hd["beta"], hd["gamma"])
    # mistake 1: no decay on the erase sub-steps
    bad = dict(sub, logdec=np.zeros_like(sub["logdec"]))
    o, S, _ = chunk_ref.chunk_forward(bad, hd["S0"], 16)
    assert np.max(np.abs(S - rS)) > 1e-3
    # mistake 2: erase sub-step written along k instead of e (the cross term lost)
    lam = sub["lam"].copy()
    lam[0::2] = sub["lam"][1::2]
    bad = dict(sub, lam=lam, kap=lam)
    o, S, _ = chunk_ref.chunk_forward(bad, hd["S0"], 16)
    assert np.max(np.abs(o - ro)) > 1e-3


@pytest.mark.parametrize("C", CHUNKS)
@pytest.mark.parametrize("P", [2, 3, 5])
@pytest.mark.parametrize("T", [300, 333])
def test_segmented_state_pass(C, P, T):
    """Segments: the maps [M_s | N_s] of every segment but the last, walked on
    the augmented state from [I | 0], their prefix, and each
    segment walked from its start state reproduce the token recurrence
    (ragged last chunk and segment, random S0, d_k != d_v)."""
    x = eda_inputs.make_inputs(1, T, 1, 16, 12, "f32", seed=700 + T + P, s0_std=0.5)
    hd = _head(x)
    sub = chunk_ref.substeps_eda(hd["q"], hd["k"], hd["e"], hd["v"], hd["alpha"], hd["beta"], hd["gamma"])
    o, S, maps = chunk_ref.segmented_forward(sub, hd["S0"], C, P, wide_log=WIDE_LOG)
    ro, rS = _oracle_head(x)
    _assert_close(o, ro, 1e-12, f"o C={C} P={P} T={T}")
    _assert_close(S, rS, 1e-12, f"S C={C} P={P} T={T}")
    assert 1 <= len(maps) <= P - 1


def test_segment_map_is_the_chunk_map_product():
    """M_s of one segment is the ordered product of its chunks' linear maps
    (a later chunk on the left), checked on a two-chunk segment; a planted
    reversal of the order fails."""
    x = eda_inputs.make_inputs(1, 64, 1, 16, 12, "f32", seed=77)
    hd = _head(x)
    sub = chunk_ref.substeps_eda(hd["q"], hd["k"], hd["e"], hd["v"], hd["alpha"], hd["beta"], hd["gamma"])
    _, _, maps = chunk_ref.segmented_forward(sub, None, 16, 2, wide_log=WIDE_LOG)
    _, _, facs = chunk_ref.chunk_forward(sub, None, 16, wide_log=WIDE_LOG)
    A = [np.diag(f["dec"]) + f["Phi"] for f in facs]
    M0 = maps[0][0]
    assert np.allclose(M0, A[1] @ A[0], atol=1e-12, rtol=0)
    assert not np.allclose(M0, A[0] @ A[1], atol=1e-6, rtol=0)
