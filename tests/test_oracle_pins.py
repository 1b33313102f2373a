"""Pins for the fp64 oracle: what the pages and the mathematics fix.

Each test checks the oracle (oracle/eda_ref.c) against something other than
itself: a value printed on the pages, a closed form, an independent
formulation of the same recurrence (explicit matrices, exact rationals, the
doubled sub-step sequence), or an invariant.  A plausible mistake in the
oracle (wrong sign, dropped gate, swapped stage order, wrong address) fails
at least one of them; `test_planted_mistakes_are_caught` plants such
mistakes in a copy of the oracle and checks exactly that.
"""
import os
import shutil
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest

import oracle
from eda_inputs import hand_example, make_inputs, random_pair_abs_cos_mean
from conftest import read_golden


# ----------------------------------------------------------------------------
# helpers (independent formulations live here, not in the oracle)
# ----------------------------------------------------------------------------
def rand_case(seed, B=1, T=6, H=1, dk=6, dv=4, alpha_lo=0.3, s0=True):
    rng = np.random.default_rng(seed)

    def unit(shape):
        x = rng.standard_normal(shape)
        return x / np.linalg.norm(x, axis=-1, keepdims=True)

    return dict(
        q=unit((B, T, H, dk)), k=unit((B, T, H, dk)), e=unit((B, T, H, dk)),
        v=rng.standard_normal((B, T, H, dv)),
        alpha=rng.uniform(alpha_lo, 1.0, (B, T, H, dk)),
        beta=rng.uniform(0.0, 1.0, (B, T, H)), gamma=rng.uniform(0.0, 1.0, (B, T, H)),
        S0=rng.standard_normal((B, H, dk, dv)) if s0 else None)


def run(x, **kw):
    return oracle.eda_ref_fwd(x["q"], x["k"], x["e"], x["v"], x["alpha"], x["beta"],
                              x["gamma"], x["S0"], **kw)


def product_form(x):
    """Eq. (8) with explicit d_k x d_k matrices:
    S_t = (I - b k k^T)(I - g e e^T) Diag(a) S_{t-1} + b k v^T,  o_t = S_t^T q_t."""
    B, T, H, dk = x["q"].shape
    dv = x["v"].shape[-1]
    o = np.zeros((B, T, H, dv))
    Sf = np.zeros((B, H, dk, dv))
    I = np.eye(dk)
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if x["S0"] is None else x["S0"][b, h].copy()
            for t in range(T):
                q, k, e = x["q"][b, t, h], x["k"][b, t, h], x["e"][b, t, h]
                a, v = x["alpha"][b, t, h], x["v"][b, t, h]
                be, ga = x["beta"][b, t, h], x["gamma"][b, t, h]
                S = (I - be * np.outer(k, k)) @ (I - ga * np.outer(e, e)) @ np.diag(a) @ S \
                    + be * np.outer(k, v)
                o[b, t, h] = S.T @ q
            Sf[b, h] = S
    return o, Sf


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ----------------------------------------------------------------------------
# values printed on the pages
# ----------------------------------------------------------------------------
def test_hand_example_golden():
    """Slides frame 'A two-dimensional example isolates the new capability'
    (also the Chinese reading notes, method part 3): EDA gives (0, 7), the
    delta rule without erase gives (3, 7); erase alone gives (0, 5)."""
    g = read_golden("hand_example.txt")
    x = {k: v.numpy().astype(np.float64) for k, v in hand_example().items()}
    x["S0"][0, 0, :, 0] = g["S_prev"]
    x["e"][0, 0, 0] = g["e"]
    x["k"][0, 0, 0] = g["k"]
    x["v"][0, 0, 0] = g["v"]
    x["alpha"][0, 0, 0] = g["alpha"]
    x["beta"][:] = g["beta"][0]
    x["gamma"][:] = g["gamma"][0]
    o, S = run(x)
    assert S[0, 0, :, 0].tolist() == g["S_eda"]
    assert o[0, 0, 0, 0] == sum(g["S_eda"])  # q = (1, 1)

    xb = dict(x, gamma=np.zeros_like(x["gamma"]))
    _, Sb = run(xb)
    assert Sb[0, 0, :, 0].tolist() == g["S_baseline"]

    xe = dict(x, beta=np.zeros_like(x["beta"]))  # beta = 0: the write is the identity
    _, Se = run(xe)
    assert Se[0, 0, :, 0].tolist() == g["S_after_erase"]


def test_hand_example_generator_matches_golden():
    g = read_golden("hand_example.txt")
    h = hand_example()
    assert h["S0"].flatten().tolist() == g["S_prev"]
    assert h["e"].flatten().tolist() == g["e"] and h["k"].flatten().tolist() == g["k"]
    assert h["v"].flatten().tolist() == g["v"]


# ----------------------------------------------------------------------------
# closed forms and identities fixed by the paper's equations
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_erase_readout_identity_eq12(seed):
    """Eq. (12): after the erase, the readout along q = e is scaled by
    (1 - gamma); a query orthogonal to e reads the same as before.  With
    alpha = 1 and beta = 0 (identity write) the oracle's o_1 is that readout."""
    x = rand_case(seed, T=1, dk=8, dv=5)
    x["alpha"][:] = 1.0
    x["beta"][:] = 0.0
    e = x["e"][0, 0, 0]
    g = x["gamma"][0, 0, 0]
    S0 = x["S0"][0, 0]
    x["q"][0, 0, 0] = e
    o, _ = run(x)
    np.testing.assert_allclose(o[0, 0, 0], (1 - g) * (S0.T @ e), rtol=0, atol=1e-14)
    rng = np.random.default_rng(100 + seed)
    qp = rng.standard_normal(8)
    qp -= (qp @ e) * e
    qp /= np.linalg.norm(qp)
    x["q"][0, 0, 0] = qp
    o, _ = run(x)
    np.testing.assert_allclose(o[0, 0, 0], S0.T @ qp, rtol=0, atol=1e-14)


@pytest.mark.parametrize("seed", [3, 4])
def test_expanded_operator_eq16(seed):
    """Eq. (16): (I - b k k^T)(I - g e e^T) = I - g e e^T - b k k^T + g b (k.e) k e^T,
    applied to the decayed state, plus the write b k v^T (one step)."""
    x = rand_case(seed, T=1, dk=7, dv=3)
    k, e = x["k"][0, 0, 0], x["e"][0, 0, 0]
    a, v = x["alpha"][0, 0, 0], x["v"][0, 0, 0]
    b, g = x["beta"][0, 0, 0], x["gamma"][0, 0, 0]
    M = np.eye(7) - g * np.outer(e, e) - b * np.outer(k, k) + g * b * (k @ e) * np.outer(k, e)
    want = M @ (a[:, None] * x["S0"][0, 0]) + b * np.outer(k, v)
    _, S = run(x)
    np.testing.assert_allclose(S[0, 0], want, rtol=0, atol=1e-13)


@pytest.mark.parametrize("seed", [5, 6])
def test_gamma_zero_is_kda_eq7(seed):
    """gamma = 0 recovers the channel-wise gated delta rule (KDA), Eq. (7):
    S_t = (I - b k k^T) Diag(a) S_{t-1} + b k v^T (Chinese reading notes,
    method part 4: gamma = 0 restores the baseline).  e is random and must
    have no effect."""
    x = rand_case(seed, B=2, T=9, H=2, dk=6, dv=5)
    x["gamma"][:] = 0.0
    o, S = run(x)
    B, T, H, dk = x["q"].shape
    I = np.eye(dk)
    for b in range(B):
        for h in range(H):
            St = x["S0"][b, h].copy()
            for t in range(T):
                k = x["k"][b, t, h]
                St = (I - x["beta"][b, t, h] * np.outer(k, k)) @ np.diag(x["alpha"][b, t, h]) @ St \
                    + x["beta"][b, t, h] * np.outer(k, x["v"][b, t, h])
                np.testing.assert_allclose(o[b, t, h], St.T @ x["q"][b, t, h], rtol=0, atol=1e-12)
            np.testing.assert_allclose(S[b, h], St, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed,shape", [(7, (1, 8, 1, 4, 3)), (8, (2, 5, 3, 6, 6)),
                                        (9, (1, 8, 2, 8, 1))])
def test_product_form_bruteforce_eq8(seed, shape):
    """Eq. (8) brute force with explicit matrices, several heads and steps."""
    B, T, H, dk, dv = shape
    x = rand_case(seed, B=B, T=T, H=H, dk=dk, dv=dv)
    o, S = run(x)
    ow, Sw = product_form(x)
    assert rel(o, ow) < 1e-13 and rel(S, Sw) < 1e-13


def test_exact_rationals_eq8():
    """Eq. (8) is an algebraic identity, so it holds for any rational inputs.
    With dyadic rationals (exact in fp64) the exact product-form result,
    computed in fractions.Fraction, must match the fp64 oracle to rounding."""
    rng = np.random.default_rng(11)
    B, T, H, dk, dv = 1, 4, 1, 3, 2

    def dy(shape, lo, hi, den=8):
        return rng.integers(lo, hi + 1, size=shape).astype(np.float64) / den

    x = dict(q=dy((B, T, H, dk), -8, 8), k=dy((B, T, H, dk), -8, 8), e=dy((B, T, H, dk), -8, 8),
             v=dy((B, T, H, dv), -16, 16), alpha=dy((B, T, H, dk), 1, 8),
             beta=dy((B, T, H), 0, 8), gamma=dy((B, T, H), 0, 8), S0=dy((B, H, dk, dv), -16, 16))
    F = lambda a: Fraction(float(a))

    def mat(rows):
        return [[F(c) for c in r] for r in rows]

    def mm(A, Bm):
        return [[sum((A[i][p] * Bm[p][j] for p in range(len(Bm))), Fraction(0))
                 for j in range(len(Bm[0]))] for i in range(len(A))]

    S = mat(x["S0"][0, 0])
    outs = []
    for t in range(T):
        q, k, e = (x[n][0, t, 0] for n in ("q", "k", "e"))
        a, v = x["alpha"][0, t, 0], x["v"][0, t, 0]
        b, g = F(x["beta"][0, t, 0]), F(x["gamma"][0, t, 0])
        Ek = [[(1 if i == j else 0) - b * F(k[i]) * F(k[j]) for j in range(dk)] for i in range(dk)]
        Ee = [[(1 if i == j else 0) - g * F(e[i]) * F(e[j]) for j in range(dk)] for i in range(dk)]
        D = [[F(a[i]) if i == j else Fraction(0) for j in range(dk)] for i in range(dk)]
        S = mm(mm(mm(Ek, Ee), D), S)
        S = [[S[i][j] + b * F(k[i]) * F(v[j]) for j in range(dv)] for i in range(dk)]
        outs.append([sum((S[i][j] * F(q[i]) for i in range(dk)), Fraction(0)) for j in range(dv)])
    o, Sf = run(x)
    exact_S = np.array([[float(c) for c in r] for r in S])
    exact_o = np.array([[float(c) for c in r] for r in outs])
    assert rel(Sf[0, 0], exact_S) < 1e-14
    assert rel(o[0, :, 0], exact_o) < 1e-14


@pytest.mark.parametrize("seed", [12, 13])
def test_doubled_sequence_eqs17_18(seed):
    """Sub-step table (slides frame 'Two virtual steps recover a standard
    delta recurrence'; paper Sec. 3.4, Eqs. (17)-(18)): token t becomes an
    erase sub-step (q'=0, k'=e, v'=0, beta'=gamma, alpha'=alpha) then a delta
    sub-step (q'=q, k'=k, v'=v, beta'=beta, alpha'=1) of the standard gated
    delta recurrence; only delta sub-steps produce output."""
    x = rand_case(seed, B=1, T=10, H=2, dk=5, dv=4)
    o, S = run(x)
    B, T, H, dk = x["q"].shape
    I = np.eye(dk)
    for h in range(H):
        St = x["S0"][0, h].copy()
        for t in range(T):
            subs = [(x["e"][0, t, h], np.zeros(4), x["gamma"][0, t, h], x["alpha"][0, t, h], None),
                    (x["k"][0, t, h], x["v"][0, t, h], x["beta"][0, t, h], np.ones(dk),
                     x["q"][0, t, h])]
            for kk, vv, bb, aa, qq in subs:
                St = (I - bb * np.outer(kk, kk)) @ (aa[:, None] * St) + bb * np.outer(kk, vv)
                if qq is not None:
                    np.testing.assert_allclose(o[0, t, h], St.T @ qq, rtol=0, atol=1e-13)
        np.testing.assert_allclose(S[0, h], St, rtol=0, atol=1e-13)


@pytest.mark.parametrize("seed", [14, 15])
def test_e_equals_k_contraction(seed):
    """e = k (Chinese reading notes, method part 4; paper Sec. 3.3): old
    content along k is scaled by (1 - beta)(1 - gamma), the new value keeps
    coefficient beta: S_1^T k = (1-b)(1-g) S_0^T k + b v (alpha = 1)."""
    x = rand_case(seed, T=1, dk=6, dv=4)
    x["alpha"][:] = 1.0
    x["e"] = x["k"].copy()
    k = x["k"][0, 0, 0]
    b, g = x["beta"][0, 0, 0], x["gamma"][0, 0, 0]
    _, S = run(x)
    want = (1 - b) * (1 - g) * (x["S0"][0, 0].T @ k) + b * x["v"][0, 0, 0]
    np.testing.assert_allclose(S[0, 0].T @ k, want, rtol=0, atol=1e-13)


def test_nonexpansive_without_writes():
    """Each rank-1 factor has eigenvalues {1 - gate, 1} for unit addresses and
    gates in [0, 1], and alpha <= 1, so with v = 0 the state's Frobenius norm
    never grows (slides frame 'Order matters...', last bullet; Chinese notes
    method part 4)."""
    x = rand_case(16, T=24, dk=6, dv=3, alpha_lo=0.5)
    x["v"][:] = 0.0
    norms = []
    for t in range(1, 25):
        sub = {n: (a if n == "S0" else a[:, :t]) for n, a in x.items()}
        _, S = run(sub)
        norms.append(np.linalg.norm(S))
    n0 = np.linalg.norm(x["S0"])
    seq = [n0] + norms
    assert all(b <= a * (1 + 1e-14) for a, b in zip(seq, seq[1:]))
    assert seq[-1] < 0.9 * seq[0]


def test_linearity_and_column_independence():
    """Eq. (8) is linear in (S_{t-1}, v_t) for fixed gates and addresses, and
    value columns never mix: permuting the columns of v and S0 permutes those
    of o and S exactly."""
    x = rand_case(17, B=1, T=7, H=2, dk=5, dv=6)
    y = dict(x, v=np.random.default_rng(5).standard_normal(x["v"].shape),
             S0=np.random.default_rng(6).standard_normal(x["S0"].shape))
    z = dict(x, v=2.0 * x["v"] - 3.0 * y["v"], S0=2.0 * x["S0"] - 3.0 * y["S0"])
    ox, Sx = run(x)
    oy, Sy = run(y)
    oz, Sz = run(z)
    assert rel(oz, 2 * ox - 3 * oy) < 1e-13 and rel(Sz, 2 * Sx - 3 * Sy) < 1e-13
    perm = np.array([3, 0, 5, 1, 4, 2])
    xp = dict(x, v=x["v"][..., perm], S0=x["S0"][..., perm])
    op, Sp = run(xp)
    assert np.array_equal(op, ox[..., perm]) and np.array_equal(Sp, Sx[..., perm])


def test_stage_order_matters():
    """Paper Sec. 3.3: the factors act right to left and diagonal decay does
    not commute with the erase unless the decay is a scalar.  The oracle must
    differ from an erase-before-decay variant for channel-wise alpha, and
    agree with it when alpha is the same on every channel."""
    x = rand_case(18, T=5, dk=6, dv=3, alpha_lo=0.2)

    def erase_first(x):
        dk = x["q"].shape[-1]
        I = np.eye(dk)
        S = x["S0"][0, 0].copy()
        for t in range(x["q"].shape[1]):
            k, e = x["k"][0, t, 0], x["e"][0, t, 0]
            b, g = x["beta"][0, t, 0], x["gamma"][0, t, 0]
            S = (I - b * np.outer(k, k)) @ np.diag(x["alpha"][0, t, 0]) @ \
                (I - g * np.outer(e, e)) @ S + b * np.outer(k, x["v"][0, t, 0])
        return S

    _, S = run(x)
    assert rel(S[0, 0], erase_first(x)) > 1e-3
    xs = dict(x, alpha=np.repeat(x["alpha"][..., :1], 6, axis=-1))
    _, Ss = run(xs)
    assert rel(Ss[0, 0], erase_first(xs)) < 1e-13


def test_thread_split_is_bit_identical():
    x = rand_case(19, B=1, T=20, H=2, dk=9, dv=13)
    o1, S1 = run(x, nthreads=1)
    for nt in (2, 3, 8, 40):
        o2, S2 = run(x, nthreads=nt)
        assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def test_no_state_is_zero_state():
    x = rand_case(20, T=4)
    o1, S1 = run(dict(x, S0=None))
    o2, S2 = run(dict(x, S0=np.zeros_like(x["S0"])))
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def test_decode_wrapper_is_the_same_recurrence():
    """A decode sequence (one token per step, state carried) equals calling
    the oracle one step at a time, feeding each S_final back as S0."""
    x = rand_case(21, B=3, T=6, H=2, dk=5, dv=4)
    stepwise = {n: (np.swapaxes(a, 0, 1) if n != "S0" else a) for n, a in x.items()}
    o, S = oracle.eda_ref_decode(**stepwise)
    Sc = x["S0"]
    for t in range(6):
        ot, Sc = oracle.eda_ref_fwd(*(x[n][:, t:t + 1] for n in
                                      ("q", "k", "e", "v", "alpha", "beta", "gamma")), Sc)
        np.testing.assert_array_equal(o[t], ot[:, 0])
    np.testing.assert_array_equal(S, Sc)


# ----------------------------------------------------------------------------
# input generator
# ----------------------------------------------------------------------------
def test_random_abs_cos_closed_form():
    """E|u.r| = Gamma(d/2)/(sqrt(pi) Gamma((d+1)/2)): 2/pi in 2-D, 1/2 in 3-D,
    and the ~0.0707 reference in 128-D quoted by the slides and the notes."""
    assert abs(random_pair_abs_cos_mean(2) - 2 / np.pi) < 1e-15
    assert abs(random_pair_abs_cos_mean(3) - 0.5) < 1e-15
    assert abs(random_pair_abs_cos_mean(128) - 0.0707) < 1e-4


def test_generator_address_geometry():
    """Independent unit e and k in 128-D have mean |cos| ~ 0.0707."""
    x = make_inputs(1, 4096, 2, 128, 128, "bf16", seed=1)
    e = x["e"].float().double()
    k = x["k"].float().double()
    n_e, n_k = e.norm(dim=-1), k.norm(dim=-1)
    assert float((n_e - 1).abs().max()) < 2 ** -7 and float((n_k - 1).abs().max()) < 2 ** -7
    c = ((e * k).sum(-1) / (n_e * n_k)).abs()
    sd = float(c.std()) / np.sqrt(c.numel())
    assert abs(float(c.mean()) - random_pair_abs_cos_mean(128)) < 4 * sd
    a = x["alpha"]
    assert float(a.min()) > 0 and float(a.max()) < 1
    assert 0.85 < float(a.mean()) < 0.89  # E sigmoid(N(2, 0.5)) ~ 0.87
    assert x["S0"] is None


def test_generator_is_seeded():
    a = make_inputs(1, 16, 2, 8, 8, "bf16", seed=3, s0_std=0.02)
    b = make_inputs(1, 16, 2, 8, 8, "bf16", seed=3, s0_std=0.02)
    c = make_inputs(1, 16, 2, 8, 8, "bf16", seed=4, s0_std=0.02)
    for n in a:
        assert a[n].equal(b[n])
    assert not a["q"].equal(c["q"])


# ----------------------------------------------------------------------------
# planted mistakes in a copy of the oracle must be caught by the pins above
# ----------------------------------------------------------------------------
MUTATIONS = {
    "erase_sign": ("S[i * w + j] - gamma * e[i] * re[j]", "S[i * w + j] + gamma * e[i] * re[j]"),
    "erase_reads_k": ("re[j] += S[i * w + j] * e[i]", "re[j] += S[i * w + j] * k[i]"),
    "dropped_beta": ("beta * k[i] * (v[j0 + j] - rk[j])", "k[i] * (v[j0 + j] - rk[j])"),
    "write_uses_e": ("beta * k[i] * (v[j0 + j] - rk[j])", "beta * e[i] * (v[j0 + j] - rk[j])"),
    "decay_by_column": ("S[i * w + j] = a[i] * S[i * w + j]", "S[i * w + j] = a[j % dk] * S[i * w + j]"),
    "read_uses_k": ("re[j] += S[i * w + j] * q[i]", "re[j] += S[i * w + j] * k[i]"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(name, monkeypatch, tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "eda_ref.c")).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mpath = tmp_path / "eda_ref_mut.c"
    mpath.write_text(src.replace(old, new))
    lib = tmp_path / "libeda_ref_mut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", str(mpath),
                    "-o", str(lib)], check=True)
    import ctypes
    mut = ctypes.CDLL(str(lib))
    dp = ctypes.POINTER(ctypes.c_double)
    mut.eda_ref_fwd.argtypes = [dp] * 10 + [ctypes.c_long] * 5 + [ctypes.c_int]
    mut.eda_ref_fwd.restype = ctypes.c_int
    monkeypatch.setattr(oracle, "_lib", mut)
    caught = []
    for test in (lambda: test_product_form_bruteforce_eq8(8, (2, 5, 3, 6, 6)),
                 test_hand_example_golden,
                 lambda: test_erase_readout_identity_eq12(0)):
        try:
            test()
        except AssertionError:
            caught.append(True)
    assert caught, f"planted mistake {name} was not caught by any pin"
