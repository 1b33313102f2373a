"""fp64 NumPy re-derivation of the chunk algebra the HIP chunked forward uses.

TEST INFRASTRUCTURE ONLY.  This is not the oracle (the oracle is the plain
token recurrence in `oracle/`): it restates, step by step and in fp64, the
factorisation the GPU kernels evaluate, so that the algebra itself is checked
against the oracle on the CPU, independently of any GPU run.  It imports
nothing from the GPU library and shares no code with it.

Sub-step form (EDA paper Sec. 3.4, Eqs. (17)-(18); reading slides, frame "Two
virtual steps recover a standard delta recurrence"): token t becomes
  erase sub-step 2t   : read/write key e_t, gate gamma_t, decay alpha_t, no value
  delta sub-step 2t+1 : read/write key k_t, gate beta_t, no decay, value v_t,
                        output S^T q_t
of the gated delta recurrence  S_j = D_j S_{j-1} + kap_j u_j^T,
u_j = b'_j (nu_j - (D_j S_{j-1})^T lam_j)  (lam = read key, kap = write key;
lam = kap for EDA, the rank-1 DPLR update of the QED slides reads along its
erase vector a and writes along k).

Unrolled over a chunk of C tokens (L = 2C sub-steps) from the chunk's initial
state S, with G_t the cumulative natural-log decay per key channel inside the
chunk, Gam_t = e^{G_t}, t(j) the token of sub-step j:
  (I + A) U = Diag(b') (N - (lam o Gam) S),   A_ji = b'_j sum_c lam_jc kap_ic Gam_t(j)c / Gam_t(i)c  (i < j)
  o_t = (q_t o Gam_t)^T S + sum_{i <= 2t+1} P_ti u_i,   P_ti = sum_c q_tc kap_ic Gam_tc / Gam_t(i)c
  S_next = Diag(Gam_C) S + Khat^T U,   Khat_i = kap_i o Gam_C / Gam_t(i)
With M = (I + A)^{-1}:
  U = T' V - W S,   W = M Diag(b') (lam o Gam)  [L x d_k],   T'[:, t] = M[:, 2t+1] b'_{2t+1}  [L x C]
so the state and the outputs are affine in S with chunk-constant factors
("Phi form", used by the kernels):
  S_next = (Diag(Gam_C) + Phi') S + Psi V,   Phi' = -Khat^T W,   Psi = Khat^T T'
  O      = Qhat S + Phat V,                  Qhat = (q o Gam) - P W,   Phat = P T'

Range-safe evaluation (what the kernels do): the decay ratio is split per
channel around r = G_C / 2,
  Kl = lam o e^{G - r},  Kr = kap o e^{r - G},  Ql = q o e^{G - r},
  A = Diag(b') strict_lower(Kl Kr^T),  P = causal(Ql Kr^T),
and every exported factor is re-scaled by e^r:  lam o Gam = Kl Diag(e^r),
Khat = Kr Diag(e^r),  q o Gam = Ql Diag(e^r).  A chunk whose decay exceeds a
threshold in some channel (a "wide" chunk) forms A and P element-wise from
e^{G_j - G_i} instead, never splitting the exponent.

Padding: a ragged last chunk is padded with zero keys and queries, alpha = 1
and zero gates, which are identity sub-steps; `chunk_forward` pads exactly as
the kernels do.

Segments (`segmented_forward`): the chunk maps S -> (Diag(Gam_C) + Phi') S +
Psi V compose, so over a run of chunks ("segment" s) S_out = M_s S_in + N_s,
with M_s the product of the chunk maps' linear parts and N_s the end state
from a zero start.  Walking segments 0 .. P-2 on the augmented state [M | N]
from [I | 0] (the M columns take no value term), taking the prefix
S_in(s + 1) = M_s S_in(s) + N_s, and then walking every segment from its
start state gives the sequential result exactly (up to rounding).
"""
from __future__ import annotations

import numpy as np


def substeps_eda(q, k, e, v, alpha, beta, gamma):
    """Doubled sequence of one head (EDA): inputs [T, d] / [T]; returns
    read keys, write keys [2T, dk], gates b' [2T], values nu [2T, dv], the
    per-token log-decay [T, dk] and the queries [T, dk]."""
    T, dk = q.shape
    lam = np.empty((2 * T, dk))
    lam[0::2], lam[1::2] = e, k
    bp = np.empty(2 * T)
    bp[0::2], bp[1::2] = gamma, beta
    nu = np.zeros((2 * T, v.shape[1]))
    nu[1::2] = v
    return dict(lam=lam, kap=lam.copy(), bp=bp, nu=nu, logdec=np.log(alpha), q=np.asarray(q, float))


def substeps_dplr(q, k, a, v, alpha):
    """Doubled sequence of the rank-1 DPLR update S_t = (I - k_t a_t^T) Diag(alpha_t) S + k_t v_t^T
    (QED slides, GDN-2 and QED frames): the erase sub-step only decays, the
    delta sub-step reads along a and writes along k with b' = 1."""
    T, dk = q.shape
    lam = np.zeros((2 * T, dk))
    kap = np.zeros((2 * T, dk))
    lam[1::2], kap[1::2] = a, k
    bp = np.zeros(2 * T)
    bp[1::2] = 1.0
    nu = np.zeros((2 * T, v.shape[1]))
    nu[1::2] = v
    return dict(lam=lam, kap=kap, bp=bp, nu=nu, logdec=np.log(alpha), q=np.asarray(q, float))


def chunk_factors(lam, kap, bp, logdec, q, *, wide_log=None):
    """State-independent factors of one chunk (C tokens, L = 2C sub-steps).

    lam, kap: [L, dk]; bp: [L]; logdec: [C, dk] natural-log decay per token;
    q: [C, dk].  `wide_log` (natural log, negative) is the decay threshold
    below which the chunk is "wide" (element-wise A and P, no split); None
    means never wide.  Returns the intermediate and exported factors."""
    L, dk = lam.shape
    C = L // 2
    G = np.cumsum(logdec, axis=0)               # [C, dk]
    Gs = np.repeat(G, 2, axis=0)                # per sub-step (both sub-steps of a token share it)
    GC = G[-1]
    wide = wide_log is not None and bool(np.any(GC < wide_log))
    jj, ii = np.meshgrid(np.arange(L), np.arange(L), indexing="ij")
    tt, si = np.meshgrid(np.arange(C), np.arange(L), indexing="ij")
    causal = si <= 2 * tt + 1                    # P_ti kept for i <= 2t + 1
    if not wide:
        r = GC / 2.0
        Kl = lam * np.exp(Gs - r)
        Kr = kap * np.exp(r - Gs)
        Ql = q * np.exp(G - r)
        A = np.where(jj > ii, bp[:, None] * (Kl @ Kr.T), 0.0)
        P = np.where(causal, Ql @ Kr.T, 0.0)
        er = np.exp(r)
    else:
        # element-wise: e^{G_j - G_i} per channel, never split
        ratio_A = np.exp(Gs[:, None, :] - Gs[None, :, :])              # [L, L, dk]
        A = np.where(jj > ii, bp[:, None] * np.einsum("jc,ic,jic->ji", lam, kap, ratio_A), 0.0)
        ratio_P = np.exp(G[:, None, :] - Gs[None, :, :])               # [C, L, dk]
        P = np.where(causal, np.einsum("tc,ic,tic->ti", q, kap, ratio_P), 0.0)
        r = np.zeros(dk)
        Kl = lam * np.exp(Gs)
        Kr = kap * np.exp(GC - Gs)
        Ql = q * np.exp(G)
        er = np.ones(dk)
    M = np.linalg.inv(np.eye(L) + A)
    W = M @ (bp[:, None] * Kl)                  # W Diag(e^r) = M Diag(b') (lam o Gam)
    Ws = W * er                                 # natural-unit W
    Tp = (M * bp[None, :])[:, 1::2]             # [L, C]
    Kh = Kr * er                                # Khat = kap o Gam_C / Gam
    Qt = Ql * er                                # q o Gam
    Qh = Qt - P @ Ws
    Ph = P @ Tp
    dec = np.exp(GC)
    Phi = -Kh.T @ Ws                            # Phi' = -Khat^T W      [dk, dk]
    Psi = Kh.T @ Tp                             # Psi  =  Khat^T T'     [dk, C]
    return dict(G=G, r=r, wide=wide, Kl=Kl, Kr=Kr, Ql=Ql, A=A, P=P, M=M, W=Ws, Tp=Tp, Kh=Kh,
                Qh=Qh, Ph=Ph, dec=dec, Phi=Phi, Psi=Psi)


def _pad_chunk(x, C, fill):
    n = x.shape[0]
    if n == C:
        return x
    pad = np.full((C - n,) + x.shape[1:], fill, dtype=float)
    return np.concatenate([x, pad], axis=0)


def chunk_forward(sub, S0, C, *, form="phi", wide_log=None):
    """Chunked forward of one head from its doubled sequence `sub` (see
    substeps_*), chunk size C tokens, initial state S0 [dk, dv] (or None).
    form = "u" (U = T'V - W S, O = Qhat S + Phat V, S_next = Gam_C S + Khat^T U)
    or "phi" (S_next = Gam_C S + Phi' S + Psi V, same O).  Returns (o [T, dv],
    S_final [dk, dv], list of per-chunk factors)."""
    T, dk = sub["q"].shape
    dv = sub["nu"].shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=float)
    outs, facs = [], []
    for t0 in range(0, T, C):
        n = min(C, T - t0)
        sl = slice(2 * t0, 2 * (t0 + n))
        lam = _pad_chunk(sub["lam"][sl], 2 * C, 0.0)
        kap = _pad_chunk(sub["kap"][sl], 2 * C, 0.0)
        bp = _pad_chunk(sub["bp"][sl], 2 * C, 0.0)
        nu = _pad_chunk(sub["nu"][sl], 2 * C, 0.0)
        logdec = _pad_chunk(sub["logdec"][t0:t0 + n], C, 0.0)
        q = _pad_chunk(sub["q"][t0:t0 + n], C, 0.0)
        f = chunk_factors(lam, kap, bp, logdec, q, wide_log=wide_log)
        V = nu[1::2]                                # values of the delta sub-steps [C, dv]
        O = f["Qh"] @ S + f["Ph"] @ V
        if form == "u":
            U = f["Tp"] @ V - f["W"] @ S
            S = f["dec"][:, None] * S + f["Kh"].T @ U
        else:
            S = f["dec"][:, None] * S + f["Phi"] @ S + f["Psi"] @ V
        outs.append(O[:n])
        facs.append(f)
    return np.concatenate(outs, axis=0), S, facs


def _chunk_list(sub, C, wide_log=None):
    """Per-chunk factors and values (padded as the kernels pad)."""
    T = sub["q"].shape[0]
    out = []
    for t0 in range(0, T, C):
        n = min(C, T - t0)
        sl = slice(2 * t0, 2 * (t0 + n))
        lam = _pad_chunk(sub["lam"][sl], 2 * C, 0.0)
        kap = _pad_chunk(sub["kap"][sl], 2 * C, 0.0)
        bp = _pad_chunk(sub["bp"][sl], 2 * C, 0.0)
        nu = _pad_chunk(sub["nu"][sl], 2 * C, 0.0)
        logdec = _pad_chunk(sub["logdec"][t0:t0 + n], C, 0.0)
        q = _pad_chunk(sub["q"][t0:t0 + n], C, 0.0)
        out.append((chunk_factors(lam, kap, bp, logdec, q, wide_log=wide_log), nu[1::2], n))
    return out


def segmented_forward(sub, S0, C, P, *, wide_log=None):
    """The chunked forward with the chunks of the head cut into P segments of
    ceil(NC / P) chunks (the last may be shorter): segment maps on the
    augmented state, their prefix, then each segment's pass with outputs.
    Returns (o [T, dv], S_final, [(M_s, N_s)])."""
    dk = sub["q"].shape[1]
    dv = sub["nu"].shape[1]
    chunks = _chunk_list(sub, C, wide_log)
    NC = len(chunks)
    ncs = -(-NC // P)
    segs = [chunks[i:i + ncs] for i in range(0, NC, ncs)]
    # maps of every segment but the last: [M | N] from [I | 0]
    maps = []
    for seg in segs[:-1]:
        X = np.concatenate([np.eye(dk), np.zeros((dk, dv))], axis=1)
        for f, V, _ in seg:
            Vaug = np.concatenate([np.zeros((V.shape[0], dk)), V], axis=1)
            X = f["dec"][:, None] * X + f["Phi"] @ X + f["Psi"] @ Vaug
        maps.append((X[:, :dk], X[:, dk:]))
    # prefix of start states
    starts = [np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=float)]
    for M, N in maps:
        starts.append(M @ starts[-1] + N)
    outs = []
    S = None
    for seg, S in zip(segs, starts):
        S = S.copy()
        for f, V, n in seg:
            O = f["Qh"] @ S + f["Ph"] @ V
            S = f["dec"][:, None] * S + f["Phi"] @ S + f["Psi"] @ V
            outs.append(O[:n])
    return np.concatenate(outs, axis=0), S, maps
