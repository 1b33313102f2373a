"""fp64 CPU oracle for the Erase-then-Delta Attention (EDA) recurrence forward.

TEST INFRASTRUCTURE ONLY: imported by `tests/`, by `__graft_entry__.smoke()`
and by the benchmark's CPU-baseline leg, never by the GPU library or its
Python binding.  It shares no code with the GPU path.

`eda_ref.c` implements the paper's three ordered stages token by token
(EDA paper Sec. 3.3, Eqs. (8)-(13)) in IEEE fp64; this module compiles it
with the system C compiler and passes numpy arrays to it.  Inputs of any
float type are widened to fp64 exactly (bf16 and fp32 values are exactly
representable in fp64).

Every function here is pinned by the `-m "not gpu"` tests in
`tests/test_oracle_pins.py` (hand-worked example, readout identity, expanded
operator, KDA reduction, explicit-matrix and exact-rational brute force,
doubled-sequence form, special cases and invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "eda_ref.c")
_LIB_PATH = os.path.join(_HERE, "libeda_ref.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile eda_ref.c into liboracle (plain gcc, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                        "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.eda_ref_fwd.argtypes = [dp] * 10 + [ctypes.c_long] * 5 + [ctypes.c_int]
        lib.eda_ref_fwd.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor -> numpy (bf16 widened exactly via fp32)
        import torch
        x = x.detach().to("cpu")
        if x.dtype == torch.bfloat16:
            x = x.float()
        x = x.numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def eda_ref_fwd(q, k, e, v, alpha, beta, gamma, S0=None, *, nthreads: Optional[int] = None,
                want_state: bool = True):
    """Token-by-token fp64 EDA forward.

    q, k, e, alpha: [B, T, H, d_k]; v: [B, T, H, d_v]; beta, gamma: [B, T, H];
    S0: [B, H, d_k, d_v] or None (zeros).  Returns (o [B, T, H, d_v],
    S_final [B, H, d_k, d_v] or None), both fp64 numpy arrays.
    """
    q, k, e, v, alpha, beta, gamma, S0 = map(_f64, (q, k, e, v, alpha, beta, gamma, S0))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    for name, a, shp in (("k", k, (B, T, H, dk)), ("e", e, (B, T, H, dk)),
                         ("v", v, (B, T, H, dv)), ("alpha", alpha, (B, T, H, dk)),
                         ("beta", beta, (B, T, H)), ("gamma", gamma, (B, T, H))):
        if a.shape != shp:
            raise ValueError(f"oracle: {name} has shape {a.shape}, expected {shp}")
    if S0 is not None and S0.shape != (B, H, dk, dv):
        raise ValueError(f"oracle: S0 has shape {S0.shape}, expected {(B, H, dk, dv)}")
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    S_final = np.zeros((B, H, dk, dv), dtype=np.float64) if want_state else None
    nt = nthreads or default_threads()
    rc = _load().eda_ref_fwd(_ptr(q), _ptr(k), _ptr(e), _ptr(v), _ptr(alpha), _ptr(beta),
                             _ptr(gamma), _ptr(S0), _ptr(o), _ptr(S_final),
                             B, T, H, dk, dv, int(nt))
    if rc != 0:
        raise RuntimeError("oracle: eda_ref_fwd failed")
    return o, S_final


def eda_ref_decode(q, k, e, v, alpha, beta, gamma, S0, *, nthreads: Optional[int] = None):
    """A sequence of one-token steps with the state carried between them.

    Inputs are stacked per step: q, k, e, alpha: [steps, N, H, d_k]; v:
    [steps, N, H, d_v]; beta, gamma: [steps, N, H]; S0: [N, H, d_k, d_v] or
    None.  Each (n, h) is one head run over `steps` tokens, so this is the
    same recurrence with the step axis as time; the arrays are only
    re-ordered (no arithmetic).  Returns (o [steps, N, H, d_v], S_final).
    """
    sw = lambda x: None if x is None else np.swapaxes(_f64(x), 0, 1)
    o, S = eda_ref_fwd(sw(q), sw(k), sw(e), sw(v), sw(alpha), sw(beta), sw(gamma),
                       _f64(S0), nthreads=nthreads)
    return np.ascontiguousarray(np.swapaxes(o, 0, 1)), S


# ---------------------------------------------------------------------------
# Layer prologue: safe decay gate, L2 normalisation of q, k, e, grouped value
# heads.  Plain fp64 numpy, written out from the definitions; the recurrence
# itself is eda_ref_fwd above.
# ---------------------------------------------------------------------------
SAFE_GATE_FLOOR = -5.0   # the lower bound l of the log-retention (EDA paper, Eqs. (14)-(15))
L2NORM_EPS = 1e-6        # x / max(||x||, eps): the pages do not state an epsilon


def softplus(x):
    """log(1 + e^x) in fp64 (the stable split max(x, 0) + log1p(e^-|x|))."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def eda_ref_safe_gate(a, A_log, dt_bias, ell: float = SAFE_GATE_FLOOR):
    """Retention alpha from the safe decay gate (EDA paper Eqs. (14)-(15); slides
    frame "EDA also changes the safe decay parameterization"):

        A = exp(A_log),  Delta_t = softplus(a_t + b_Delta),
        g_t = l + (-l) exp(-(A / |l|) Delta_t),  alpha_t = exp(g_t),

    element-wise per key channel.  a: [..., H, d_k]; A_log, dt_bias: [H, d_k]
    (broadcast over the leading axes).  Returns alpha (fp64), in (e^l, 1].
    """
    a, A_log, dt_bias = _f64(a), _f64(A_log), _f64(dt_bias)
    A = np.exp(A_log)
    delta = softplus(a + dt_bias)
    g = ell + (-ell) * np.exp(-(A / abs(ell)) * delta)
    return np.exp(g)


def eda_ref_l2norm(x, eps: float = L2NORM_EPS):
    """x / max(||x||_2, eps) over the last axis (the layer's normalisation of
    q, k and e; EDA paper Fig. 1)."""
    x = _f64(x)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, eps)


def expand_key_heads(x, H_v: int):
    """Key-head tensor [B, T, H_k, ...] -> value-head tensor [B, T, H_v, ...]:
    value head h reads key head h // (H_v / H_k) (grouped value heads, EDA paper
    Appendix, model table)."""
    x = _f64(x)
    H_k = x.shape[2]
    if H_v % H_k:
        raise ValueError(f"oracle: H_v={H_v} is not a multiple of H_k={H_k}")
    return np.repeat(x, H_v // H_k, axis=2)


def eda_ref_fwd_layer(q, k, e, v, a, A_log, dt_bias, beta, gamma, S0=None, *,
                      nthreads: Optional[int] = None, want_state: bool = True):
    """The kernel-level EDA forward with its layer prologue:

    q, k, e, a: [B, T, H_k, d_k] raw (unnormalised) queries, keys, erase
    addresses and decay inputs; v: [B, T, H_v, d_v]; A_log, dt_bias: [H_k, d_k];
    beta, gamma: [B, T, H_v]; S0: [B, H_v, d_k, d_v] or None.  q, k, e are
    L2-normalised per token and head, alpha comes from the safe gate, key heads
    are shared by H_v / H_k value heads, then the token recurrence runs per
    value head.  Returns (o [B, T, H_v, d_v], S_final).
    """
    v = _f64(v)
    H_v = v.shape[2]
    qn, kn, en = (expand_key_heads(eda_ref_l2norm(x), H_v) for x in (q, k, e))
    alpha = expand_key_heads(eda_ref_safe_gate(a, A_log, dt_bias), H_v)
    return eda_ref_fwd(qn, kn, en, v, alpha, beta, gamma, S0, nthreads=nthreads, want_state=want_state)


# ---------------------------------------------------------------------------
# Second workload: the rank-1 DPLR update of GDN-2 and QED (QED slides, frames
# "GDN-2 separates decay, erase, and write" and "QED adds a query term to the
# erase vector").  Plain fp64 numpy, token by token, vectorised over heads.
# ---------------------------------------------------------------------------
def gdn2_erase_vector(k, b):
    """a_t = b_t o k_t (GDN-2's erase vector: a channel-gated key)."""
    return _f64(b) * _f64(k)


def qed_erase_vector(q, k, b, lam):
    """QED's erase vector: u = b o q, d = u - k (k . u) (the gated query with
    its component along the unit key removed, gate first, then projection),
    a = b o k + lam d.  q, k, b: [..., d_k]; lam: scalar or broadcastable."""
    q, k, b = _f64(q), _f64(k), _f64(b)
    u = b * q
    d = u - k * np.sum(k * u, axis=-1, keepdims=True)
    lam = np.asarray(lam, dtype=np.float64)
    return b * k + (lam[..., None] if lam.ndim else lam) * d


def eda_ref_dplr_fwd(q, k, a, v, alpha, S0=None, want_state: bool = True):
    """Token-by-token fp64 forward of the rank-1 DPLR recurrence

        Sbar_t = Diag(alpha_t) S_{t-1},   S_t = Sbar_t + k_t (v_t - Sbar_t^T a_t)^T,   o_t = S_t^T q_t,

    i.e. S_t = (I - k_t a_t^T) Diag(alpha_t) S_{t-1} + k_t v_t^T.  v stands for
    the gated value w o v of GDN-2/QED.  q, k, a, alpha: [B, T, H, d_k];
    v: [B, T, H, d_v]; S0: [B, H, d_k, d_v] or None.  Returns (o, S_final)."""
    q, k, a, v, alpha = map(_f64, (q, k, a, v, alpha))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else _f64(S0).copy()
    o = np.zeros((B, T, H, dv))
    for t in range(T):
        Sb = alpha[:, t, :, :, None] * S                             # decay rows (key channels)
        r = v[:, t] - np.einsum("bhkv,bhk->bhv", Sb, a[:, t])         # residual to write
        S = Sb + k[:, t, :, :, None] * r[:, :, None, :]               # write along k
        o[:, t] = np.einsum("bhkv,bhk->bhv", S, q[:, t])              # read the new state
    return o, (S if want_state else None)


# ---------------------------------------------------------------------------
# Backward pass: fp64 gradients of the token recurrence.  The forward is the
# three ordered stages of eda_ref_fwd written out once more in fp64 torch
# (EDA paper Sec. 3.3, Eqs. (9)-(13)), and the adjoint is taken by reverse-mode
# automatic differentiation of exactly that computation -- a library
# primitive standing in for the hand-derived reverse recurrence.  Pinned by
# finite differences of the C oracle and by closed forms.
# ---------------------------------------------------------------------------
def eda_ref_bwd(q, k, e, v, alpha, beta, gamma, S0, dO, dS_final=None):
    """Gradients of L = <o, dO> + <S_final, dS_final> (o = eda_ref_fwd's
    outputs) with respect to q, k, e, v, alpha, beta, gamma and S0 (S0 = None
    means zeros, and its gradient is still returned).  Shapes as for
    eda_ref_fwd; dO: [B, T, H, d_v]; dS_final: [B, H, d_k, d_v] or None.
    Returns a dict of fp64 numpy arrays keyed dq, dk, de, dv, dalpha, dbeta,
    dgamma, dS0."""
    import torch

    names = ("q", "k", "e", "v", "alpha", "beta", "gamma")
    x = {n: torch.tensor(_f64(a), dtype=torch.float64, requires_grad=True)
         for n, a in zip(names, (q, k, e, v, alpha, beta, gamma))}
    B, T, H, dk = x["q"].shape
    dv = x["v"].shape[-1]
    S0t = torch.zeros((B, H, dk, dv), dtype=torch.float64) if S0 is None else \
        torch.tensor(_f64(S0), dtype=torch.float64)
    S0t.requires_grad_(True)
    S = S0t
    outs = []
    for t in range(T):
        qt, kt, et, vt = (x[n][:, t] for n in ("q", "k", "e", "v"))
        Sh = x["alpha"][:, t, :, :, None] * S                                   # decay
        re = torch.einsum("bhkv,bhk->bhv", Sh, et)
        St = Sh - x["gamma"][:, t, :, None, None] * et[..., None] * re[..., None, :]   # erase
        rk = torch.einsum("bhkv,bhk->bhv", St, kt)
        S = St + x["beta"][:, t, :, None, None] * kt[..., None] * (vt - rk)[..., None, :]   # write
        outs.append(torch.einsum("bhkv,bhk->bhv", S, qt))                       # read
    o = torch.stack(outs, dim=1)
    loss = (o * torch.tensor(_f64(dO))).sum()
    if dS_final is not None:
        loss = loss + (S * torch.tensor(_f64(dS_final))).sum()
    loss.backward()
    g = {"d" + n: x[n].grad.numpy() for n in names}
    g["dS0"] = S0t.grad.numpy()
    return g
