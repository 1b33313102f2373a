"""Shared helpers for the parity tests (comparison metrics, sampled oracle runs)."""
import numpy as np
import torch

import oracle

# Tolerances: fp32 inputs -> max |gpu - oracle| <= 1e-4 over every element;
# bf16 inputs with fp32 state -> ||gpu - oracle||_F / ||oracle||_F <= 5e-3,
# taken over the whole o tensor and the whole final-state tensor (or over
# every sampled head together at full size).
TOL_F32_MAXABS = 1e-4
TOL_BF16_RELFRO = 5e-3


def to64(x):
    if x is None:
        return None
    return x.detach().float().cpu().double().numpy()


def rel_frob(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def max_abs(got, ref):
    return float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))))


def oracle_heads(x, heads, t_end=None):
    """Run the oracle on selected (b, h) heads of a [B, T, H, d] input set.
    Each head is independent, so slicing it out is exact.  Returns lists of
    (o [T, dv], S_final [dk, dv]) in fp64."""
    outs = []
    for (b, h) in heads:
        sl = lambda t: None if t is None else t[b:b + 1, :t_end, h:h + 1]
        S0 = None if x["S0"] is None else x["S0"][b:b + 1, h:h + 1]
        o, S = oracle.eda_ref_fwd(sl(x["q"]), sl(x["k"]), sl(x["e"]), sl(x["v"]), sl(x["alpha"]),
                                  sl(x["beta"]), sl(x["gamma"]), S0)
        outs.append((o[0, :, 0], S[0, 0]))
    return outs


def check(got_o, got_S, ref_o, ref_S, dtype, label=""):
    """Assert the tolerance for `dtype` ('f32' or 'bf16'); returns the errors."""
    if dtype == "f32":
        eo, es = max_abs(got_o, ref_o), max_abs(got_S, ref_S)
        assert eo <= TOL_F32_MAXABS and es <= TOL_F32_MAXABS, f"{label} max-abs o={eo:.3e} S={es:.3e}"
    else:
        eo, es = rel_frob(got_o, ref_o), rel_frob(got_S, ref_S)
        assert eo <= TOL_BF16_RELFRO and es <= TOL_BF16_RELFRO, f"{label} rel-frob o={eo:.3e} S={es:.3e}"
    print(f"[parity] {label} {dtype} o={eo:.3e} S={es:.3e}", flush=True)
    return eo, es
