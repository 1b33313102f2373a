"""GPU parity of the backward pass (eda_bwd) against the fp64 oracle's
adjoint (oracle.eda_ref_bwd) on the same inputs and output gradients.

Tolerances: the backward computes in fp32 from exactly representable
inputs, so fp32 inputs are held to max |gpu - oracle| <= 1e-4 * max(1,
max |oracle|) per gradient, and bf16 inputs to the forward's relative
Frobenius bound 5e-3 per gradient tensor."""
import numpy as np
import pytest
import torch

import oracle
import recurrent_memory_amd as eda
from eda_inputs import make_inputs
from _helpers import rel_frob, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GRADS = ("dq", "dk", "de", "dv", "dalpha", "dbeta", "dgamma", "dS0")


def say(msg):
    print(f"[case] {msg}", flush=True)


def run_case(B, T, H, dk, dv, dtype, seed, s0=True, dsf=True):
    x = make_inputs(B, T, H, dk, dv, dtype, seed=seed, s0_std=0.05 if s0 else 0.0)
    g = torch.Generator().manual_seed(seed + 99)
    dO = torch.randn((B, T, H, dv), generator=g).to(x["q"].dtype)
    dS = torch.randn((B, H, dk, dv), generator=g) if dsf else None
    xd = {n: (None if t is None else t.to(DEV)) for n, t in x.items()}
    got = eda.backward(xd["q"], xd["k"], xd["e"], xd["v"], xd["alpha"], xd["beta"], xd["gamma"], xd["S0"],
                       dO.to(DEV), None if dS is None else dS.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.eda_ref_bwd(x["q"], x["k"], x["e"], x["v"], x["alpha"], x["beta"], x["gamma"], x["S0"], dO, dS)
    return got, ref


def check_grads(got, ref, dtype, label):
    for n in GRADS:
        g, r = to64(got[n]), ref[n]
        assert np.all(np.isfinite(g)), f"{label} {n} not finite"
        if dtype == "f32":
            err = float(np.max(np.abs(g - r)))
            lim = 1e-4 * max(1.0, float(np.max(np.abs(r))))
            assert err <= lim, f"{label} {n}: max-abs {err:.3e} > {lim:.3e}"
        else:
            err = rel_frob(g, r)
            assert err <= 5e-3, f"{label} {n}: rel-frob {err:.3e}"
        print(f"[parity] {label} {n} {err:.3e}", flush=True)


@pytest.mark.parametrize("dtype,B,T,H,dk,dv,s0,dsf", [
    ("f32", 1, 20, 2, 16, 16, True, True),
    ("f32", 2, 13, 1, 31, 20, True, False),      # ragged segment, two value slices, padded rows
    ("f32", 1, 9, 1, 2, 1, False, True),
    ("f32", 1, 3, 2, 16, 16, True, True),        # shorter than one input segment
    ("bf16", 2, 70, 2, 128, 128, True, True),
    ("bf16", 1, 40, 3, 64, 48, False, False),
])
def test_bwd_parity(dtype, B, T, H, dk, dv, s0, dsf):
    say(f"bwd {dtype} B={B} T={T} H={H} dk={dk} dv={dv} S0={s0} dS_final={dsf}")
    got, ref = run_case(B, T, H, dk, dv, dtype, seed=T * 7 + dk, s0=s0, dsf=dsf)
    check_grads(got, ref, dtype, f"bwd {dtype} T={T} dk={dk} dv={dv}")


def test_bwd_without_dS0_output():
    say("bwd without dS0")
    x = make_inputs(1, 16, 1, 16, 16, "f32", seed=3)
    xd = {n: (None if t is None else t.to(DEV)) for n, t in x.items()}
    dO = torch.randn((1, 16, 1, 16), device=DEV)
    g1 = eda.backward(xd["q"], xd["k"], xd["e"], xd["v"], xd["alpha"], xd["beta"], xd["gamma"], None, dO,
                      want_dS0=False)
    g2 = eda.backward(xd["q"], xd["k"], xd["e"], xd["v"], xd["alpha"], xd["beta"], xd["gamma"], None, dO)
    torch.cuda.synchronize()
    assert g1["dS0"] is None
    for n in GRADS[:-1]:
        assert torch.equal(g1[n], g2[n])


def test_bwd_train_shape_sampled():
    # the training shape at full size; the oracle checks two sampled heads
    B, T, H, d = 4, 2048, 16, 128
    say(f"bwd bf16 full size B={B} T={T} H={H}")
    x = make_inputs(B, T, H, d, d, "bf16", seed=1, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(5)
    dO = torch.randn((B, T, H, d), generator=g, device=DEV).to(torch.bfloat16)
    got = eda.backward(x["q"], x["k"], x["e"], x["v"], x["alpha"], x["beta"], x["gamma"], None, dO)
    torch.cuda.synchronize()
    for name in GRADS[:-1]:
        assert torch.isfinite(got[name]).all()
    for (b, h) in [(1, 3), (3, 14)]:
        sl = lambda t: t[b:b + 1, :, h:h + 1].cpu()
        ref = oracle.eda_ref_bwd(sl(x["q"]), sl(x["k"]), sl(x["e"]), sl(x["v"]), sl(x["alpha"]), sl(x["beta"]),
                                 sl(x["gamma"]), None, sl(dO))
        sub = {n: got[n][b:b + 1, :, h:h + 1] for n in GRADS[:-1]}
        sub["dS0"] = got["dS0"][b:b + 1, h:h + 1]
        check_grads(sub, ref, "bf16", f"bwd train head=({b},{h})")
