"""GPU parity of the rank-1 DPLR update (eda_fwd_chunked_dplr,
eda_fwd_recurrent_step_dplr) -- the GDN-2 / QED state update -- against the
fp64 oracle (oracle.eda_ref_dplr_fwd) on the same inputs.  The erase vector a
and the gated value w o v are formed here, in the test, and handed to both
sides.  Same tolerances as the EDA forward."""
import numpy as np
import pytest
import torch

import oracle
import recurrent_memory_amd as eda
from eda_inputs import WORKLOADS, make_dplr_inputs
from _helpers import check, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"[case] {msg}", flush=True)


def prepare(x, qed=True):
    """a = b o k (+ lam (b o q - k (k . (b o q))) for QED), v' = w o v, in the inputs' dtype."""
    td = x["q"].dtype
    q, k, b = x["q"].float(), x["k"].float(), x["b"]
    a = b * k
    if qed:
        u = b * q
        a = a + x["lam"].view(1, 1, -1, 1) * (u - k * (k * u).sum(-1, keepdim=True))
    return dict(q=x["q"], k=x["k"], a=a.to(td), v=(x["w"] * x["v"].float()).to(td), alpha=x["alpha"],
                S0=x["S0"])


def gpu_dplr(y, chunk=0):
    yd = {n: (None if t is None else t.to(DEV)) for n, t in y.items()}
    o, S = eda.fwd_chunked_dplr(yd["q"], yd["k"], yd["a"], yd["v"], yd["alpha"], yd["S0"], chunk=chunk)
    torch.cuda.synchronize()
    return o, S


def ref_dplr(y):
    return oracle.eda_ref_dplr_fwd(y["q"], y["k"], y["a"], y["v"], y["alpha"], y["S0"])


@pytest.mark.parametrize("dtype,B,T,H,dk,dv,chunk,qed", [
    ("f32", 1, 64, 2, 16, 16, 16, True),
    ("f32", 2, 45, 1, 31, 7, 32, False),
    ("bf16", 2, 200, 2, 128, 128, 32, True),
    ("bf16", 1, 333, 2, 128, 128, 16, True),
    ("bf16", 1, 150, 3, 64, 64, 32, False),
    ("bf16", 1, 100, 2, 100, 80, 32, True),     # element-wise loads (d_k < 128)
    ("f32", 1, 130, 2, 32, 16, 64, True),
    ("bf16", 2, 200, 2, 128, 128, 64, True),
    ("bf16", 1, 190, 3, 64, 64, 64, False),
    ("bf16", 1, 140, 2, 100, 80, 64, True),
    ("bf16", 1, 32 * 520 + 9, 2, 128, 128, 32, True),  # the state pass in 8 segments
])
def test_dplr_chunked(dtype, B, T, H, dk, dv, chunk, qed):
    say(f"dplr chunked {dtype} B={B} T={T} H={H} dk={dk} dv={dv} chunk={chunk} qed={qed}")
    y = prepare(make_dplr_inputs(B, T, H, dk, dv, dtype, seed=T + dk, s0_std=0.02), qed)
    o, S = gpu_dplr(y, chunk)
    ro, rS = ref_dplr(y)
    check(to64(o), to64(S), ro, rS, dtype, f"dplr B={B} T={T} H={H} dk={dk} qed={qed}")


def test_dplr_fast_decay_wide_chunks():
    # alpha = e^-5 everywhere: 32 tokens decay by e^-160, past the split-exponent
    # range, so every chunk takes the element-wise path
    say("dplr chunked bf16 with alpha = e^-5")
    x = make_dplr_inputs(1, 128, 2, 128, 128, "bf16", seed=3)
    x["alpha"] = torch.full_like(x["alpha"], float(np.exp(-5.0)))
    y = prepare(x)
    o, S = gpu_dplr(y)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    ro, rS = ref_dplr(y)
    check(to64(o), to64(S), ro, rS, "bf16", "dplr alpha floor")


def test_dplr_gamma_zero_eda_agrees():
    # GPU cross-check: EDA with gamma = 0 is the DPLR update with a = beta k and v -> beta v
    say("dplr vs eda with gamma = 0")
    from eda_inputs import make_inputs
    x = make_inputs(2, 130, 2, 128, 128, "f32", seed=4)
    xd = {n: (None if t is None else t.to(DEV)) for n, t in x.items()}
    zero = torch.zeros_like(xd["gamma"])
    o1, S1 = eda.fwd_chunked(xd["q"], xd["k"], xd["e"], xd["v"], xd["alpha"], xd["beta"], zero)
    bk = (xd["beta"][..., None] * xd["k"]).contiguous()
    bv = (xd["beta"][..., None] * xd["v"]).contiguous()
    o2, S2 = eda.fwd_chunked_dplr(xd["q"], xd["k"], bk, bv, xd["alpha"])
    torch.cuda.synchronize()
    assert float((o1 - o2).abs().max()) <= 1e-4 and float((S1 - S2).abs().max()) <= 1e-4


def test_train_qed_workload_sampled():
    w = WORKLOADS["train_qed"]
    say(f"train_qed full size B={w.B} T={w.T} H={w.H}")
    y = prepare(make_dplr_inputs(w.B, w.T, w.H, w.dk, w.dv, w.dtype, seed=w.seed, device=DEV))
    o, S = eda.fwd_chunked_dplr(y["q"], y["k"], y["a"], y["v"], y["alpha"], y["S0"])
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    rng = np.random.default_rng(4)
    heads = sorted({(int(rng.integers(w.B)), int(rng.integers(w.H))) for _ in range(6)})
    go, gs, ro, rs = [], [], [], []
    for b, h in heads:
        sl = lambda t: t[b:b + 1, :, h:h + 1].cpu()
        r_o, r_S = oracle.eda_ref_dplr_fwd(sl(y["q"]), sl(y["k"]), sl(y["a"]), sl(y["v"]), sl(y["alpha"]))
        go.append(to64(o[b, :, h])); ro.append(r_o[0, :, 0])
        gs.append(to64(S[b, h])); rs.append(r_S[0, 0])
    check(np.concatenate(go), np.concatenate(gs), np.concatenate(ro), np.concatenate(rs), "bf16",
          f"train_qed heads={heads}")


@pytest.mark.parametrize("dtype,dk,dv", [("f32", 48, 40), ("bf16", 128, 128)])
def test_dplr_decode_steps(dtype, dk, dv):
    say(f"dplr decode {dtype} dk={dk} dv={dv}")
    steps, N, H = 6, 5, 3
    y = prepare(make_dplr_inputs(steps, N, H, dk, dv, dtype, seed=30 + dk, s0_std=0.0))
    S0 = 0.02 * torch.randn((N, H, dk, dv), generator=torch.Generator().manual_seed(8))
    yd = {n: (None if t is None else t.to(DEV)) for n, t in y.items()}
    S = S0.to(DEV)
    outs = []
    for t in range(steps):
        o, S = eda.recurrent_step_dplr(yd["q"][t], yd["k"][t], yd["a"][t], yd["v"][t], yd["alpha"][t], S,
                                       inplace=True)
        outs.append(o)
    torch.cuda.synchronize()
    sw = lambda t: np.swapaxes(to64(t), 0, 1)
    r_o, r_S = oracle.eda_ref_dplr_fwd(sw(y["q"]), sw(y["k"]), sw(y["a"]), sw(y["v"]), sw(y["alpha"]), S0)
    check(to64(torch.stack(outs)), to64(S), np.swapaxes(r_o, 0, 1), r_S, dtype, f"dplr decode {dtype}")
