"""GPU parity of the layer form (eda_fwd_chunked_layer,
eda_fwd_recurrent_step_layer): safe gate, L2 normalisation of raw q, k, e and
grouped value heads fused in front of the recurrence, against the fp64
oracle's prologue plus token recurrence (oracle.eda_ref_fwd_layer).
Same tolerances as the plain form."""
import numpy as np
import pytest
import torch

import oracle
import recurrent_memory_amd as eda
from eda_inputs import WORKLOADS, make_layer_inputs, make_workload
from _helpers import check, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NAMES = ("q", "k", "e", "v", "a", "A_log", "dt_bias", "beta", "gamma")


def say(msg):
    print(f"[case] {msg}", flush=True)


def dev(x):
    return {n: (None if t is None else t.to(DEV)) for n, t in x.items()}


def run_layer(x, chunk=0):
    o, S = eda.fwd_chunked_layer(*(x[n] for n in NAMES), x["S0"], chunk=chunk)
    torch.cuda.synchronize()
    return o, S


def ref_layer(x):
    return oracle.eda_ref_fwd_layer(*(x[n] for n in NAMES), x["S0"])


CASES = [
    # dtype, B, T, H_k, H_v, d_k, d_v, chunk
    ("f32", 1, 64, 1, 1, 16, 16, 16),
    ("f32", 2, 70, 1, 2, 16, 16, 32),
    ("f32", 1, 45, 2, 4, 31, 7, 16),
    ("bf16", 2, 100, 2, 4, 128, 128, 32),
    ("bf16", 1, 333, 1, 2, 128, 128, 16),
    ("bf16", 1, 200, 2, 2, 64, 64, 32),
    ("bf16", 1, 130, 1, 3, 100, 80, 32),     # d_k < 128: the element-wise load path
    ("f32", 1, 150, 1, 2, 64, 48, 64),
    ("bf16", 2, 200, 2, 4, 128, 128, 64),
    ("bf16", 1, 129, 1, 2, 64, 64, 64),
    ("bf16", 1, 140, 1, 3, 100, 80, 64),
    ("bf16", 1, 64 * 260 + 3, 1, 2, 128, 128, 64),  # the state pass in 4 segments
]


@pytest.mark.parametrize("dtype,B,T,Hk,Hv,dk,dv,chunk", CASES)
def test_layer_chunked(dtype, B, T, Hk, Hv, dk, dv, chunk):
    say(f"layer chunked {dtype} B={B} T={T} Hk={Hk} Hv={Hv} dk={dk} dv={dv} chunk={chunk}")
    x = make_layer_inputs(B, T, Hk, Hv, dk, dv, dtype, seed=B * 1000 + T + Hv, s0_std=0.02)
    o, S = run_layer(dev(x), chunk=chunk)
    ro, rS = ref_layer(x)
    check(to64(o), to64(S), ro, rS, dtype, f"layer B={B} T={T} Hk={Hk} Hv={Hv} dk={dk}")


def test_layer_unaligned_inputs():
    # q at a 2-byte offset: the factor kernel reads element-wise
    say("layer chunked bf16, q at a 2-byte offset")
    x = make_layer_inputs(1, 96, 2, 4, 128, 128, "bf16", seed=77)
    xd = dev(x)
    buf = torch.empty(xd["q"].numel() + 1, dtype=torch.bfloat16, device=DEV)
    buf[1:].copy_(xd["q"].flatten())
    xd["q"] = buf[1:].view(xd["q"].shape)
    assert xd["q"].data_ptr() % 16 != 0
    o, S = run_layer(xd)
    ro, rS = ref_layer(x)
    check(to64(o), to64(S), ro, rS, "bf16", "layer unaligned q")


@pytest.mark.parametrize("chunk", [32, 64])
def test_layer_gate_floor_wide_chunks(chunk):
    # every retention at the safe gate's floor e^-5: 32 tokens decay by e^-160,
    # past the split-exponent range, so every chunk takes the element-wise path
    say(f"layer chunked bf16 at the gate floor chunk={chunk}")
    x = make_layer_inputs(1, 160, 1, 2, 128, 128, "bf16", seed=5)
    x["a"] = torch.full_like(x["a"], 40.0)
    x["A_log"] = torch.full_like(x["A_log"], float(np.log(16.0)))
    al = oracle.eda_ref_safe_gate(x["a"], x["A_log"], x["dt_bias"])
    assert np.allclose(al, np.exp(-5.0), rtol=1e-6)
    o, S = run_layer(dev(x), chunk=chunk)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    ro, rS = ref_layer(x)
    check(to64(o), to64(S), ro, rS, "bf16", "layer gate floor")


def test_layer_equals_plain_form_on_prepared_inputs():
    # H_k = H_v, q, k, e given unit-norm in bf16 and the gate replaced by its
    # alpha: the two entry points see the same recurrence
    say("layer vs plain form")
    x = make_layer_inputs(2, 96, 2, 2, 128, 128, "bf16", seed=9)
    o1, S1 = run_layer(dev(x))
    alpha = torch.from_numpy(oracle.eda_ref_safe_gate(x["a"], x["A_log"], x["dt_bias"])).float()
    xn = {n: torch.from_numpy(oracle.eda_ref_l2norm(x[n])).float() for n in ("q", "k", "e")}
    ref_o, ref_S = oracle.eda_ref_fwd(xn["q"], xn["k"], xn["e"], x["v"], alpha, x["beta"], x["gamma"])
    check(to64(o1), to64(S1), ref_o, ref_S, "bf16", "layer vs plain oracle")
    # the plain form takes the prepared q, k, e in bf16: its oracle reads those rounded values
    xb = {n: xn[n].bfloat16() for n in ("q", "k", "e")}
    rb_o, rb_S = oracle.eda_ref_fwd(xb["q"], xb["k"], xb["e"], x["v"], alpha, x["beta"], x["gamma"])
    xd = dev(dict(v=x["v"], alpha=alpha, beta=x["beta"], gamma=x["gamma"], **xb))
    o2, S2 = eda.fwd_chunked(xd["q"], xd["k"], xd["e"], xd["v"], xd["alpha"], xd["beta"], xd["gamma"])
    torch.cuda.synchronize()
    check(to64(o2), to64(S2), rb_o, rb_S, "bf16", "plain on prepared inputs")


def test_train_layer_workload_sampled():
    w = WORKLOADS["train_layer"]
    say(f"train_layer full size B={w.B} T={w.T} Hk={w.hk} Hv={w.H}")
    x = make_workload(w, device=DEV)
    o, S = run_layer(x)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    xc = {n: (None if t is None else t.cpu()) for n, t in x.items()}
    rng = np.random.default_rng(3)
    heads = sorted({(int(rng.integers(w.B)), int(rng.integers(w.H))) for _ in range(6)})
    grp = w.H // w.hk
    go, gs, ro, rs = [], [], [], []
    for b, h in heads:
        hk = h // grp
        ks = lambda t: t[b:b + 1, :, hk:hk + 1]
        vs = lambda t: t[b:b + 1, :, h:h + 1]
        r_o, r_S = oracle.eda_ref_fwd_layer(ks(xc["q"]), ks(xc["k"]), ks(xc["e"]), vs(xc["v"]), ks(xc["a"]),
                                            xc["A_log"][hk:hk + 1], xc["dt_bias"][hk:hk + 1],
                                            vs(xc["beta"]), vs(xc["gamma"]))
        go.append(to64(o[b, :, h])); ro.append(r_o[0, :, 0])
        gs.append(to64(S[b, h])); rs.append(r_S[0, 0])
    check(np.concatenate(go), np.concatenate(gs), np.concatenate(ro), np.concatenate(rs), "bf16",
          f"train_layer heads={heads}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layer_decode_small(dtype):
    say(f"layer decode {dtype}")
    steps, N, Hk, Hv, dk, dv = 5, 3, 2, 4, 48, 40
    x = make_layer_inputs(steps, N, Hk, Hv, dk, dv, dtype, seed=21)   # step axis first
    S0 = 0.02 * torch.randn((N, Hv, dk, dv), generator=torch.Generator().manual_seed(4))
    xd, S = dev(x), S0.to(DEV)
    outs = []
    for t in range(steps):
        o, S = eda.recurrent_step_layer(*(xd[n][t] if n not in ("A_log", "dt_bias") else xd[n] for n in NAMES),
                                        S, inplace=True)
        outs.append(o)
    torch.cuda.synchronize()
    sw = lambda t: np.swapaxes(to64(t), 0, 1)     # [steps, N, ...] -> [N, steps, ...]
    r_o, r_S = oracle.eda_ref_fwd_layer(sw(x["q"]), sw(x["k"]), sw(x["e"]), sw(x["v"]), sw(x["a"]),
                                        x["A_log"], x["dt_bias"], sw(x["beta"]), sw(x["gamma"]), S0)
    check(to64(torch.stack(outs)), to64(S), np.swapaxes(r_o, 0, 1), r_S, dtype, f"layer decode {dtype}")


def test_decode_layer_workload_sampled():
    w = WORKLOADS["decode_layer"]
    say(f"decode_layer N={w.B} Hk={w.hk} Hv={w.H} steps={w.steps}")
    x = make_workload(w, device=DEV)
    S = x["S0"].clone()
    outs = []
    for t in range(w.steps):
        o, S = eda.recurrent_step_layer(*(x[n][t] if n not in ("A_log", "dt_bias") else x[n] for n in NAMES),
                                        S, inplace=True)
        outs.append(o)
    torch.cuda.synchronize()
    got = torch.stack(outs)
    xc = {n: t.cpu() for n, t in x.items()}
    rng = np.random.default_rng(2)
    heads = sorted({(int(rng.integers(w.B)), int(rng.integers(w.H))) for _ in range(16)})
    grp = w.H // w.hk
    go, gs, ro, rs = [], [], [], []
    for n_, h in heads:
        hk = h // grp
        ks = lambda t: np.swapaxes(to64(t[:, n_:n_ + 1, hk:hk + 1]), 0, 1)
        vs = lambda t: np.swapaxes(to64(t[:, n_:n_ + 1, h:h + 1]), 0, 1)
        r_o, r_S = oracle.eda_ref_fwd_layer(ks(xc["q"]), ks(xc["k"]), ks(xc["e"]), vs(xc["v"]), ks(xc["a"]),
                                            xc["A_log"][hk:hk + 1], xc["dt_bias"][hk:hk + 1],
                                            vs(xc["beta"]), vs(xc["gamma"]), xc["S0"][n_:n_ + 1, h:h + 1])
        go.append(to64(got[:, n_, h])); ro.append(r_o[0, :, 0])
        gs.append(to64(S[n_, h])); rs.append(r_S[0, 0])
    check(np.concatenate(go), np.concatenate(gs), np.concatenate(ro), np.concatenate(rs), "bf16",
          f"decode_layer heads={len(heads)}")
