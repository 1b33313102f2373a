"""Seeded synthetic inputs for the Erase-then-Delta Attention (EDA) forward.

This module is shared by the HIP path's tests/bench and by the CPU oracle's
tests.  It draws random tensors only: it contains none of the recurrence's
arithmetic (no decay, erase or write step), so neither side can inherit a
mistake in the method from it.

Distributions follow the inputs the EDA paper's layer hands to its recurrence
(paper Sec. 3.3 and the reading slides' frame "EDA preserves the delta write
after cleanup"): q, k, e are L2-normalised directions, v is an unconstrained
value, alpha is a per-key-channel retention in (0, 1], beta and gamma are
scalar gates in (0, 1).  "N(mu, s)" below means mean mu and standard
deviation s.

Layouts (all contiguous, row-major):
  q, k, e : [B, T, H, d_k]      v : [B, T, H, d_v]
  alpha   : [B, T, H, d_k] fp32 beta, gamma : [B, T, H] fp32
  S0      : [B, H, d_k, d_v] fp32 (None means zeros)
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    dtype: str  # "f32" or "bf16": storage type of q, k, e, v and o
    alpha_mu: float = 2.0
    gamma_mu: float = 0.0
    s0_std: float = 0.0  # 0 => S0 is zeros
    chunk: int = 64
    seed: int = 0
    steps: int = 0  # decode workloads: number of one-token steps (T == 1)
    hk: int = 0  # layer-form workloads: key heads (H counts value heads); 0 = plain form

    @property
    def token_heads(self) -> int:
        return self.B * self.T * self.H * max(self.steps, 1)


# The workloads the forward is measured and checked on.  d_k = d_v = 128 and
# 16 or 32 heads are the head shapes of the paper's Dense/MoE models
# (paper Appendix A, Table 4); 2K, 32K and 128K contexts follow its 4K
# pretraining, 32K midtraining and RULER 4K-128K evaluation lengths.
WORKLOADS = {
    "tiny": Workload("tiny", B=1, T=64, H=1, dk=16, dv=16, dtype="f32", seed=0),
    "train": Workload("train", B=4, T=2048, H=16, dk=128, dv=128, dtype="bf16", seed=1),
    "long": Workload("long", B=1, T=32768, H=32, dk=128, dv=128, dtype="bf16",
                     s0_std=0.02, seed=2),
    "long_h16": Workload("long_h16", B=1, T=32768, H=16, dk=128, dv=128, dtype="bf16",
                         s0_std=0.02, seed=12),
    "verylong": Workload("verylong", B=1, T=131072, H=16, dk=128, dv=128, dtype="bf16",
                         alpha_mu=3.0, gamma_mu=-1.0, seed=3),
    "decode": Workload("decode", B=256, T=1, H=32, dk=128, dv=128, dtype="bf16",
                       s0_std=0.02, seed=4, steps=128),
    # layer form (raw q, k, e, safe-gate input a): the Dense model's 8 key /
    # 16 value heads at the training length, the MoE model's 16 / 32 for decode
    "train_layer": Workload("train_layer", B=4, T=2048, H=16, dk=128, dv=128, dtype="bf16",
                            seed=6, hk=8),
    "decode_layer": Workload("decode_layer", B=256, T=1, H=32, dk=128, dv=128, dtype="bf16",
                             s0_std=0.02, seed=7, steps=8, hk=16),
    # the second workload (rank-1 DPLR, QED erase vectors) at the training shape
    "train_qed": Workload("train_qed", B=4, T=2048, H=16, dk=128, dv=128, dtype="bf16", seed=8),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _unit(g: torch.Generator, shape, device) -> torch.Tensor:
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x / x.norm(dim=-1, keepdim=True)


def make_inputs(B: int, T: int, H: int, dk: int, dv: int, dtype: str = "bf16", *,
                seed: int = 0, alpha_mu: float = 2.0, alpha_std: float = 0.5,
                gamma_mu: float = 0.0, s0_std: float = 0.0,
                device: str | torch.device = "cpu") -> dict:
    """Draw one batch of inputs.

    q, k, e ~ N(0, 1) per element, L2-normalised over the channel axis in
    fp32, then stored in `dtype` (bf16 rounding is round-to-nearest-even, so
    the stored vectors have norm 1 up to ~2^-9).  v ~ N(0, 1).
    alpha = sigmoid(N(alpha_mu, alpha_std)) per key channel; beta =
    sigmoid(N(0, 1)); gamma = sigmoid(N(gamma_mu, 1)); S0 ~ N(0, s0_std) or
    None when s0_std == 0.  Draw order is fixed (q, k, e, v, alpha, beta,
    gamma, S0) so a seed names one input set on a given device.
    """
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    td = torch_dtype(dtype)
    q = _unit(g, (B, T, H, dk), device).to(td)
    k = _unit(g, (B, T, H, dk), device).to(td)
    e = _unit(g, (B, T, H, dk), device).to(td)
    v = torch.randn((B, T, H, dv), generator=g, device=device).to(td)
    alpha = torch.sigmoid(alpha_mu + alpha_std * torch.randn((B, T, H, dk), generator=g,
                                                              device=device))
    beta = torch.sigmoid(torch.randn((B, T, H), generator=g, device=device))
    gamma = torch.sigmoid(gamma_mu + torch.randn((B, T, H), generator=g, device=device))
    S0: Optional[torch.Tensor] = None
    if s0_std > 0:
        S0 = s0_std * torch.randn((B, H, dk, dv), generator=g, device=device)
    return dict(q=q, k=k, e=e, v=v, alpha=alpha.contiguous(), beta=beta.contiguous(),
                gamma=gamma.contiguous(), S0=S0)


# Address-overlap recipes: the erase address e and the write address k
# interact through the cross term gamma beta (k^T e) k e^T of the one-step
# operator (EDA paper Sec. 3.3, Eq. (16); slides frame "Order matters when the
# two addresses overlap"), which independent random directions leave at
# |cos(e, k)| ~ 0.07.  Each recipe below rebuilds e (or the gates) of a
# make_inputs() draw so that term is large:
#   e_eq_k     e = k (the paper's degenerate case: old content along k shrinks
#              by (1 - beta)(1 - gamma))
#   e_neg_k    e = -k
#   e_prev_k   e_t = k_{t-1} (e_0 kept): erase what the previous token wrote
#   cos09      e = 0.9 k + sqrt(1 - 0.81) n, n a unit vector orthogonal to k
#   gates_one  beta = gamma = 1 (the worked example's limit)
#   beta_zero  beta = 0 (no write)
#   gamma_zero gamma = 0 (no erase: the KDA update)
OVERLAP_KINDS = ("e_eq_k", "e_neg_k", "e_prev_k", "cos09", "gates_one", "beta_zero", "gamma_zero")


def make_overlap_inputs(kind: str, B: int, T: int, H: int, dk: int, dv: int, dtype: str = "bf16", *,
                        seed: int = 0, s0_std: float = 0.5, device: str | torch.device = "cpu") -> dict:
    """make_inputs() draw with one address-overlap recipe applied (see
    OVERLAP_KINDS).  Rebuilt vectors are formed in fp32 from the stored
    (rounded) k and re-normalised before the cast, so they are unit vectors
    up to the storage rounding like every other address."""
    if kind not in OVERLAP_KINDS:
        raise ValueError(f"unknown overlap recipe {kind!r}")
    x = make_inputs(B, T, H, dk, dv, dtype, seed=seed, s0_std=s0_std, device=device)
    td = torch_dtype(dtype)
    k = x["k"].float()
    if kind == "e_eq_k":
        x["e"] = x["k"].clone()
    elif kind == "e_neg_k":
        x["e"] = (-k).to(td)
    elif kind == "e_prev_k":
        e = x["e"].clone()
        e[:, 1:] = x["k"][:, :-1]
        x["e"] = e
    elif kind == "cos09":
        g = torch.Generator(device=device)
        g.manual_seed(seed + 7_000_001)
        n = torch.randn(k.shape, generator=g, device=device)
        n = n - (n * k).sum(-1, keepdim=True) * k / (k * k).sum(-1, keepdim=True)
        n = n / n.norm(dim=-1, keepdim=True)
        e = 0.9 * k + math.sqrt(1.0 - 0.81) * n
        x["e"] = (e / e.norm(dim=-1, keepdim=True)).to(td)
    elif kind == "gates_one":
        x["beta"] = torch.ones_like(x["beta"])
        x["gamma"] = torch.ones_like(x["gamma"])
    elif kind == "beta_zero":
        x["beta"] = torch.zeros_like(x["beta"])
    elif kind == "gamma_zero":
        x["gamma"] = torch.zeros_like(x["gamma"])
    return x


def make_layer_inputs(B: int, T: int, H_k: int, H_v: int, dk: int, dv: int, dtype: str = "bf16", *,
                      seed: int = 0, gamma_mu: float = 0.0, s0_std: float = 0.0,
                      device: str | torch.device = "cpu") -> dict:
    """Inputs of the layer form: raw (unnormalised) q, k, e ~ N(0, 1) per
    element and the decay gate's input a ~ N(0, 1), all [B, T, H_k, d_k] in
    `dtype`; A_log = log(U(1, 16)) and dt_bias ~ U(-7, -2.3) per key head and
    channel (so softplus(dt_bias) lies in about [1e-3, 0.1]); v ~ N(0, 1)
    [B, T, H_v, d_v]; beta = sigmoid(N(0, 1)), gamma = sigmoid(N(gamma_mu, 1))
    per value head; S0 ~ N(0, s0_std) [B, H_v, d_k, d_v] or None.  The pages
    fix the gate's form, not its parameter values; these give retentions
    spread over roughly (0.05, 1)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    td = torch_dtype(dtype)
    q = torch.randn((B, T, H_k, dk), generator=g, device=device).to(td)
    k = torch.randn((B, T, H_k, dk), generator=g, device=device).to(td)
    e = torch.randn((B, T, H_k, dk), generator=g, device=device).to(td)
    a = torch.randn((B, T, H_k, dk), generator=g, device=device).to(td)
    v = torch.randn((B, T, H_v, dv), generator=g, device=device).to(td)
    A_log = torch.log(1.0 + 15.0 * torch.rand((H_k, dk), generator=g, device=device))
    dt_bias = -7.0 + 4.7 * torch.rand((H_k, dk), generator=g, device=device)
    beta = torch.sigmoid(torch.randn((B, T, H_v), generator=g, device=device))
    gamma = torch.sigmoid(gamma_mu + torch.randn((B, T, H_v), generator=g, device=device))
    S0: Optional[torch.Tensor] = None
    if s0_std > 0:
        S0 = s0_std * torch.randn((B, H_v, dk, dv), generator=g, device=device)
    return dict(q=q, k=k, e=e, v=v, a=a, A_log=A_log.contiguous(), dt_bias=dt_bias.contiguous(),
                beta=beta.contiguous(), gamma=gamma.contiguous(), S0=S0)


def make_dplr_inputs(B: int, T: int, H: int, dk: int, dv: int, dtype: str = "bf16", *,
                     seed: int = 0, alpha_mu: float = 2.0, s0_std: float = 0.0,
                     device: str | torch.device = "cpu") -> dict:
    """Raw draws for the rank-1 DPLR workloads (GDN-2 / QED): unit q, k
    (N(0, 1), L2-normalised in fp32, stored in `dtype`); channel gates
    b = sigmoid(N(0, 1)) [B, T, H, d_k] and w = sigmoid(N(0, 1)) [B, T, H, d_v]
    (fp32); v ~ N(0, 1) (`dtype`); a per-head query weight lam ~ U(0, 0.5) [H];
    alpha = sigmoid(N(alpha_mu, 0.5)) per key channel; S0 ~ N(0, s0_std) or
    None.  The erase vector and the gated value are formed by the caller."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    td = torch_dtype(dtype)
    q = _unit(g, (B, T, H, dk), device).to(td)
    k = _unit(g, (B, T, H, dk), device).to(td)
    b = torch.sigmoid(torch.randn((B, T, H, dk), generator=g, device=device))
    w = torch.sigmoid(torch.randn((B, T, H, dv), generator=g, device=device))
    v = torch.randn((B, T, H, dv), generator=g, device=device).to(td)
    lam = 0.5 * torch.rand((H,), generator=g, device=device)
    alpha = torch.sigmoid(alpha_mu + 0.5 * torch.randn((B, T, H, dk), generator=g, device=device))
    S0: Optional[torch.Tensor] = None
    if s0_std > 0:
        S0 = s0_std * torch.randn((B, H, dk, dv), generator=g, device=device)
    return dict(q=q, k=k, b=b, w=w, v=v, lam=lam, alpha=alpha.contiguous(), S0=S0)


def make_workload(w: Workload, device: str | torch.device = "cpu", seed: Optional[int] = None) -> dict:
    """Inputs for a named workload.  Decode workloads return per-step inputs
    stacked on a leading step axis: q, k, e, v, alpha are [steps, N, H, d],
    beta, gamma are [steps, N, H], and S0 is [N, H, d_k, d_v]."""
    s = w.seed if seed is None else seed
    if w.hk:
        if w.steps:
            x = make_layer_inputs(w.steps, w.B, w.hk, w.H, w.dk, w.dv, w.dtype, seed=s,
                                  gamma_mu=w.gamma_mu, device=device)
            gen = torch.Generator(device=device)
            gen.manual_seed(s + 1_000_003)
            x["S0"] = w.s0_std * torch.randn((w.B, w.H, w.dk, w.dv), generator=gen, device=device)
            return x
        return make_layer_inputs(w.B, w.T, w.hk, w.H, w.dk, w.dv, w.dtype, seed=s,
                                 gamma_mu=w.gamma_mu, s0_std=w.s0_std, device=device)
    if w.steps:
        x = make_inputs(w.steps, w.B, w.H, w.dk, w.dv, w.dtype, seed=s,
                        alpha_mu=w.alpha_mu, gamma_mu=w.gamma_mu, s0_std=0.0,
                        device=device)
        g = torch.Generator(device=device)
        g.manual_seed(s + 1_000_003)
        x["S0"] = w.s0_std * torch.randn((w.B, w.H, w.dk, w.dv), generator=g, device=device)
        return x
    return make_inputs(w.B, w.T, w.H, w.dk, w.dv, w.dtype, seed=s, alpha_mu=w.alpha_mu,
                       gamma_mu=w.gamma_mu, s0_std=w.s0_std, device=device)


def hand_example() -> dict:
    """The two-dimensional teaching example of the reading slides (frame "A
    two-dimensional example isolates the new capability") and the Chinese
    reading notes (method part 3): d_k = 2, d_v = 1, S_{t-1} = (3, 5)^T,
    e = (1, 0), k = (0, 1), v = 7, D = I, beta = gamma = 1.  q is not given
    on the pages; q = (1, 1) reads the sum of both rows.  fp32 storage."""
    f = torch.float32
    return dict(
        q=torch.tensor([1.0, 1.0], dtype=f).view(1, 1, 1, 2),
        k=torch.tensor([0.0, 1.0], dtype=f).view(1, 1, 1, 2),
        e=torch.tensor([1.0, 0.0], dtype=f).view(1, 1, 1, 2),
        v=torch.tensor([7.0], dtype=f).view(1, 1, 1, 1),
        alpha=torch.ones((1, 1, 1, 2), dtype=f),
        beta=torch.ones((1, 1, 1), dtype=f),
        gamma=torch.ones((1, 1, 1), dtype=f),
        S0=torch.tensor([[3.0], [5.0]], dtype=f).view(1, 1, 2, 1),
    )


def random_pair_abs_cos_mean(d: int) -> float:
    """E|u.r| for independent uniform unit vectors in R^d:
    Gamma(d/2) / (sqrt(pi) * Gamma((d+1)/2)).  For d = 128 this is the
    ~0.0707 random-direction reference the paper's address-geometry probe
    compares against (paper Sec. 4.5; slides frame on |cos(e, k)|)."""
    return math.exp(math.lgamma(d / 2) - math.lgamma((d + 1) / 2)) / math.sqrt(math.pi)
