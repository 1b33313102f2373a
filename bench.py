"""Throughput of the Erase-then-Delta Attention (EDA) forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload train]

A step is one chunked forward (`eda_fwd_chunked`: the chunk-factor kernel,
then the state pass) over one batch of synthetic inputs already resident in
HBM.  The default workload is the training shape B=4, H=16, T=2048,
d_k=d_v=128, bf16 q/k/e/v, fp32 gates and state.  One JSON line is printed:
tokens/s of the whole batch (wall clock around K steps), the roofline of the
dominant kernel (its average duration from HIP events recorded on the launch
stream around each kernel, over a second run of K steps through
`eda_fwd_chunked_timed`), both kernels' figures, the fp64 CPU oracle timed on
the host on a bounded sample of the same workload, and a decode section (256
sequences x 32 heads, one token per step, state updated in place) with its own
HBM roofline, and a layer section: the layer-form forward
(`eda_fwd_chunked_layer`: safe gate, q/k/e normalisation and 8 key heads shared
by 16 value heads fused into the factor kernel) beside the same computation
unfused (the prologue as PyTorch element-wise ops, then `eda_fwd_chunked` on
the expanded value-head inputs), and the layer-form decode step; and a dplr
section: the rank-1 DPLR update of GDN-2/QED (`eda_fwd_chunked_dplr`) on the
same training shape with QED erase vectors; and a backward section: `eda_bwd`
(gradients of every input) on the training shape; and a long_context section:
the chunked forward at T = 32768 with 32 heads (the long-context
configuration), with 16 heads (the metric's H = 16), and at T = 131072 with 16
heads (the very-long configuration), tokens/s each.

Algorithmic work (d_k = d_v = d, C tokens per chunk, L = 2C sub-steps; each
token is an erase sub-step and a delta sub-step), per chunk and head, in the
canonical chunk formulation:
  factor side: L^2 d (decayed Gram) + L^3/6 (triangular inverse)
               + L^2 d (W factor) + C L d (query-key products)  multiply-adds
  state side:  L d^2 (W S) + L C d (value part of U) + C d^2 (query-state
               product) + C L d (intra-chunk output) + L d^2 (state update)
(counted once, however the kernels regroup them: the factor kernel here also
forms the chunk's state map Phi = -Khat^T W and Psi = Khat^T T', so the state
pass issues d^2 d_v + d C d_v + C d d_v + C^2 d_v per chunk instead).
Algorithmic bytes per token and head: the factor kernel must read q, k, e
(storage type), alpha (fp32 per key channel), beta and gamma (fp32); the state
pass must read v and write o (storage type), plus the fp32 initial state read
and final state written once per head.  The whole path moves the sum (1800 B
per token-head for bf16, d = 128).  Decode moves the fp32 state in and out
once per step (2 d_k d_v 4 bytes) plus the token's inputs and output.
Peaks: MI355X dense bf16 matrix 2.5 PFLOP/s, fp32 matrix 157.3 TFLOP/s,
HBM3E 8 TB/s.  `traffic` is the measured HBM bytes per launch of the dominant
kernel (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated on a copy of known
size), read from the committed summary under profiles/ and reported only while
the kernel source it was measured on is unchanged; each chunked kernel's
`rocprof_mfma` is, on the same terms, its measured matrix-core busy fraction
and issued bf16 flop per launch (SQ_VALU_MFMA_BUSY_CYCLES,
SQ_INSTS_VALU_MFMA_MOPS_BF16 over GRBM_GUI_ACTIVE).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "EDA fwd tokens/sec (H=16,d=128, T=2K/32K) + % MFMA/HBM roofline"
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


# ---------------------------------------------------------------------------
# algorithmic work
# ---------------------------------------------------------------------------
def intra_macs_per_chunk_head(C: int, d: int) -> float:
    L = 2 * C
    return L * L * d + L ** 3 / 6.0 + L * L * d + C * L * d


def state_macs_per_chunk_head(C: int, d: int) -> float:
    L = 2 * C
    return L * d * d + L * C * d + C * d * d + C * L * d + L * d * d


def token_bytes(dk: int, dv: int, es: int) -> dict:
    """Algorithmic bytes per token-head, split by the kernel that must move them."""
    factors = 3 * dk * es + dk * 4 + 2 * 4        # q, k, e, alpha, beta, gamma
    state = dv * es + dv * es                     # v, o
    return dict(factors=factors, state=state, chunked=factors + state)


def decode_bytes_per_head(dk: int, dv: int, es: int) -> int:
    return 2 * dk * dv * 4 + (3 * dk + dv) * es + dk * 4 + 8 + dv * es


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None when there is none or the kernel source changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            key, val = line.split("=", 1)
            kv[key.strip()] = val.strip()
    src = os.path.join(ROOT, "recurrent_memory_amd", "csrc", kv.get("source", ""))
    if not os.path.exists(src) or hashlib.sha1(open(src, "rb").read()).hexdigest() != kv.get("source_sha1"):
        return None
    try:
        return float(kv["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def measured_mfma(kernel: str, workload: str):
    """Matrix-core busy fraction and issued bf16 flop per launch of `kernel`
    from the committed rocprofv3 counter summary (SQ_VALU_MFMA_BUSY_CYCLES,
    SQ_INSTS_VALU_MFMA_MOPS_BF16, GRBM_GUI_ACTIVE), or None when there is none
    or the kernel source changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"mfma_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            key, val = line.split("=", 1)
            kv[key.strip()] = val.strip()
    src = os.path.join(ROOT, "recurrent_memory_amd", "csrc", kv.get("source", ""))
    if not os.path.exists(src) or hashlib.sha1(open(src, "rb").read()).hexdigest() != kv.get("source_sha1"):
        return None
    try:
        return dict(busy_fraction=float(kv["mfma_busy_fraction"]), issued_bf16_flop=float(kv["issued_bf16_flop"]),
                    issued_over_canonical=float(kv["issued_over_canonical"]))
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# timing helpers (events on the stream the library launches on)
# ---------------------------------------------------------------------------
def time_events(torch, fn, reps: int) -> float:
    """Average milliseconds of `fn` over `reps` back-to-back calls, measured
    with HIP events recorded on the current stream (the launch stream)."""
    s = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(s)
    for _ in range(reps):
        fn()
    end.record(s)
    end.synchronize()
    return start.elapsed_time(end) / reps


def measure_chunked(torch, eda, x, w, chunk: int, steps: int, warmup: int = 3) -> dict:
    """One chunked forward per step on resident inputs: wall-clock tokens/s
    over `steps` steps, then the same steps through eda_fwd_chunked_timed for
    each kernel's average duration (HIP events on the launch stream), and the
    path- and kernel-level fractions of the bf16 matrix and HBM peaks."""
    dev = x["q"].device
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    es = 2 if w.dtype == "bf16" else 4
    o = torch.empty((B, T, H, dv), dtype=x["q"].dtype, device=dev)
    S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    need = eda.workspace_size(B, T, H, dk, dv, x["q"].dtype, chunk)
    ws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None

    def step(events=None):
        eda.fwd_chunked(x["q"], x["k"], x["e"], x["v"], x["alpha"], x["beta"], x["gamma"], x["S0"],
                        chunk=chunk, out=o, S_final=S_final, workspace=ws, events=events)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(s)
    for _ in range(steps):
        step()
    ev1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_kernel = ev0.elapsed_time(ev1) / steps
    # per-kernel durations: the same steps through the timed entry point
    trip = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for t3 in trip:
        for ev in t3:
            ev.record(s)   # materialise the events before handing them over
    torch.cuda.synchronize()
    for t3 in trip:
        step(events=[ev.cuda_event for ev in t3])
    torch.cuda.synchronize()
    ms_k1 = sum(t3[0].elapsed_time(t3[1]) for t3 in trip) / steps
    ms_k2 = sum(t3[1].elapsed_time(t3[2]) for t3 in trip) / steps

    d = dk
    n_ch = B * H * ((T + chunk - 1) // chunk)
    tb = token_bytes(dk, dv, es)
    peak_mm = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    state_io = (2 if x["S0"] is not None else 1) * B * H * dk * dv * 4
    work = {
        "factors": dict(flop=2 * intra_macs_per_chunk_head(chunk, d) * n_ch,
                        bytes=tb["factors"] * B * T * H, ms=ms_k1),
        "state": dict(flop=2 * state_macs_per_chunk_head(chunk, d) * n_ch,
                      bytes=tb["state"] * B * T * H + state_io, ms=ms_k2),
    }
    names = dict(factors="eda_bf16_factors", state="eda_bf16_state") if w.dtype == "bf16" else \
        dict(factors="eda_chunk_intra", state="eda_chunk_state")

    def roof(kind: str) -> dict:
        wk = work[kind]
        sec = wk["ms"] * 1e-3
        # the binding roofline at the algorithmic level is the one with the larger floor
        mfma = wk["flop"] / (peak_mm * 1e12) >= wk["bytes"] / (PEAK_HBM_GBS * 1e9)
        tf, gb = wk["flop"] / sec / 1e12, wk["bytes"] / sec / 1e9
        if mfma:
            r = dict(kernel=names[kind], bound="mfma", achieved=round(tf, 3), peak=peak_mm,
                     unit="TFLOP/s", frac=round(tf / peak_mm, 5))
        else:
            r = dict(kernel=names[kind], bound="hbm", achieved=round(gb, 2), peak=PEAK_HBM_GBS,
                     unit="GB/s", frac=round(gb / PEAK_HBM_GBS, 5))
        r.update(ms=round(wk["ms"], 5), algorithmic_bytes=wk["bytes"], algorithmic_flop=wk["flop"],
                 mfma_frac=round(tf / peak_mm, 5), hbm_frac=round(gb / PEAK_HBM_GBS, 5),
                 rocprof_mfma=measured_mfma(names[kind], w.name) if chunk == eda.DEFAULT_CHUNK else None)
        return r

    kernels = {k: roof(k) for k in work}
    flop = work["factors"]["flop"] + work["state"]["flop"]
    byts = tb["chunked"] * B * T * H + state_io
    sec = ms_kernel * 1e-3
    tflops, gbs = flop / sec / 1e12, byts / sec / 1e9
    # path-level binding roofline: the larger of the two floors over the path's time
    mfma_bound = flop / (peak_mm * 1e12) >= byts / (PEAK_HBM_GBS * 1e9)
    path_roof = (dict(bound="mfma", achieved=round(tflops, 3), peak=peak_mm, unit="TFLOP/s",
                      frac=round(tflops / peak_mm, 5)) if mfma_bound else
                 dict(bound="hbm", achieved=round(gbs, 2), peak=PEAK_HBM_GBS, unit="GB/s",
                      frac=round(gbs / PEAK_HBM_GBS, 5)))
    dom = max(work, key=lambda k: work[k]["ms"])
    return dict(chunk=chunk, value=round(B * T * steps / wall, 1), unit="tokens/s",
                ms_per_step=round(wall * 1e3 / steps, 5), kernel_ms=round(ms_kernel, 5),
                token_heads_per_s=round(B * T * H * steps / wall, 1),
                canonical_flop=flop, compulsory_bytes=byts,
                mfma_tflops=round(tflops, 3), mfma_frac=round(tflops / peak_mm, 5),
                hbm_gbs=round(gbs, 2), hbm_frac=round(gbs / PEAK_HBM_GBS, 5),
                canonical_flop_per_token_head=flop / (B * T * H),
                compulsory_bytes_per_token_head=tb["chunked"], path_roofline=path_roof,
                dominant=dom, kernels=kernels)


def bench_layer(torch, eda, dev, chunk: int, steps: int) -> dict:
    """Layer form (fused prologue) against the unfused pipeline on the same
    inputs, and the layer-form decode step."""
    import torch.nn.functional as Fn
    from eda_inputs import WORKLOADS, make_workload

    w = WORKLOADS["train_layer"]
    x = make_workload(w, device=dev)
    B, T, Hk, Hv, dk, dv = w.B, w.T, w.hk, w.H, w.dk, w.dv
    o = torch.empty((B, T, Hv, dv), dtype=x["q"].dtype, device=dev)
    Sf = torch.empty((B, Hv, dk, dv), dtype=torch.float32, device=dev)
    ws = torch.empty(eda.layer_workspace_size(B, T, Hk, Hv, dk, dv, x["q"].dtype, chunk),
                     dtype=torch.uint8, device=dev)
    names = ("q", "k", "e", "v", "a", "A_log", "dt_bias", "beta", "gamma")

    def fused():
        eda.fwd_chunked_layer(*(x[n] for n in names), x["S0"], chunk=chunk, out=o, S_final=Sf,
                              workspace=ws)

    ws2 = torch.empty(eda.workspace_size(B, T, Hv, dk, dv, x["q"].dtype, chunk), dtype=torch.uint8,
                      device=dev)

    def unfused():
        # the same prologue as separate element-wise passes over HBM
        grp = Hv // Hk
        qn, kn, en = (Fn.normalize(x[n].float(), dim=-1, eps=1e-6).to(x[n].dtype)
                      .repeat_interleave(grp, dim=2) for n in ("q", "k", "e"))
        delta = Fn.softplus(x["a"].float() + x["dt_bias"])
        alpha = torch.exp(-5.0 + 5.0 * torch.exp(-(torch.exp(x["A_log"]) / 5.0) * delta))
        alpha = alpha.repeat_interleave(grp, dim=2)
        eda.fwd_chunked(qn, kn, en, x["v"], alpha, x["beta"], x["gamma"], x["S0"], chunk=chunk,
                        out=o, S_final=Sf, workspace=ws2)

    for f in (fused, unfused):
        f()
    torch.cuda.synchronize()
    ms_f = time_events(torch, fused, steps)
    ms_u = time_events(torch, unfused, steps)
    tok = B * T
    res = dict(workload=f"{w.name}: layer-form chunked forward B={B} T={T} H_k={Hk} H_v={Hv} "
                        f"d_k=d_v={dk} {w.dtype}, chunk={chunk}",
               value=round(tok / (ms_f * 1e-3), 1), unit="tokens/s", ms_per_step=round(ms_f, 5),
               unfused_ms_per_step=round(ms_u, 5), fused_speedup=round(ms_u / ms_f, 3))
    print(f"[bench] layer fused {ms_f:.4f} ms, unfused {ms_u:.4f} ms", file=sys.stderr, flush=True)
    del x, o, Sf, ws, ws2

    wd = WORKLOADS["decode_layer"]
    xd = make_workload(wd, device=dev)
    Sd = xd["S0"].clone()
    od = torch.empty((wd.B, wd.H, wd.dv), dtype=xd["q"].dtype, device=dev)
    per = [tuple(xd[n][t] if n not in ("A_log", "dt_bias") else xd[n] for n in names)
           for t in range(wd.steps)]

    def dec():
        for t in range(wd.steps):
            eda.recurrent_step_layer(*per[t], Sd, S_out=Sd, o=od)

    dec()
    torch.cuda.synchronize()
    ms_tok = time_events(torch, dec, 3) / wd.steps
    dbytes = (2 * wd.dk * wd.dv * 4 + wd.dv * 4) * wd.B * wd.H   # state in and out dominate
    res["decode"] = dict(workload=f"{wd.name}: N={wd.B} H_k={wd.hk} H_v={wd.H} d_k=d_v={wd.dk} "
                                  f"{wd.dtype}, {wd.steps} steps in place",
                         value=round(wd.B / (ms_tok * 1e-3), 1), unit="tokens/s",
                         ms_per_token_step=round(ms_tok, 5),
                         state_gbs=round(dbytes / (ms_tok * 1e-3) / 1e9, 2))
    print(f"[bench] layer decode {ms_tok * 1e3:.2f} us/step", file=sys.stderr, flush=True)
    return res


def bench_dplr(torch, eda, dev, chunk: int, steps: int) -> dict:
    """The second workload: rank-1 DPLR update with QED erase vectors."""
    from eda_inputs import WORKLOADS, make_dplr_inputs

    w = WORKLOADS["train_qed"]
    x = make_dplr_inputs(w.B, w.T, w.H, w.dk, w.dv, w.dtype, seed=w.seed, device=dev)
    q, k, b = x["q"].float(), x["k"].float(), x["b"]
    u = b * q
    a = (b * k + x["lam"].view(1, 1, -1, 1) * (u - k * (k * u).sum(-1, keepdim=True))).to(x["q"].dtype)
    v = (x["w"] * x["v"].float()).to(x["q"].dtype)
    o = torch.empty((w.B, w.T, w.H, w.dv), dtype=x["q"].dtype, device=dev)
    Sf = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    ws = torch.empty(eda.workspace_size(w.B, w.T, w.H, w.dk, w.dv, x["q"].dtype, chunk), dtype=torch.uint8,
                     device=dev)

    def run():
        eda.fwd_chunked_dplr(x["q"], x["k"], a, v, x["alpha"], None, chunk=chunk, out=o, S_final=Sf,
                             workspace=ws)

    run()
    torch.cuda.synchronize()
    ms = time_events(torch, run, steps)
    print(f"[bench] dplr {ms:.4f} ms", file=sys.stderr, flush=True)
    return dict(workload=f"{w.name}: rank-1 DPLR (QED erase vectors) chunked forward B={w.B} T={w.T} "
                         f"H={w.H} d_k=d_v={w.dk} {w.dtype}, chunk={chunk}",
                value=round(w.B * w.T / (ms * 1e-3), 1), unit="tokens/s", ms_per_step=round(ms, 5))


def bench_long(torch, eda, dev, chunk: int) -> dict:
    """The chunked forward at the long-context workloads: T = 32768 with 32
    and 16 heads, and T = 131072 with 16 heads; tokens/s, both fractions of
    the path and the per-kernel split for each."""
    from eda_inputs import WORKLOADS, make_workload

    out = {}
    for name in ("long", "long_h16", "verylong"):
        w = WORKLOADS[name]
        x = make_workload(w, device=dev)
        r = measure_chunked(torch, eda, x, w, chunk, steps=5, warmup=1)
        s0 = f"S0 ~ N(0, {w.s0_std})" if w.s0_std > 0 else "S0 = 0"
        r["workload"] = f"{name}: B={w.B} T={w.T} H={w.H} d_k=d_v={w.dk} {w.dtype}, {s0}, chunk={chunk}"
        out[name] = r
        print(f"[bench] {name} {r['kernel_ms']:.3f} ms (factors {r['kernels']['factors']['ms']:.3f}, "
              f"state {r['kernels']['state']['ms']:.3f}); mfma {100 * r['mfma_frac']:.1f} %, "
              f"hbm {100 * r['hbm_frac']:.1f} %", file=sys.stderr, flush=True)
        del x
        torch.cuda.empty_cache()
    return out


def bench_bwd(torch, eda, dev, w) -> dict:
    """Backward pass on the benchmark workload's shape: gradients of every
    input for a random dO (and no final-state gradient)."""
    from eda_inputs import make_workload

    x = make_workload(w, device=dev)
    g = torch.Generator(device=dev).manual_seed(7)
    dO = torch.randn((w.B, w.T, w.H, w.dv), generator=g, device=dev).to(x["q"].dtype)
    ws = torch.empty(eda.load_library().eda_bwd_workspace_size(w.B, w.T, w.H, w.dk, w.dv), dtype=torch.uint8,
                     device=dev)

    def run():
        eda.backward(x["q"], x["k"], x["e"], x["v"], x["alpha"], x["beta"], x["gamma"], x["S0"], dO,
                     workspace=ws)

    run()
    torch.cuda.synchronize()
    ms = time_events(torch, run, 3)
    es = 2 if w.dtype == "bf16" else 4
    # algorithmic bytes per token-head: q, k, e, v, dO in, alpha, beta, gamma in,
    # dq, dk, de, dalpha, dv, dbeta, dgamma out (fp32)
    per = (3 * w.dk + 2 * w.dv) * es + w.dk * 4 + 8 + (4 * w.dk + w.dv) * 4 + 8
    gbs = per * w.B * w.T * w.H / (ms * 1e-3) / 1e9
    print(f"[bench] backward {ms:.3f} ms", file=sys.stderr, flush=True)
    return dict(workload=f"{w.name}: backward (all input gradients) B={w.B} T={w.T} H={w.H} d_k={w.dk} "
                         f"d_v={w.dv} {w.dtype}", value=round(w.B * w.T / (ms * 1e-3), 1), unit="tokens/s",
                ms_per_step=round(ms, 4), hbm_gbs_algorithmic=round(gbs, 1),
                hbm_frac_algorithmic=round(gbs / PEAK_HBM_GBS, 5))


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="train", choices=["train", "long", "long_h16", "verylong"])
    ap.add_argument("--chunk", type=int, default=0, help="tokens per chunk (0 = library default)")
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU time over which the oracle baseline is averaged")
    ap.add_argument("--no-layer", action="store_true")
    ap.add_argument("--no-dplr", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--no-long", action="store_true")
    ap.add_argument("--no-chunk-sweep", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the EDA forward is independent per (batch, head), "
              "so more GPUs would each run this same kernel on their own share of heads; "
              "run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import recurrent_memory_amd as eda
    from eda_inputs import WORKLOADS, make_workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (the EDA path has no CPU implementation)", file=sys.stderr)
        return 1
    eda.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    w = WORKLOADS[args.workload]
    chunk = args.chunk or eda.DEFAULT_CHUNK
    x = make_workload(w, device=dev)
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    print(f"[bench] workload {w.name}: B={B} T={T} H={H} d_k={dk} d_v={dv} {w.dtype} chunk={chunk}",
          file=sys.stderr, flush=True)
    path = measure_chunked(torch, eda, x, w, chunk, args.steps, args.warmup)
    value, ms_per_step, tokens = path["value"], path["ms_per_step"], B * T
    print(f"[bench] {ms_per_step:.4f} ms/step (events {path['kernel_ms']:.4f} ms), {value:.4g} tokens/s",
          file=sys.stderr, flush=True)
    kernels = path["kernels"]
    roof_line = dict(kernels[path["dominant"]])
    roof_line["traffic"] = measured_traffic(roof_line["kernel"], w.name) if chunk == eda.DEFAULT_CHUNK else None
    for k in ("ms", "algorithmic_bytes", "algorithmic_flop", "rocprof_mfma", "mfma_frac", "hbm_frac"):
        roof_line.pop(k)
    print(f"[bench] chunked path: {json.dumps(path)}", file=sys.stderr, flush=True)
    # the same step at the other chunk sizes, for comparison
    other_chunks = {}
    if not args.no_chunk_sweep:
        for c in (32, 16):
            if c == chunk:
                continue
            r = measure_chunked(torch, eda, x, w, c, max(5, args.steps // 2), 2)
            for kk in r["kernels"].values():
                kk.pop("rocprof_mfma")
            other_chunks[f"chunk_{c}"] = r
            print(f"[bench] chunk {c}: {r['kernel_ms']:.4f} ms ({r['value']:.4g} tokens/s)", file=sys.stderr,
                  flush=True)
    del x
    torch.cuda.empty_cache()

    # decode: N sequences x H heads, one token per step, state in place
    decode = None
    if not args.no_decode:
        wd = WORKLOADS["decode"]
        xd = make_workload(wd, device=dev)
        Sd = xd["S0"].clone()
        od = torch.empty((wd.B, wd.H, wd.dv), dtype=xd["q"].dtype, device=dev)
        nsteps = min(args.decode_steps, wd.steps)
        per = [tuple(xd[n][t] for n in ("q", "k", "e", "v", "alpha", "beta", "gamma"))
               for t in range(nsteps)]

        def decode_run():
            for t in range(nsteps):
                eda.recurrent_step(*per[t], Sd, S_out=Sd, o=od)

        decode_run(); torch.cuda.synchronize()
        ms_run = time_events(torch, decode_run, 3)
        ms_tok = ms_run / nsteps
        dbytes = decode_bytes_per_head(wd.dk, wd.dv, 2 if wd.dtype == "bf16" else 4) * wd.B * wd.H
        gbs = dbytes / (ms_tok * 1e-3) / 1e9
        decode = dict(workload=f"decode: N={wd.B} H={wd.H} d_k=d_v={wd.dk} {wd.dtype}, "
                               f"{nsteps} steps in place",
                      value=round(wd.B / (ms_tok * 1e-3), 1), unit="tokens/s",
                      ms_per_token_step=round(ms_tok, 5),
                      roofline=dict(kernel="eda_decode_kernel", bound="hbm", achieved=round(gbs, 2),
                                    peak=PEAK_HBM_GBS, unit="GB/s", frac=round(gbs / PEAK_HBM_GBS, 5),
                                    traffic=measured_traffic("eda_decode_kernel", "decode")))
        print(f"[bench] decode {ms_tok * 1e3:.2f} us/step, {gbs:.1f} GB/s", file=sys.stderr, flush=True)
        del xd, per

    layer = None if args.no_layer else bench_layer(torch, eda, dev, chunk, args.steps)
    dplr = None if args.no_dplr else bench_dplr(torch, eda, dev, chunk, args.steps)
    bwd = None if args.no_bwd else bench_bwd(torch, eda, dev, w)
    longc = None if (args.no_long or args.workload != "train") else bench_long(torch, eda, dev, chunk)

    # fp64 CPU oracle on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        from eda_inputs import make_inputs
        threads = oracle.default_threads()   # every core this process may run on
        Tc = min(T, 2048)
        Bc = 1 if w.B * Tc * w.H > 4 * 2048 * 16 else w.B
        xc = make_inputs(Bc, Tc, w.H, dk, dv, w.dtype, seed=w.seed, alpha_mu=w.alpha_mu,
                         gamma_mu=w.gamma_mu, s0_std=w.s0_std)
        # the sample is repeated until about 10 s of CPU time have accumulated
        reps, dt = 0, 0.0
        while reps == 0 or dt < args.cpu_seconds:
            t1 = time.perf_counter()
            oracle.eda_ref_fwd(xc["q"], xc["k"], xc["e"], xc["v"], xc["alpha"], xc["beta"], xc["gamma"],
                               xc["S0"], nthreads=threads)
            dt += time.perf_counter() - t1
            reps += 1
        model = None
        try:
            for ln in open("/proc/cpuinfo"):
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
        cpu = dict(value=round(reps * Bc * Tc / dt, 2), unit="tokens/s", cores=threads, kind="oracle",
                   host_cpu_count=os.cpu_count(), cpu_model=model,
                   sample=f"B={Bc} T={Tc} H={w.H} d_k=d_v={dk} (all heads), fp64 token recurrence, "
                          f"{reps} passes in {dt:.2f} s")
        print(f"[bench] cpu oracle {cpu}", file=sys.stderr, flush=True)

    line = dict(
        metric=METRIC, value=round(value, 1), unit="tokens/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=round(ms_per_step, 5), higher_is_better=True,
        scaling="weak", vs_baseline=None, dtype=w.dtype, data="synthetic",
        config=dict(workload=f"{w.name}: EDA chunked forward B={B} T={T} H={H} d_k={dk} d_v={dv} "
                             f"{w.dtype} inputs, fp32 gates and state, chunk={chunk}",
                    B=B, T=T, H=H, d_k=dk, d_v=dv, chunk=chunk, tokens_per_step=tokens,
                    parallelism="single GPU"),
        roofline=roof_line, roofline_path=path["path_roofline"], cpu_baseline=cpu, chunked_path=path,
        other_chunk_sizes=other_chunks or None, decode=decode, layer=layer,
        dplr=dplr, backward=bwd, long_context=longc)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
