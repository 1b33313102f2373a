"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small cases compare every element; full-size workloads compare every output
of a seeded sample of heads (heads are independent, so each sampled head's
oracle run is exact).  Tolerances: fp32 inputs max-abs <= 1e-4; bf16 inputs
relative Frobenius <= 5e-3 on o and on the final state.
"""
import math

import numpy as np
import pytest
import torch

import recurrent_memory_amd as eda
import oracle
from eda_inputs import OVERLAP_KINDS, WORKLOADS, hand_example, make_inputs, make_overlap_inputs, make_workload
from _helpers import check, oracle_heads, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev(x):
    return {n: (None if t is None else t.to(DEV)) for n, t in x.items()}


def say(msg):
    print(f"[case] {msg}", flush=True)


def run_chunked(x, chunk=0, **kw):
    o, S = eda.fwd_chunked(x["q"], x["k"], x["e"], x["v"], x["alpha"], x["beta"], x["gamma"],
                           x["S0"], chunk=chunk, **kw)
    torch.cuda.synchronize()
    return o, S


def full_oracle(x):
    return oracle.eda_ref_fwd(x["q"], x["k"], x["e"], x["v"], x["alpha"], x["beta"], x["gamma"],
                              x["S0"])


# ---------------------------------------------------------------------------
# the hand-worked example, exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_hand_example_chunked(dtype, chunk):
    say(f"hand example chunked {dtype} chunk={chunk}")
    x = hand_example()
    for n in ("q", "k", "e", "v"):
        x[n] = x[n].to(dtype)
    o, S = run_chunked(dev(x), chunk=chunk)
    assert S.cpu().flatten().tolist() == [0.0, 7.0]
    assert float(o.float().cpu()) == 7.0
    x["gamma"] = torch.zeros_like(x["gamma"])
    o, S = run_chunked(dev(x), chunk=chunk)
    assert S.cpu().flatten().tolist() == [3.0, 7.0]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_hand_example_decode(dtype):
    say(f"hand example decode {dtype}")
    x = hand_example()
    d = {n: t[:, 0] for n, t in x.items() if n != "S0"}
    for n in ("q", "k", "e", "v"):
        d[n] = d[n].to(dtype)
    d = dev(d)
    o, S = eda.recurrent_step(d["q"], d["k"], d["e"], d["v"], d["alpha"], d["beta"], d["gamma"],
                              x["S0"].to(DEV))
    torch.cuda.synchronize()
    assert S.cpu().flatten().tolist() == [0.0, 7.0]
    assert float(o.float().cpu()) == 7.0


# ---------------------------------------------------------------------------
# small and ragged cases, every element
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_tiny_workload_fp32(chunk):
    w = WORKLOADS["tiny"]
    say(f"tiny fp32 chunk={chunk}")
    x = make_workload(w)
    ro, rS = full_oracle(x)
    o, S = run_chunked(dev(x), chunk=chunk)
    check(to64(o), to64(S), ro, rS, "f32", f"tiny chunk={chunk}")


def test_tiny_workload_fp32_decode():
    w = WORKLOADS["tiny"]
    say("tiny fp32 decode over T=64 steps")
    x = make_workload(w)
    ro, rS = full_oracle(x)
    xd = dev(x)
    S = torch.zeros((1, 1, 16, 16), device=DEV)
    outs = []
    for t in range(w.T):
        o, S = eda.recurrent_step(*(xd[n][:, t].contiguous() for n in
                                    ("q", "k", "e", "v", "alpha", "beta", "gamma")), S, inplace=True)
        outs.append(o.clone())
    torch.cuda.synchronize()
    got = torch.stack(outs, 1)
    check(to64(got), to64(S), ro, rS, "f32", "tiny decode")


RAGGED = [(1, 1, 1, 16), (1, 1, 1, 32), (2, 15, 3, 16), (1, 33, 2, 32), (2, 100, 2, 16),
          (1, 64, 1, 32), (1, 65, 1, 32), (3, 47, 1, 16),
          (1, 1, 1, 64), (1, 63, 1, 64), (2, 64, 2, 64), (1, 65, 2, 64), (1, 127, 1, 64),
          (2, 129, 1, 64), (1, 200, 3, 64)]


def segment_count(B, T, H, dk, dv, chunk):
    """Segments per head of the bf16 state pass, read back from the workspace
    size: the chunk factors (one block per chunk and head, as documented in
    eda.h) plus, with P > 1 segments, B H (P - 1) d_k (d_k + 2 d_v) fp32."""
    D = 32 if max(dk, dv) <= 32 else 64 if max(dk, dv) <= 64 else 128
    nc = -(-T // chunk)
    frag = (D // 16) * (D // 32) + (D // 16) * -(-chunk // 32) + (chunk // 16) * (D // 32) + (chunk // 16) * -(-chunk // 32)
    blk = -(-(frag * 1024 + 4 * D) // 256) * 256
    extra = eda.workspace_size(B, T, H, dk, dv, torch.bfloat16, chunk) - B * H * nc * blk
    assert extra % (B * H * dk * (dk + 2 * dv) * 4) == 0
    return 1 + extra // (B * H * dk * (dk + 2 * dv) * 4)


# Few heads and long sequences: the state pass cuts each head's chunks into
# segments walked at the same time (B, T, H, d_k, d_v, chunk, segments)
SEGMENTED = [(1, 64 * 260 + 17, 2, 128, 128, 64, 4),     # ragged last chunk and segment
             (1, 16 * 520, 2, 128, 128, 16, 8),
             (2, 32 * 300 + 5, 1, 64, 40, 32, 4),        # d_k != d_v, partial value slice
             (1, 16 * 1100, 1, 128, 100, 16, 16),
             (1, 64 * 512, 1, 128, 128, 64, 8),          # 64-chunk segments, as at 16 heads and T = 32768
             (1, 16 * 520, 1, 128, 30, 16, 8)]           # d_k + d_v not a multiple of 4: element-wise prefix reads


@pytest.mark.parametrize("B,T,H,dk,dv,chunk,P", SEGMENTED)
def test_segmented_state_pass(B, T, H, dk, dv, chunk, P):
    """Segment maps [M | N], their prefix and the segments' passes against the
    token recurrence over whole heads, with an initial state."""
    assert segment_count(B, T, H, dk, dv, chunk) == P
    say(f"segmented B={B} T={T} H={H} dk={dk} dv={dv} chunk={chunk} P={P}")
    x = make_inputs(B, T, H, dk, dv, "bf16", seed=300 + T, s0_std=0.05)
    ro, rS = full_oracle(x)
    o, S = run_chunked(dev(x), chunk=chunk)
    check(to64(o), to64(S), ro, rS, "bf16", f"segmented P={P} T={T}")


def test_segmented_strong_decay_and_no_decay():
    """Segments where the chunk maps contract to nearly zero (alpha ~ e^-5 per
    token) and where they do not contract at all (alpha = 1), with S0."""
    B, T, H, d, chunk = 1, 64 * 300, 1, 128, 64
    assert segment_count(B, T, H, d, d, chunk) == 4
    for kind in ("floor", "one"):
        say(f"segmented decay {kind}")
        x = make_inputs(B, T, H, d, d, "bf16", seed=41, s0_std=0.05)
        x["alpha"] = torch.full_like(x["alpha"], math.exp(-5.0) if kind == "floor" else 1.0)
        ro, rS = full_oracle(x)
        o, S = run_chunked(dev(x), chunk=chunk)
        check(to64(o), to64(S), ro, rS, "bf16", f"segmented {kind}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,H,chunk", RAGGED)
def test_ragged(dtype, B, T, H, chunk):
    dk, dv = (48, 80) if dtype == "f32" else (128, 128)
    say(f"ragged {dtype} B={B} T={T} H={H} chunk={chunk} dk={dk} dv={dv}")
    x = make_inputs(B, T, H, dk, dv, dtype, seed=100 + T, s0_std=0.5)
    ro, rS = full_oracle(x)
    o, S = run_chunked(dev(x), chunk=chunk)
    check(to64(o), to64(S), ro, rS, dtype, f"ragged T={T}")


@pytest.mark.parametrize("dk,dv", [(2, 1), (16, 16), (31, 7), (48, 80), (64, 64), (100, 128),
                                   (128, 33), (128, 128)])
def test_head_dims_fp32(dk, dv):
    say(f"head dims fp32 dk={dk} dv={dv}")
    x = make_inputs(2, 40, 2, dk, dv, "f32", seed=dk * 1000 + dv, s0_std=0.3)
    ro, rS = full_oracle(x)
    o, S = run_chunked(dev(x))
    check(to64(o), to64(S), ro, rS, "f32", f"dims {dk}x{dv}")
    xs = {n: t[:, 0].contiguous() for n, t in x.items() if n != "S0"}
    xs = dev(xs)
    od, Sd = eda.recurrent_step(xs["q"], xs["k"], xs["e"], xs["v"], xs["alpha"], xs["beta"],
                                xs["gamma"], x["S0"].to(DEV))
    ro1, rS1 = oracle.eda_ref_fwd(*(x[n][:, :1] for n in ("q", "k", "e", "v", "alpha", "beta", "gamma")),
                                  x["S0"])
    torch.cuda.synchronize()
    check(to64(od), to64(Sd), ro1[:, 0], rS1, "f32", f"decode dims {dk}x{dv}")


def test_chunk_sizes_agree_bf16():
    """Chunks of 16, 32 and 64 tokens each match the oracle on the same
    inputs (the chunk size is an implementation parameter)."""
    say("chunk 16 vs 32 vs 64 bf16")
    x = dev(make_inputs(2, 300, 4, 128, 128, "bf16", seed=5, s0_std=0.02))
    xo = {n: (None if t is None else t.cpu()) for n, t in x.items()}
    ro, rS = full_oracle(xo)
    for chunk in (16, 32, 64):
        o, S = run_chunked(x, chunk=chunk)
        check(to64(o), to64(S), ro, rS, "bf16", f"chunk{chunk}")


def test_resume_and_inplace_state():
    """chunked(T1) -> S; chunked(T2, S0=S) continues the same recurrence
    (the state is the whole checkpoint); S_final may be S0 itself."""
    say("resume T1=200 + T2=137, in-place state")
    x = make_inputs(2, 337, 3, 128, 128, "bf16", seed=9, s0_std=0.02)
    ro, rS = full_oracle(x)
    xd = dev(x)
    part = lambda a, b_: {n: (t[:, a:b_].contiguous() if n != "S0" else t) for n, t in xd.items()}
    x1 = part(0, 200)
    o1, S1 = run_chunked(x1)
    x2 = part(200, 337)
    x2["S0"] = S1
    o2, S2 = eda.fwd_chunked(*(x2[n].contiguous() for n in ("q", "k", "e", "v", "alpha", "beta", "gamma")),
                             S1, S_final=S1)  # in place
    torch.cuda.synchronize()
    assert S2.data_ptr() == S1.data_ptr()
    got_o = torch.cat([o1, o2], 1)
    check(to64(got_o), to64(S2), ro, rS, "bf16", "resume")


def test_prefill_then_decode_handoff():
    say("prefill 150 tokens then 20 decode steps")
    x = make_inputs(2, 170, 4, 128, 128, "bf16", seed=21, s0_std=0.02)
    ro, rS = full_oracle(x)
    xd = dev(x)
    pre = {n: (t[:, :150].contiguous() if n != "S0" else t) for n, t in xd.items()}
    o1, S = run_chunked(pre)
    outs = [o1]
    for t in range(150, 170):
        o, S = eda.recurrent_step(*(xd[n][:, t].contiguous() for n in
                                    ("q", "k", "e", "v", "alpha", "beta", "gamma")), S, inplace=True)
        outs.append(o[:, None])
    torch.cuda.synchronize()
    check(to64(torch.cat(outs, 1)), to64(S), ro, rS, "bf16", "handoff")


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("kind", ["floor", "one"])
def test_stress_decay_extremes(kind, chunk):
    """alpha at the safe gate's floor e^-5 on every channel (the chunk's decay
    leaves fp32 range, exercising the exact wide-decay path) and alpha = 1."""
    say(f"stress alpha={kind} chunk={chunk}")
    x = make_inputs(1, 4096, 2, 128, 128, "bf16", seed=5)
    x["alpha"] = torch.full_like(x["alpha"], math.exp(-5.0) if kind == "floor" else 1.0)
    ro, rS = full_oracle(x)
    o, S = run_chunked(dev(x), chunk=chunk)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    check(to64(o), to64(S), ro, rS, "bf16", f"stress {kind} chunk={chunk}")


@pytest.mark.parametrize("decay", [100.0, 145.0])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_strong_decay_inside_split_range(chunk, decay):
    """Half of the key channels decay by e^-100 or e^-145 over each chunk:
    still inside the split-exponent range (the element-wise path starts past
    e^-150), where the split operands reach e^{72} and a product of two of
    them would leave the fp32 range; the other half barely decays."""
    say(f"strong decay inside the split range chunk={chunk} decay={decay}")
    x = make_inputs(2, 3 * chunk + 9, 2, 128, 128, "bf16", seed=41, s0_std=0.5)
    x["alpha"][..., ::2] = math.exp(-decay / chunk)
    x["alpha"][..., 1::2] = 0.999
    ro, rS = full_oracle(x)
    o, S = run_chunked(dev(x), chunk=chunk)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    check(to64(o), to64(S), ro, rS, "bf16", f"strong decay chunk={chunk}")


# ---------------------------------------------------------------------------
# address overlap: the erase and write addresses interact through Eq. (16)'s
# cross term gamma beta (k^T e) k e^T, which independent random directions
# leave small (|cos| ~ 0.07); gates at their limits
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("kind", OVERLAP_KINDS)
def test_address_overlap_chunked(kind, chunk, dtype):
    """d = 128, an initial state, three chunks and a ragged tail."""
    T = 3 * chunk + 5
    say(f"overlap {kind} {dtype} chunk={chunk} T={T}")
    x = make_overlap_inputs(kind, 2, T, 2, 128, 128, dtype, seed=31, s0_std=0.5)
    ro, rS = full_oracle(x)
    o, S = run_chunked(dev(x), chunk=chunk)
    check(to64(o), to64(S), ro, rS, dtype, f"overlap {kind} chunk={chunk}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind", OVERLAP_KINDS)
def test_address_overlap_decode(kind, dtype):
    """The decode step on the same recipes, 40 steps in place."""
    steps = 40
    say(f"overlap decode {kind} {dtype} steps={steps}")
    x = make_overlap_inputs(kind, 64, steps, 4, 128, 128, dtype, seed=33, s0_std=0.5)
    ro, rS = full_oracle(x)
    xd = dev(x)
    S = xd["S0"].clone()
    outs = []
    for t in range(steps):
        o, S = eda.recurrent_step(*(xd[n][:, t].contiguous() for n in
                                    ("q", "k", "e", "v", "alpha", "beta", "gamma")), S, inplace=True)
        outs.append(o.clone())
    torch.cuda.synchronize()
    check(to64(torch.stack(outs, 1)), to64(S), ro, rS, dtype, f"overlap decode {kind}")


# ---------------------------------------------------------------------------
# full-size workloads, sampled heads
# ---------------------------------------------------------------------------
def sampled_check(name, n_heads, seed=0, chunk=0):
    w = WORKLOADS[name]
    say(f"{name} full size B={w.B} T={w.T} H={w.H} chunk={chunk}, {n_heads} sampled heads")
    x = make_workload(w, device=DEV)
    o, S = run_chunked(x, chunk=chunk)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    rng = np.random.default_rng(seed)
    heads = sorted({(int(rng.integers(w.B)), int(rng.integers(w.H))) for _ in range(n_heads)})
    xc = {n: (None if t is None else t.cpu()) for n, t in x.items()}
    refs = oracle_heads(xc, heads)
    go = np.concatenate([to64(o[b, :, h]) for b, h in heads])
    gs = np.concatenate([to64(S[b, h]) for b, h in heads])
    ro = np.concatenate([r[0] for r in refs])
    rs = np.concatenate([r[1] for r in refs])
    return check(go, gs, ro, rs, "bf16", f"{name} chunk={chunk} heads={heads}")


def test_timed_entry_point_matches_plain_call():
    """eda_fwd_chunked_timed (the benchmark's per-kernel timing) computes the
    same outputs, bit for bit, as eda_fwd_chunked, and its events bracket the
    two kernels in order."""
    say("timed entry point")
    x = dev(make_inputs(2, 300, 3, 128, 128, "bf16", seed=71, s0_std=0.02))
    o0, S0 = run_chunked(x)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    for ev in evs:
        ev.record()
    torch.cuda.synchronize()
    o1, S1 = run_chunked(x, events=[ev.cuda_event for ev in evs])
    assert torch.equal(o0, o1) and torch.equal(S0, S1)
    assert evs[0].elapsed_time(evs[1]) > 0 and evs[1].elapsed_time(evs[2]) > 0


@pytest.mark.slow
def test_large_workspace_ragged_slices():
    """A workspace beyond 256 MB (the state pass then warms L2 ahead of its
    factor fetches) with a ragged tail, d_v = 100 (at 8 heads the pass runs 8
    segments on two 64-column slices per head, the second one partial, and
    the segment maps on whole-width slices) and an initial state; sampled
    heads against the oracle."""
    B, T, H, dk, dv = 1, 32768 + 17, 8, 128, 100
    need = eda.workspace_size(B, T, H, dk, dv, torch.bfloat16)
    assert need > 256 << 20
    say(f"large workspace B={B} T={T} H={H} dk={dk} dv={dv} ({need >> 20} MB)")
    x = make_inputs(B, T, H, dk, dv, "bf16", seed=51, s0_std=0.02)
    o, S = run_chunked(dev(x))
    heads = [(0, 0), (0, H - 1)]
    refs = oracle_heads(x, heads)
    go = np.concatenate([to64(o[b, :, h]) for b, h in heads])
    gs = np.concatenate([to64(S[b, h]) for b, h in heads])
    check(go, gs, np.concatenate([r[0] for r in refs]), np.concatenate([r[1] for r in refs]), "bf16",
          f"large workspace heads={heads}")


@pytest.mark.slow
def test_maximum_size_heads_match_single_head_runs():
    """The largest input the ABI accepts in one call: B*T*H*d just below 2^31
    elements per token tensor (T = 131072, 127 heads) and a 24.8 GB
    workspace, so every 32-bit product of token, head and channel indices
    would overflow.  Heads are independent, so the first and last heads must
    equal, bit for bit, a run of that head repeated over 64 heads, for which
    the state pass takes the same plan (32-column slices, no segments) and so
    the same instructions per output column (the oracle checks this length in
    the very-long workload test)."""
    B, T, H, d = 1, 131072, 127, 128
    assert B * T * H * d < 2 ** 31 <= B * T * (H + 1) * d
    say(f"maximum size B={B} T={T} H={H} d={d}")
    x = make_inputs(B, T, H, d, d, "bf16", seed=61, s0_std=0.02, device=DEV)
    o, S = run_chunked(x)
    for h in (0, H - 1):
        say(f"maximum size: head {h} repeated")
        rep = [h] * 64
        xh = {n: (None if t is None else t[:, :, rep].contiguous() if t.dim() >= 3 and n != "S0"
                  else t[:, rep].contiguous()) for n, t in x.items()}
        oh, Sh = run_chunked(xh)
        assert torch.equal(oh[:, :, 0], o[:, :, h]) and torch.equal(Sh[:, 0], S[:, h]), f"head {h}"
        del xh, oh, Sh
    del x, o, S
    torch.cuda.empty_cache()


@pytest.mark.parametrize("chunk", [32, 64])
def test_train_workload_sampled(chunk):
    sampled_check("train", 8, chunk=chunk)


@pytest.mark.slow
def test_long_workload_sampled():
    sampled_check("long", 3)


@pytest.mark.slow
def test_verylong_workload_sampled():
    sampled_check("verylong", 2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_uneven_grid(dtype):
    """300 states of 128 x 128 on a grid of at most one workgroup per compute
    unit: workgroups take one or two states, so the software-pipelined loop
    runs both its prologue-only and its steady path; five steps in place,
    element-wise against the oracle's five-token recurrence."""
    N, H, d, steps = 100, 3, 128, 5
    say(f"decode uneven grid {dtype} N={N} H={H} d={d} steps={steps}")
    x = make_inputs(N, steps, H, d, d, dtype, seed=81, s0_std=0.02)
    ro, rS = full_oracle(x)
    xd = dev(x)
    S = xd["S0"].clone()
    outs = []
    for t in range(steps):
        o, S = eda.recurrent_step(*(xd[n][:, t].contiguous() for n in
                                    ("q", "k", "e", "v", "alpha", "beta", "gamma")), S, inplace=True)
        outs.append(o.clone())
    torch.cuda.synchronize()
    got = torch.stack(outs, 1)
    check(to64(got), to64(S), ro, rS, dtype, f"decode uneven grid")


def test_decode_workload_sampled():
    """256 sequences x 32 heads, 128 one-token steps updating the state in
    place; the oracle runs the sampled (n, h) heads over the same 128 steps."""
    w = WORKLOADS["decode"]
    say(f"decode N={w.B} H={w.H} steps={w.steps}")
    x = make_workload(w, device=DEV)
    S = x["S0"].clone()
    outs = []
    for t in range(w.steps):
        o, S = eda.recurrent_step(*(x[n][t] for n in ("q", "k", "e", "v", "alpha", "beta", "gamma")),
                                  S, inplace=True)
        outs.append(o)
    torch.cuda.synchronize()
    got = torch.stack(outs)  # [steps, N, H, dv]
    rng = np.random.default_rng(1)
    heads = sorted({(int(rng.integers(w.B)), int(rng.integers(w.H))) for _ in range(24)})
    xc = {n: t.cpu() for n, t in x.items()}
    go, gs, ro, rs = [], [], [], []
    for n_, h in heads:
        sel = {n: xc[n][:, n_:n_ + 1, h:h + 1] for n in ("q", "k", "e", "v", "alpha", "beta", "gamma")}
        o_ref, S_ref = oracle.eda_ref_decode(**sel, S0=xc["S0"][n_:n_ + 1, h:h + 1])
        go.append(to64(got[:, n_, h])); ro.append(o_ref[:, 0, 0])
        gs.append(to64(S[n_, h])); rs.append(S_ref[0, 0])
    check(np.concatenate(go), np.concatenate(gs), np.concatenate(ro), np.concatenate(rs), "bf16",
          f"decode heads={len(heads)}")
