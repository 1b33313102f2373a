"""eda_fwd_chunked_noalloc (workspace in the library's per-device scratch
array) against eda_fwd_chunked (caller workspace) on the same inputs.

Both run the same kernels, so the outputs must agree to the parity bar, and
in fact bit for bit.  Three calls in a row, each smaller than the one
before, show that the contents left in the shared array by one call do not
leak into the next.  The first has one head and 300 chunks, so the bf16
state pass runs in segments (4 at chunk 64, 8 at chunk 32), with the segment
maps and their prefix in the array as well.
"""
import pytest
import torch

import recurrent_memory_amd as eda
from eda_inputs import make_inputs
from _helpers import check, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"[case] {msg}", flush=True)


def both(x, chunk):
    args = (x["q"], x["k"], x["e"], x["v"], x["alpha"], x["beta"], x["gamma"], x["S0"])
    o_ref, S_ref = eda.fwd_chunked(*args, chunk=chunk)
    B, T, H, dk = x["q"].shape
    dv = x["v"].shape[-1]
    out = torch.empty((B, T, H, dv), dtype=x["q"].dtype, device=DEV)
    S_fin = torch.empty((B, H, dk, dv), dtype=torch.float32, device=DEV)
    o, S = eda.fwd_chunked_noalloc(*args, out=out, S_final=S_fin, chunk=chunk)
    torch.cuda.synchronize()
    return o, S, o_ref, S_ref


# (B, T, H, d_k, d_v): a segmented call, a smaller one, then one with a ragged tail
SHAPES = [(1, 64 * 300, 1, 128, 128), (2, 1000, 8, 128, 128), (1, 77, 3, 64, 40)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("chunk", [0, 32])
def test_noalloc_matches_workspace_call(dtype, chunk):
    for i, (B, T, H, dk, dv) in enumerate(SHAPES):
        say(f"noalloc {dtype} chunk={chunk} call {i}: B={B} T={T} H={H} dk={dk} dv={dv}")
        x = make_inputs(B, T, H, dk, dv, dtype, seed=900 + i, s0_std=0.05, device=DEV)
        o, S, o_ref, S_ref = both(x, chunk)
        check(to64(o), to64(S), to64(o_ref), to64(S_ref), dtype, label=f"noalloc call {i}")
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref)


def test_noalloc_rejects_oversize_problem():
    # bf16, chunk 64, d = 128, 64 heads: 36 chunks per head need more than the 160 MiB array
    B, T, H = 4, 64 * 36, 16
    assert eda.workspace_size(B, T, H, 128, 128, torch.bfloat16, 64) > 160 << 20
    say("noalloc oversize rejection")
    x = make_inputs(B, T, H, 128, 128, "bf16", seed=7, device=DEV)
    out = torch.empty_like(x["v"])
    with pytest.raises(eda.EdaError) as err:
        eda.fwd_chunked_noalloc(x["q"], x["k"], x["e"], x["v"], x["alpha"], x["beta"], x["gamma"], None,
                                out=out, chunk=64)
    assert err.value.code == 9
