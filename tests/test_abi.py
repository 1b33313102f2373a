"""C-ABI contract tests that need the built library but no GPU.

Every argument check in libeda.so runs before any HIP call, so invalid
calls can be made with fake (never dereferenced) device addresses.
"""
import ctypes
import os
import re

import pytest

import recurrent_memory_amd as eda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "eda.h")

pytestmark = pytest.mark.skipif(not os.path.exists(eda.library_path()),
                                reason="libeda.so not built")


def declared_functions():
    src = open(HDR).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(eda_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("eda_fwd_chunked", "eda_fwd_chunked_timed", "eda_fwd_recurrent_step",
              "eda_fwd_chunked_workspace_size", "eda_status_string", "eda_fwd_chunked_layer",
              "eda_fwd_chunked_layer_workspace_size", "eda_fwd_recurrent_step_layer",
              "eda_fwd_chunked_dplr", "eda_fwd_recurrent_step_dplr", "eda_bwd",
              "eda_bwd_workspace_size"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(eda.library_path())
    for n in declared_functions():
        assert hasattr(lib, n), f"libeda.so does not export {n}"


def test_status_strings():
    lib = eda.load_library()
    for code in range(10):
        s = lib.eda_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.eda_status_string(99).decode() == "unknown status"


def test_workspace_size():
    lib = eda.load_library()
    ws = lib.eda_fwd_chunked_workspace_size
    # bf16: one block per chunk and head holding Phi (d_k x d_k), Psi (d_k x C),
    # Qhat (C x d_k), Phat (C x C) as 1 KB operand fragments and e^{G_C} (fp32)
    frag = lambda C, D: (D // 16) * (D // 32) + (D // 16) * -(-C // 32) + (C // 16) * (D // 32) + (C // 16) * -(-C // 32)
    blk = lambda C, D: -(-(frag(C, D) * 1024 + 4 * D) // 256) * 256
    assert (blk(64, 128), blk(32, 128), blk(16, 128)) == (74240, 51712, 46592)
    bf = ws(4, 2048, 16, 128, 128, 1, 32)
    assert bf == 4 * 16 * (2048 // 32) * blk(32, 128)
    assert ws(4, 2048 + 1, 16, 128, 128, 1, 32) == bf + 4 * 16 * blk(32, 128)   # a ragged tail is a chunk
    bf64 = ws(4, 2048, 16, 128, 128, 1, 64)
    assert bf64 == 4 * 16 * (2048 // 64) * blk(64, 128)
    assert ws(4, 2048, 16, 128, 128, 1, 0) == bf64            # 0 selects the default chunk, 64
    assert ws(1, 100, 3, 64, 40, 1, 16) == 3 * 7 * blk(16, 64)   # head dims padded to 32, 64 or 128
    big = ws(4, 2048, 16, 128, 128, 0, 32)                    # fp32 chunk factors
    assert big > 0
    # fp32 computes chunk 64 as 32-token chunks (same workspace)
    assert ws(4, 2048, 16, 128, 128, 0, 64) == big
    assert ws(4, 2048, 16, 128, 128, 0, 0) == big            # 0 selects the default chunk
    assert ws(4, 4096, 16, 128, 128, 0, 32) == 2 * big        # linear in the chunk count
    assert ws(1, 1, 1, 2, 1, 0, 16) > 0
    assert ws(4, 2048, 16, 129, 128, 0, 32) == 0              # unsupported head dim
    assert ws(4, 2048, 16, 128, 128, 0, 48) == 0              # unsupported chunk
    assert ws(4, 2048, 16, 128, 128, 7, 32) == 0              # bad dtype
    assert ws(0, 2048, 16, 128, 128, 0, 32) == 0


def _bf16_segments(B, T, H, dk, dv, chunk=64):
    """Segments per head of the bf16 state pass, read back from the workspace
    size (the chunk factors plus, with P > 1, B H (P - 1) d_k (d_k + 2 d_v) fp32)."""
    ws = eda.load_library().eda_fwd_chunked_workspace_size
    D = 32 if max(dk, dv) <= 32 else 64 if max(dk, dv) <= 64 else 128
    frag = (D // 16) * (D // 32) + (D // 16) * -(-chunk // 32) + (chunk // 16) * (D // 32) + (chunk // 16) * -(-chunk // 32)
    blk = -(-(frag * 1024 + 4 * D) // 256) * 256
    extra = ws(B, T, H, dk, dv, 1, chunk) - B * H * -(-T // chunk) * blk
    per = B * H * dk * (dk + 2 * dv) * 4
    assert extra >= 0 and extra % per == 0
    return 1 + extra // per


@pytest.mark.parametrize("B,T,H,dk,dv,P", [
    (4, 2048, 16, 128, 128, 1),       # the training shape: many heads, 32 chunks
    (1, 32768, 32, 128, 128, 1),      # 32 heads fill the chip with 16-column slices
    (1, 32768, 16, 128, 128, 8),      # 16 heads at T = 32768: 8 segments of 64 chunks
    (1, 131072, 16, 128, 128, 8),     # 16 would need 512 pass workgroups
    (1, 64 * 255, 1, 128, 128, 1),    # fewer than 256 chunks
    (1, 64 * 256, 1, 128, 128, 4),    # at least 64 chunks per segment
    (2, 32768, 4, 128, 128, 8),
    (1, 65536, 8, 128, 128, 16),      # 256 pass and 240 map workgroups
    (1, 32768, 16, 64, 64, 8),        # d = 64: whole-width slices of 64 columns
])
def test_segment_plan(B, T, H, dk, dv, P):
    """The state pass's segment count at chunk 64: the largest power of two that
    keeps at least 64 chunks per segment and at most 256 workgroups both in the
    pass (64-column slices) and in the segment maps (two whole-width slices per
    head and segment), for few heads (B H d / 16 < 256) and at least 256 chunks."""
    assert _bf16_segments(B, T, H, dk, dv) == P


# Fake device addresses: distinct, 256-byte aligned, far apart, never dereferenced.
BASE = 1 << 40


def fake(i, off=0):
    return ctypes.c_void_p(BASE + (i << 32) + off)


def chunked_args(**kw):
    # fp32 (dt=0): the path that needs a workspace, so every rejection below is
    # decided by a check before any launch
    B, T, H, dk, dv, dt, chunk = 2, 64, 2, 64, 64, 0, 32
    a = dict(q=fake(1), k=fake(2), e=fake(3), v=fake(4), alpha=fake(5), beta=fake(6),
             gamma=fake(7), S0=fake(8), o=fake(9), S_final=fake(10), B=B, T=T, H=H, dk=dk, dv=dv,
             dt=dt, chunk=chunk, ws=fake(11), wsb=1 << 30, stream=None)
    a.update(kw)
    return a


def call_chunked(a):
    lib = eda.load_library()
    return lib.eda_fwd_chunked(a["q"], a["k"], a["e"], a["v"], a["alpha"], a["beta"], a["gamma"],
                               a["S0"], a["o"], a["S_final"], a["B"], a["T"], a["H"], a["dk"],
                               a["dv"], a["dt"], a["chunk"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("field,val,code", [
    ("q", None, 1), ("v", None, 1), ("alpha", None, 1), ("o", None, 1),
    ("dt", 5, 3),
    ("B", 0, 2), ("T", -1, 2), ("dk", 0, 2),
    ("dk", 129, 5), ("dv", 200, 5), ("chunk", 128, 5), ("chunk", 7, 5),
    ("q", fake(1, 2), 4), ("alpha", fake(5, 2), 4), ("S0", fake(8, 4), 4), ("o", fake(9, 8), 4),
    ("ws", fake(11, 128), 4),
    ("ws", None, 6), ("wsb", 1024, 6),
    ("o", fake(1, 256), 7),           # o inside q
    ("S_final", fake(8, 256), 7),     # partial overlap with S0
    ("o", fake(11, 512), 7),          # o inside the workspace
])
def test_chunked_rejects(field, val, code):
    assert call_chunked(chunked_args(**{field: val})) == code


def test_scalar_inputs_need_only_element_alignment():
    # per-token gates sliced out of a stacked tensor sit at 4-byte offsets
    assert call_chunked(chunked_args(beta=fake(6, 4), gamma=fake(7, 12), alpha=fake(5, 4),
                                     q=fake(1, 4), wsb=16)) == 6  # reaches the workspace check


def test_bf16_misaligned_input_rejected():
    assert call_chunked(chunked_args(q=fake(1, 1), dt=1)) == 4


def call_chunked_timed(a, events):
    lib = eda.load_library()
    return lib.eda_fwd_chunked_timed(a["q"], a["k"], a["e"], a["v"], a["alpha"], a["beta"], a["gamma"],
                                     a["S0"], a["o"], a["S_final"], a["B"], a["T"], a["H"], a["dk"],
                                     a["dv"], a["dt"], a["chunk"], a["ws"], a["wsb"], a["stream"], events)


def test_timed_variant_checks_like_the_plain_call():
    # a missing event is a NULL argument; every other check is the plain call's
    evs = (ctypes.c_void_p * 3)(fake(20), None, fake(22))
    assert call_chunked_timed(chunked_args(), evs) == 1
    evs = (ctypes.c_void_p * 3)(fake(20), fake(21), fake(22))
    assert call_chunked_timed(chunked_args(q=None), evs) == 1
    assert call_chunked_timed(chunked_args(chunk=7), evs) == 5
    assert call_chunked_timed(chunked_args(ws=None), evs) == 6
    assert call_chunked_timed(chunked_args(o=fake(1, 256)), None) == 7


def call_chunked_noalloc(a):
    lib = eda.load_library()
    return lib.eda_fwd_chunked_noalloc(a["q"], a["k"], a["e"], a["v"], a["alpha"], a["beta"], a["gamma"],
                                       a["S0"], a["o"], a["S_final"], a["B"], a["T"], a["H"], a["dk"],
                                       a["dv"], a["dt"], a["chunk"], a["stream"])


def test_noalloc_variant_checks_before_any_hip_call():
    # argument checks are the plain call's; a problem beyond the scratch array
    # is rejected (EDA_ERR_SCRATCH) before the array is looked up
    assert call_chunked_noalloc(chunked_args(q=None)) == 1
    assert call_chunked_noalloc(chunked_args(dt=5)) == 3
    assert call_chunked_noalloc(chunked_args(chunk=7)) == 5
    assert call_chunked_noalloc(chunked_args(o=fake(9, 8))) == 4
    ws = eda.load_library().eda_fwd_chunked_workspace_size
    limit = 160 << 20
    # bf16, d = 128, chunk 64, 64 heads: 74240 bytes per chunk-head, 35 chunks fit
    assert ws(4, 64 * 35, 16, 128, 128, 1, 64) <= limit < ws(4, 64 * 36, 16, 128, 128, 1, 64)
    assert call_chunked_noalloc(chunked_args(B=4, T=64 * 36, H=16, dk=128, dv=128, dt=1, chunk=64)) == 9
    assert call_chunked_noalloc(chunked_args(B=8, T=4096, H=16, dk=128, dv=128, dt=0, chunk=0)) == 9


def test_chunked_too_large_shape():
    assert call_chunked(chunked_args(B=1 << 12, T=1 << 12, H=1 << 4, dk=128, dv=128)) == 2


def call_step(**kw):
    a = dict(q=fake(1), k=fake(2), e=fake(3), v=fake(4), alpha=fake(5), beta=fake(6), gamma=fake(7),
             S_in=fake(8), S_out=fake(9), o=fake(10), N=4, H=2, dk=128, dv=128, dt=1, stream=None)
    a.update(kw)
    lib = eda.load_library()
    return lib.eda_fwd_recurrent_step(a["q"], a["k"], a["e"], a["v"], a["alpha"], a["beta"],
                                      a["gamma"], a["S_in"], a["S_out"], a["o"], a["N"], a["H"],
                                      a["dk"], a["dv"], a["dt"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(S_out=None), 1), (dict(o=None), 1), (dict(k=None), 1),
    (dict(dt=2), 3), (dict(N=0), 2), (dict(dv=0), 2), (dict(dk=130), 5),
    (dict(e=fake(3, 1)), 4), (dict(beta=fake(6, 2)), 4), (dict(S_in=fake(8, 8)), 4),
    (dict(S_out=fake(8, 1024)), 7),    # partial overlap with S_in
    (dict(o=fake(1, 64)), 7),          # o inside q
    (dict(S_out=fake(5)), 7),          # state written over alpha
])
def test_step_rejects(kw, code):
    assert call_step(**kw) == code


def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros((1, 4, 1, 8))
    with pytest.raises(ValueError, match="GPU tensor"):
        eda.fwd_chunked(x, x, x, x, x, x[..., 0], x[..., 0])


# ---- layer form ------------------------------------------------------------
def test_layer_workspace_size():
    lib = eda.load_library()
    ws, lws = lib.eda_fwd_chunked_workspace_size, lib.eda_fwd_chunked_layer_workspace_size
    # bf16: the prologue is fused, the workspace is the value heads' factor blocks
    assert lws(4, 2048, 8, 16, 128, 128, 1, 32) == ws(4, 2048, 16, 128, 128, 1, 32)
    # fp32: the prologue pass adds q, k, e, alpha per value head after the factors
    base = ws(1, 64, 4, 16, 16, 0, 16)
    assert lws(1, 64, 2, 4, 16, 16, 0, 16) >= base + 4 * 64 * 4 * 16 * 4
    assert lws(1, 64, 3, 4, 16, 16, 0, 16) == 0              # H_v not a multiple of H_k
    assert lws(1, 64, 0, 4, 16, 16, 0, 16) == 0


def layer_args(**kw):
    a = dict(q=fake(1), k=fake(2), e=fake(3), v=fake(4), a=fake(5), A_log=fake(12), dt_bias=fake(13),
             beta=fake(6), gamma=fake(7), S0=fake(8), o=fake(9), S_final=fake(10), B=2, T=64, Hk=2,
             Hv=4, dk=64, dv=64, dt=0, chunk=32, ws=fake(11), wsb=1 << 30, stream=None)
    a.update(kw)
    return a


def call_layer(a):
    lib = eda.load_library()
    return lib.eda_fwd_chunked_layer(a["q"], a["k"], a["e"], a["v"], a["a"], a["A_log"], a["dt_bias"],
                                     a["beta"], a["gamma"], a["S0"], a["o"], a["S_final"], a["B"], a["T"],
                                     a["Hk"], a["Hv"], a["dk"], a["dv"], a["dt"], a["chunk"], a["ws"],
                                     a["wsb"], a["stream"])


@pytest.mark.parametrize("field,val,code", [
    ("a", None, 1), ("A_log", None, 1), ("dt_bias", None, 1), ("q", None, 1),
    ("dt", 4, 3),
    ("Hv", 5, 2), ("Hk", 0, 2), ("Hv", 1, 2),          # H_v must be a positive multiple of H_k
    ("dk", 200, 5), ("chunk", 48, 5),
    ("A_log", fake(12, 2), 4), ("a", fake(5, 2), 4),
    ("ws", None, 6), ("wsb", 4096, 6),
    ("o", fake(5, 512), 7),           # o inside a
    ("S_final", fake(12), 7),         # state over A_log
])
def test_layer_rejects(field, val, code):
    assert call_layer(layer_args(**{field: val})) == code


def call_step_layer(**kw):
    a = dict(q=fake(1), k=fake(2), e=fake(3), v=fake(4), a=fake(5), A_log=fake(12), dt_bias=fake(13),
             beta=fake(6), gamma=fake(7), S_in=fake(8), S_out=fake(9), o=fake(10), N=4, Hk=2, Hv=4,
             dk=128, dv=128, dt=1, stream=None)
    a.update(kw)
    lib = eda.load_library()
    return lib.eda_fwd_recurrent_step_layer(a["q"], a["k"], a["e"], a["v"], a["a"], a["A_log"],
                                            a["dt_bias"], a["beta"], a["gamma"], a["S_in"], a["S_out"],
                                            a["o"], a["N"], a["Hk"], a["Hv"], a["dk"], a["dv"], a["dt"],
                                            a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(a=None), 1), (dict(dt_bias=None), 1), (dict(S_out=None), 1),
    (dict(dt=9), 3), (dict(Hv=3), 2), (dict(N=0), 2), (dict(dk=0), 2), (dict(dv=129), 5),
    (dict(dt_bias=fake(13, 2)), 4), (dict(S_out=fake(9, 8)), 4),
    (dict(o=fake(5, 64)), 7), (dict(S_out=fake(8, 4096)), 7),
])
def test_step_layer_rejects(kw, code):
    assert call_step_layer(**kw) == code


# ---- rank-1 DPLR update -----------------------------------------------------
def call_dplr(**kw):
    a = chunked_args(**kw)
    a.setdefault("a", fake(3))
    lib = eda.load_library()
    return lib.eda_fwd_chunked_dplr(a["q"], a["k"], a.get("a_vec", fake(3)), a["v"], a["alpha"], a["S0"], a["o"],
                                    a["S_final"], a["B"], a["T"], a["H"], a["dk"], a["dv"], a["dt"], a["chunk"],
                                    a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(a_vec=None), 1), (dict(q=None), 1), (dict(alpha=None), 1),
    (dict(dt=3), 3), (dict(T=0), 2), (dict(dk=256), 5), (dict(chunk=8), 5),
    (dict(a_vec=fake(3, 2)), 4), (dict(ws=None), 6), (dict(o=fake(3, 256)), 7),
])
def test_dplr_rejects(kw, code):
    assert call_dplr(**kw) == code


def test_dplr_reaches_the_workspace_check_without_gates():
    # beta and gamma are not arguments of the DPLR update: a valid call fails only on the workspace
    assert call_dplr(wsb=16) == 6


@pytest.mark.parametrize("kw,code", [
    (dict(a=None), 1), (dict(S_out=None), 1), (dict(dt=7), 3), (dict(H=0), 2), (dict(dk=129), 5),
    (dict(a=fake(3, 1)), 4), (dict(o=fake(1, 64)), 7),
])
def test_step_dplr_rejects(kw, code):
    a = dict(q=fake(1), k=fake(2), a=fake(3), v=fake(4), alpha=fake(5), S_in=fake(8), S_out=fake(9),
             o=fake(10), N=4, H=2, dk=128, dv=128, dt=1, stream=None)
    a.update(kw)
    lib = eda.load_library()
    assert lib.eda_fwd_recurrent_step_dplr(a["q"], a["k"], a["a"], a["v"], a["alpha"], a["S_in"], a["S_out"],
                                           a["o"], a["N"], a["H"], a["dk"], a["dv"], a["dt"],
                                           a["stream"]) == code


# ---- backward ----------------------------------------------------------------
def call_bwd(**kw):
    a = dict(q=fake(1), k=fake(2), e=fake(3), v=fake(4), alpha=fake(5), beta=fake(6), gamma=fake(7),
             S0=fake(8), dO=fake(9), dSf=fake(10), dq=fake(20), dk=fake(21), de=fake(22), dv=fake(23),
             da=fake(24), db=fake(25), dg=fake(26), dS0=fake(27), B=2, T=64, H=2, dk_=64, dv_=64, dt=1,
             ws=fake(11), wsb=1 << 34, stream=None)
    a.update(kw)
    lib = eda.load_library()
    return lib.eda_bwd(a["q"], a["k"], a["e"], a["v"], a["alpha"], a["beta"], a["gamma"], a["S0"], a["dO"],
                       a["dSf"], a["dq"], a["dk"], a["de"], a["dv"], a["da"], a["db"], a["dg"], a["dS0"], a["B"],
                       a["T"], a["H"], a["dk_"], a["dv_"], a["dt"], a["ws"], a["wsb"], a["stream"])


def test_bwd_workspace_size():
    ws = eda.load_library().eda_bwd_workspace_size
    assert ws(4, 2048, 16, 128, 128) > ws(4, 1024, 16, 128, 128) > 0
    assert ws(1, 1, 1, 129, 4) == 0 and ws(0, 8, 1, 4, 4) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(dO=None), 1), (dict(dq=None), 1), (dict(dg=None), 1), (dict(gamma=None), 1),
    (dict(dt=5), 3), (dict(T=0), 2), (dict(dk_=130), 5),
    (dict(dO=fake(9, 1)), 4), (dict(da=fake(24, 2)), 4), (dict(ws=fake(11, 64)), 4),
    (dict(ws=None), 6), (dict(wsb=1024), 6),
    (dict(dq=fake(1, 256)), 7),       # gradient over an input
    (dict(dk=fake(20, 4096)), 7),     # two gradients overlap
    (dict(dv=fake(11, 512)), 7),      # gradient inside the workspace
])
def test_bwd_rejects(kw, code):
    assert call_bwd(**kw) == code


def test_bwd_optional_state_arguments():
    # S0, dS_final and dS0 may be NULL; such a call fails only on the workspace
    assert call_bwd(S0=None, dSf=None, dS0=None, wsb=16) == 6

