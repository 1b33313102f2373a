"""MI355X (gfx950) Erase-then-Delta Attention forward.

Thin Python binding over `libeda.so` (C ABI in include/eda.h).  This module
only checks tensor placement and passes device pointers and sizes; every
step of the computation runs in the library's HIP kernels.  There is no CPU
or PyTorch fallback: if the library is not built, or a tensor is not on a
GPU, the call raises.

    o, S = fwd_chunked(q, k, e, v, alpha, beta, gamma, S0=None)
    o, S = recurrent_step(q, k, e, v, alpha, beta, gamma, S_in, inplace=True)
    o, S = fwd_chunked_layer(q, k, e, v, a, A_log, dt_bias, beta, gamma, S0=None)
    o, S = recurrent_step_layer(q, k, e, v, a, A_log, dt_bias, beta, gamma, S_in)
    o, S = fwd_chunked_dplr(q, k, a, v, alpha, S0=None)       # GDN-2 / QED update
    o, S = recurrent_step_dplr(q, k, a, v, alpha, S_in)
    grads = backward(q, k, e, v, alpha, beta, gamma, S0, dO, dS_final)

Layouts follow the C ABI: q, k, e, alpha [B, T, H, d_k]; v, o [B, T, H, d_v];
beta, gamma [B, T, H]; states [B, H, d_k, d_v] fp32 (decode drops the T
axis).  q, k, e, v share one dtype (bfloat16 or float32); alpha, beta,
gamma and the states are float32.  The layer forms take raw q, k, e and the
decay gate's input a per key head ([..., H_k, d_k]), A_log and dt_bias
[H_k, d_k] float32, and v, beta, gamma, o, states per value head (H_v, a
multiple of H_k).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = ["fwd_chunked", "recurrent_step", "fwd_chunked_layer", "recurrent_step_layer",
           "fwd_chunked_dplr", "recurrent_step_dplr", "backward",
           "workspace_size", "layer_workspace_size", "library_path", "load_library",
           "EdaError", "STATUS", "DEFAULT_CHUNK"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libeda.so")
_lib = None
DEFAULT_CHUNK = 64

STATUS = {0: "EDA_OK", 1: "EDA_ERR_NULL", 2: "EDA_ERR_SHAPE", 3: "EDA_ERR_DTYPE",
          4: "EDA_ERR_ALIGN", 5: "EDA_ERR_UNSUPPORTED", 6: "EDA_ERR_WORKSPACE",
          7: "EDA_ERR_ALIAS", 8: "EDA_ERR_HIP", 9: "EDA_ERR_SCRATCH"}
EDA_F32, EDA_BF16 = 0, 1


class EdaError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn}: {STATUS.get(code, code)} ({msg})")
        self.code = code


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libeda.so; raise if it has not been built (no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"EDA HIP library not built: {_LIB_PATH} is missing "
                           "(run `python -m recurrent_memory_amd.build`)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, fp, i, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.eda_status_string.argtypes = [i]
    lib.eda_status_string.restype = ctypes.c_char_p
    lib.eda_fwd_chunked_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.eda_fwd_chunked_workspace_size.restype = sz
    lib.eda_fwd_chunked.argtypes = [vp, vp, vp, vp, fp, fp, fp, fp, vp, fp,
                                    i, i, i, i, i, i, i, vp, sz, vp]
    lib.eda_fwd_chunked.restype = i
    lib.eda_fwd_chunked_noalloc.argtypes = [vp, vp, vp, vp, fp, fp, fp, fp, vp, fp,
                                            i, i, i, i, i, i, i, vp]
    lib.eda_fwd_chunked_noalloc.restype = i
    lib.eda_fwd_chunked_timed.argtypes = [vp, vp, vp, vp, fp, fp, fp, fp, vp, fp,
                                          i, i, i, i, i, i, i, vp, sz, vp, ctypes.POINTER(vp)]
    lib.eda_fwd_chunked_timed.restype = i
    lib.eda_fwd_recurrent_step.argtypes = [vp, vp, vp, vp, fp, fp, fp, fp, fp, vp,
                                           i, i, i, i, i, vp]
    lib.eda_fwd_recurrent_step.restype = i
    lib.eda_fwd_chunked_layer_workspace_size.argtypes = [i, i, i, i, i, i, i, i]
    lib.eda_fwd_chunked_layer_workspace_size.restype = sz
    lib.eda_fwd_chunked_layer.argtypes = [vp, vp, vp, vp, vp, fp, fp, fp, fp, fp, vp, fp,
                                          i, i, i, i, i, i, i, i, vp, sz, vp]
    lib.eda_fwd_chunked_layer.restype = i
    lib.eda_fwd_recurrent_step_layer.argtypes = [vp, vp, vp, vp, vp, fp, fp, fp, fp, fp, fp, vp,
                                                 i, i, i, i, i, i, vp]
    lib.eda_fwd_recurrent_step_layer.restype = i
    lib.eda_fwd_chunked_dplr.argtypes = [vp, vp, vp, vp, fp, fp, vp, fp, i, i, i, i, i, i, i, vp, sz, vp]
    lib.eda_fwd_chunked_dplr.restype = i
    lib.eda_fwd_recurrent_step_dplr.argtypes = [vp, vp, vp, vp, fp, fp, fp, vp, i, i, i, i, i, vp]
    lib.eda_fwd_recurrent_step_dplr.restype = i
    lib.eda_bwd_workspace_size.argtypes = [i, i, i, i, i]
    lib.eda_bwd_workspace_size.restype = sz
    lib.eda_bwd.argtypes = [vp, vp, vp, vp, fp, fp, fp, fp, vp, fp, fp, fp, fp, fp, fp, fp, fp, fp,
                            i, i, i, i, i, i, vp, sz, vp]
    lib.eda_bwd.restype = i
    _lib = lib
    return lib


def _check(fn: str, code: int):
    if code != 0:
        msg = load_library().eda_status_string(code).decode()
        raise EdaError(fn, code, msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return EDA_BF16
    if t.dtype == torch.float32:
        return EDA_F32
    raise TypeError(f"unsupported input dtype {t.dtype} (use bfloat16 or float32)")


def _ptr(t: Optional[torch.Tensor], name: str, dtype: Optional[torch.dtype] = None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def workspace_size(B: int, T: int, H: int, d_k: int, d_v: int, dtype: torch.dtype,
                   chunk: int = 0) -> int:
    code = EDA_BF16 if dtype == torch.bfloat16 else EDA_F32
    return int(load_library().eda_fwd_chunked_workspace_size(B, T, H, d_k, d_v, code, chunk))


def fwd_chunked(q, k, e, v, alpha, beta, gamma, S0=None, *, chunk: int = 0,
                want_state: bool = True, out: Optional[torch.Tensor] = None,
                S_final: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None,
                events=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunk-parallel forward over [B, T, H, d] inputs; returns (o, S_final).
    `events`: optional three raw HIP event handles recorded before the factor
    kernel, between the two kernels and after the state pass
    (eda_fwd_chunked_timed)."""
    lib = load_library()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    if S_final is None and want_state:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    need = int(lib.eda_fwd_chunked_workspace_size(B, T, H, dk, dv, dt, chunk))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    args = (_ptr(q, "q", q.dtype), _ptr(k, "k", q.dtype), _ptr(e, "e", q.dtype), _ptr(v, "v", q.dtype),
            _ptr(alpha, "alpha", torch.float32), _ptr(beta, "beta", torch.float32),
            _ptr(gamma, "gamma", torch.float32), _ptr(S0, "S0", torch.float32),
            _ptr(out, "o", q.dtype), _ptr(S_final, "S_final", torch.float32),
            B, T, H, dk, dv, dt, chunk, _ptr(workspace, "workspace"),
            0 if workspace is None else workspace.numel(), _stream(q.device))
    if events is None:
        _check("eda_fwd_chunked", lib.eda_fwd_chunked(*args))
    else:
        evs = (ctypes.c_void_p * 3)(*[ctypes.c_void_p(int(x)) for x in events])
        _check("eda_fwd_chunked_timed", lib.eda_fwd_chunked_timed(*args, evs))
    return out, S_final


def fwd_chunked_noalloc(q, k, e, v, alpha, beta, gamma, S0=None, *, out: torch.Tensor,
                        S_final: Optional[torch.Tensor] = None,
                        chunk: int = 0) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """fwd_chunked through eda_fwd_chunked_noalloc: the caller passes the
    outputs (`out`, and `S_final` or None) and the library takes its workspace
    from its per-device scratch array, so nothing is allocated."""
    lib = load_library()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    args = (_ptr(q, "q", q.dtype), _ptr(k, "k", q.dtype), _ptr(e, "e", q.dtype), _ptr(v, "v", q.dtype),
            _ptr(alpha, "alpha", torch.float32), _ptr(beta, "beta", torch.float32),
            _ptr(gamma, "gamma", torch.float32), _ptr(S0, "S0", torch.float32),
            _ptr(out, "o", q.dtype), _ptr(S_final, "S_final", torch.float32),
            B, T, H, dk, dv, dt, chunk, _stream(q.device))
    _check("eda_fwd_chunked_noalloc", lib.eda_fwd_chunked_noalloc(*args))
    return out, S_final


def recurrent_step(q, k, e, v, alpha, beta, gamma, S_in=None, *, S_out: Optional[torch.Tensor] = None,
                   o: Optional[torch.Tensor] = None, inplace: bool = False):
    """One decode token for [N, H, d] inputs; returns (o, S_out).  With
    inplace=True the state is updated in S_in's memory."""
    lib = load_library()
    N, H, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    if inplace:
        if S_in is None:
            raise ValueError("inplace=True needs S_in")
        S_out = S_in
    if S_out is None:
        S_out = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    code = lib.eda_fwd_recurrent_step(
        _ptr(q, "q", q.dtype), _ptr(k, "k", q.dtype), _ptr(e, "e", q.dtype), _ptr(v, "v", q.dtype),
        _ptr(alpha, "alpha", torch.float32), _ptr(beta, "beta", torch.float32),
        _ptr(gamma, "gamma", torch.float32), _ptr(S_in, "S_in", torch.float32),
        _ptr(S_out, "S_out", torch.float32), _ptr(o, "o", q.dtype), N, H, dk, dv, dt,
        _stream(q.device))
    _check("eda_fwd_recurrent_step", code)
    return o, S_out


def layer_workspace_size(B: int, T: int, H_k: int, H_v: int, d_k: int, d_v: int,
                         dtype: torch.dtype, chunk: int = 0) -> int:
    code = EDA_BF16 if dtype == torch.bfloat16 else EDA_F32
    return int(load_library().eda_fwd_chunked_layer_workspace_size(B, T, H_k, H_v, d_k, d_v, code, chunk))


def fwd_chunked_layer(q, k, e, v, a, A_log, dt_bias, beta, gamma, S0=None, *, chunk: int = 0,
                      want_state: bool = True, out: Optional[torch.Tensor] = None,
                      S_final: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None):
    """Layer-form chunked forward (eda_fwd_chunked_layer): raw q, k, e, a
    [B, T, H_k, d_k], v [B, T, H_v, d_v]; returns (o, S_final)."""
    lib = load_library()
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty((B, T, Hv, dv), dtype=q.dtype, device=q.device)
    if S_final is None and want_state:
        S_final = torch.empty((B, Hv, dk, dv), dtype=torch.float32, device=q.device)
    need = int(lib.eda_fwd_chunked_layer_workspace_size(B, T, Hk, Hv, dk, dv, dt, chunk))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    code = lib.eda_fwd_chunked_layer(
        _ptr(q, "q", q.dtype), _ptr(k, "k", q.dtype), _ptr(e, "e", q.dtype), _ptr(v, "v", q.dtype),
        _ptr(a, "a", q.dtype), _ptr(A_log, "A_log", torch.float32),
        _ptr(dt_bias, "dt_bias", torch.float32), _ptr(beta, "beta", torch.float32),
        _ptr(gamma, "gamma", torch.float32), _ptr(S0, "S0", torch.float32),
        _ptr(out, "o", q.dtype), _ptr(S_final, "S_final", torch.float32),
        B, T, Hk, Hv, dk, dv, dt, chunk, _ptr(workspace, "workspace"),
        0 if workspace is None else workspace.numel(), _stream(q.device))
    _check("eda_fwd_chunked_layer", code)
    return out, S_final


def recurrent_step_layer(q, k, e, v, a, A_log, dt_bias, beta, gamma, S_in=None, *,
                         S_out: Optional[torch.Tensor] = None, o: Optional[torch.Tensor] = None,
                         inplace: bool = False):
    """Layer-form decode token (eda_fwd_recurrent_step_layer): raw q, k, e, a
    [N, H_k, d_k], v [N, H_v, d_v]; returns (o, S_out)."""
    lib = load_library()
    N, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    dt = _dtype_code(q)
    if inplace:
        if S_in is None:
            raise ValueError("inplace=True needs S_in")
        S_out = S_in
    if S_out is None:
        S_out = torch.empty((N, Hv, dk, dv), dtype=torch.float32, device=q.device)
    if o is None:
        o = torch.empty((N, Hv, dv), dtype=q.dtype, device=q.device)
    code = lib.eda_fwd_recurrent_step_layer(
        _ptr(q, "q", q.dtype), _ptr(k, "k", q.dtype), _ptr(e, "e", q.dtype), _ptr(v, "v", q.dtype),
        _ptr(a, "a", q.dtype), _ptr(A_log, "A_log", torch.float32),
        _ptr(dt_bias, "dt_bias", torch.float32), _ptr(beta, "beta", torch.float32),
        _ptr(gamma, "gamma", torch.float32), _ptr(S_in, "S_in", torch.float32),
        _ptr(S_out, "S_out", torch.float32), _ptr(o, "o", q.dtype), N, Hk, Hv, dk, dv, dt,
        _stream(q.device))
    _check("eda_fwd_recurrent_step_layer", code)
    return o, S_out


def fwd_chunked_dplr(q, k, a, v, alpha, S0=None, *, chunk: int = 0, want_state: bool = True,
                     out: Optional[torch.Tensor] = None, S_final: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None):
    """Rank-1 DPLR (GDN-2 / QED) chunked forward (eda_fwd_chunked_dplr):
    q, k, a, alpha [B, T, H, d_k], v [B, T, H, d_v]; returns (o, S_final)."""
    lib = load_library()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    if S_final is None and want_state:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    need = int(lib.eda_fwd_chunked_workspace_size(B, T, H, dk, dv, dt, chunk))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    code = lib.eda_fwd_chunked_dplr(
        _ptr(q, "q", q.dtype), _ptr(k, "k", q.dtype), _ptr(a, "a", q.dtype), _ptr(v, "v", q.dtype),
        _ptr(alpha, "alpha", torch.float32), _ptr(S0, "S0", torch.float32), _ptr(out, "o", q.dtype),
        _ptr(S_final, "S_final", torch.float32), B, T, H, dk, dv, dt, chunk,
        _ptr(workspace, "workspace"), 0 if workspace is None else workspace.numel(), _stream(q.device))
    _check("eda_fwd_chunked_dplr", code)
    return out, S_final


def recurrent_step_dplr(q, k, a, v, alpha, S_in=None, *, S_out: Optional[torch.Tensor] = None,
                        o: Optional[torch.Tensor] = None, inplace: bool = False):
    """One DPLR decode token (eda_fwd_recurrent_step_dplr) for [N, H, d] inputs."""
    lib = load_library()
    N, H, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    if inplace:
        if S_in is None:
            raise ValueError("inplace=True needs S_in")
        S_out = S_in
    if S_out is None:
        S_out = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    code = lib.eda_fwd_recurrent_step_dplr(
        _ptr(q, "q", q.dtype), _ptr(k, "k", q.dtype), _ptr(a, "a", q.dtype), _ptr(v, "v", q.dtype),
        _ptr(alpha, "alpha", torch.float32), _ptr(S_in, "S_in", torch.float32),
        _ptr(S_out, "S_out", torch.float32), _ptr(o, "o", q.dtype), N, H, dk, dv, dt, _stream(q.device))
    _check("eda_fwd_recurrent_step_dplr", code)
    return o, S_out


def backward(q, k, e, v, alpha, beta, gamma, S0, dO, dS_final=None, *, want_dS0: bool = True,
             workspace: Optional[torch.Tensor] = None) -> dict:
    """Gradients of <o, dO> + <S_final, dS_final> (eda_bwd); returns a dict of
    float32 tensors dq, dk, de, dv, dalpha, dbeta, dgamma and dS0 (None when
    want_dS0 is False)."""
    lib = load_library()
    B, T, H, dk = q.shape
    dvd = v.shape[-1]
    dt = _dtype_code(q)
    f32 = dict(dtype=torch.float32, device=q.device)
    g = dict(dq=torch.empty((B, T, H, dk), **f32), dk=torch.empty((B, T, H, dk), **f32),
             de=torch.empty((B, T, H, dk), **f32), dv=torch.empty((B, T, H, dvd), **f32),
             dalpha=torch.empty((B, T, H, dk), **f32), dbeta=torch.empty((B, T, H), **f32),
             dgamma=torch.empty((B, T, H), **f32),
             dS0=torch.empty((B, H, dk, dvd), **f32) if want_dS0 else None)
    need = int(lib.eda_bwd_workspace_size(B, T, H, dk, dvd))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    code = lib.eda_bwd(
        _ptr(q, "q", q.dtype), _ptr(k, "k", q.dtype), _ptr(e, "e", q.dtype), _ptr(v, "v", q.dtype),
        _ptr(alpha, "alpha", torch.float32), _ptr(beta, "beta", torch.float32),
        _ptr(gamma, "gamma", torch.float32), _ptr(S0, "S0", torch.float32), _ptr(dO, "dO", q.dtype),
        _ptr(dS_final, "dS_final", torch.float32),
        *(_ptr(g[n], n, torch.float32) for n in ("dq", "dk", "de", "dv", "dalpha", "dbeta", "dgamma", "dS0")),
        B, T, H, dk, dvd, dt, _ptr(workspace, "workspace"), workspace.numel(), _stream(q.device))
    _check("eda_bwd", code)
    return g

