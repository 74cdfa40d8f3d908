"""Python binding of libkda.so (argument marshalling only).

Every step of the forward runs in the HIP kernels behind the C ABI
(include/kda.h); this module only checks Python-level types, allocates the
caller-owned outputs and workspace with torch, and passes raw device
pointers plus the current HIP stream.  If the library is not built the calls
raise: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")

KDA_OK = 0
KDA_ERR_WORKSPACE = -6
GATE_SOFTPLUS = 0
GATE_SAFE_SIGMOID = 1
GATE_PREGATED = 2
STATE_NONE = 0
STATE_F32 = 1
STATE_BF16 = 2
FLAG_QK_L2NORM = 1
FLAG_BETA_IS_PROB = 2

_STATUS = {0: "KDA_OK", -1: "KDA_ERR_NULL", -2: "KDA_ERR_SHAPE", -3: "KDA_ERR_DTYPE", -4: "KDA_ERR_RANGE",
           -5: "KDA_ERR_ALIGN", -6: "KDA_ERR_WORKSPACE", -7: "KDA_ERR_LAUNCH", -8: "KDA_ERR_UNSUPPORTED"}

# Every function the header declares.
EXPORTS = ("kda_fwd_workspace_size", "kda_fwd_segments", "kda_fwd_check", "kda_fwd", "kda_fwd_intra", "kda_fwd_state",
           "kda_fwd_noalloc", "kda_fused_recurrent_fwd", "kda_bwd_workspace_size", "kda_bwd", "kda_status_string",
           "kda_last_error")


class KdaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


class Params(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H_qk", ctypes.c_int32), ("H_v", ctypes.c_int32),
                ("K", ctypes.c_int32), ("V", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
                ("scale", ctypes.c_float), ("lower_bound", ctypes.c_float), ("gate_mode", ctypes.c_int32),
                ("init_state_dtype", ctypes.c_int32), ("final_state_dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("segments", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libkda.so not built at {path}; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    PP = ctypes.POINTER(Params)
    lib.kda_fwd_workspace_size.restype = ctypes.c_size_t
    lib.kda_fwd_workspace_size.argtypes = [PP]
    lib.kda_fwd_segments.restype = ctypes.c_int
    lib.kda_fwd_segments.argtypes = [PP, ctypes.c_int]
    lib.kda_fwd_check.restype = ctypes.c_int
    lib.kda_fwd_check.argtypes = [PP] + [P] * 12 + [ctypes.c_size_t]
    for fn in (lib.kda_fwd, lib.kda_fwd_intra, lib.kda_fwd_state):
        fn.restype = ctypes.c_int
        fn.argtypes = [PP] + [P] * 12 + [ctypes.c_size_t, P]
    for fn in (lib.kda_fused_recurrent_fwd, lib.kda_fwd_noalloc):
        fn.restype = ctypes.c_int
        fn.argtypes = [PP] + [P] * 11 + [P]
    lib.kda_bwd_workspace_size.restype = ctypes.c_size_t
    lib.kda_bwd_workspace_size.argtypes = [PP]
    lib.kda_bwd.restype = ctypes.c_int
    lib.kda_bwd.argtypes = [PP] + [P] * 20 + [ctypes.c_size_t, P]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_last_error.argtypes = []
    _lib = lib
    return lib


def make_params(*, B, T, H_qk, H_v, K=128, V=128, num_seqs=None, scale, lower_bound=-1.0,
                gate_mode=GATE_SOFTPLUS, init_state_dtype=STATE_NONE, final_state_dtype=STATE_F32,
                flags=FLAG_QK_L2NORM, segments=0) -> Params:
    return Params(B, T, H_qk, H_v, K, V, B if num_seqs is None else num_seqs, scale, lower_bound, gate_mode,
                  init_state_dtype, final_state_dtype, flags, segments)


def workspace_size(p: Params) -> int:
    return int(load_library().kda_fwd_workspace_size(ctypes.byref(p)))


def segments_of(p: Params, packed: bool = False) -> int:
    """Time segments per state chain kda_fwd uses for these parameters (0 if invalid)."""
    return int(load_library().kda_fwd_segments(ctypes.byref(p), int(packed)))


def last_error() -> str:
    return load_library().kda_last_error().decode()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


_ws_cache: dict = {}


def _workspace(nbytes: int, device) -> torch.Tensor:
    key = (device, torch.cuda.current_stream(device).cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def _state_code(t: Optional[torch.Tensor]) -> int:
    if t is None:
        return STATE_NONE
    if t.dtype == torch.float32:
        return STATE_F32
    if t.dtype == torch.bfloat16:
        return STATE_BF16
    raise TypeError(f"state tensors must be float32 or bfloat16, got {t.dtype}")


def fwd(q, k, v, g, beta, A_log, dt_bias, scale, lower_bound=-1.0, gate_mode=GATE_SOFTPLUS,
        initial_state=None, final_state_dtype=torch.float32, cu_seqlens=None, out=None,
        final_state=None, workspace=None, stage=None, qk_l2norm=True, beta_is_prob=False, recurrent=False,
        segments=0, noalloc=False):
    """Chunked KDA forward on the current HIP stream.

    q, k [B,T,Hqk,128] bf16; v, g [B,T,Hv,128] bf16; beta [B,T,Hv] bf16 logits
    (probabilities with ``beta_is_prob``); A_log [Hv] fp32 or None (required
    by the softplus gate; None means a multiplier of one for the safe gate);
    dt_bias [Hv,128] fp32 or None (zero bias; must be None with pre-gated g,
    where g is the log-space decay); initial_state [N,Hv,128,128] fp32/bf16
    or None; cu_seqlens [N+1] int64 or None (then B must be 1).
    Returns (out bf16 [B,T,Hv,128], final_state or None).  ``stage`` = "intra"
    or "state" runs only that half of the forward (kda_fwd_intra /
    kda_fwd_state); the two halves in order are the full forward.
    ``recurrent`` runs the token-recurrent entry (kda_fused_recurrent_fwd)
    instead: no workspace.  ``noalloc`` runs kda_fwd_noalloc: the chunked
    forward on the library's own device array, no workspace (``out`` and
    ``final_state`` should then be passed in, as that entry is for callers
    that allocate nothing).  ``final_state`` may be ``initial_state`` in both
    entries.  ``segments`` splits each state chain of dense input into that
    many parallel time segments (0: the library decides, 1: never).
    """
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous bf16 device tensor")
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or t.device != q.device):
            raise TypeError(f"{name} must be a contiguous fp32 tensor on the same device")
    B, T, Hqk, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    if k.shape != q.shape or g.shape != (B, T, Hv, K) or tuple(v.shape[:2]) != (B, T) or \
            beta.shape != (B, T, Hv) or (A_log is not None and A_log.shape != (Hv,)) or \
            (dt_bias is not None and dt_bias.shape != (Hv, K)):
        raise ValueError("inconsistent tensor shapes")
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int64 or cu_seqlens.device != q.device or not cu_seqlens.is_contiguous():
            raise TypeError("cu_seqlens must be a contiguous int64 tensor on the same device")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if initial_state is not None and (not initial_state.is_contiguous() or tuple(initial_state.shape) != (N, Hv, V, K)):
        raise ValueError("initial_state must be contiguous [N, Hv, V, K]")
    if out is None:
        out = torch.empty((B, T, Hv, V), dtype=torch.bfloat16, device=q.device)
    if final_state is None and final_state_dtype is not None:
        final_state = torch.empty((N, Hv, V, K), dtype=final_state_dtype, device=q.device)
    p = make_params(B=B, T=T, H_qk=Hqk, H_v=Hv, K=K, V=V, num_seqs=N, scale=float(scale),
                    lower_bound=float(lower_bound), gate_mode=int(gate_mode),
                    init_state_dtype=_state_code(initial_state), final_state_dtype=_state_code(final_state),
                    flags=(FLAG_QK_L2NORM if qk_l2norm else 0) | (FLAG_BETA_IS_PROB if beta_is_prob else 0),
                    segments=int(segments))
    stream = torch.cuda.current_stream(q.device).cuda_stream
    if recurrent or noalloc:
        if stage is not None or workspace is not None or (recurrent and noalloc):
            raise ValueError("the recurrent and allocation-free entries have no stages and no workspace")
        fn = lib.kda_fused_recurrent_fwd if recurrent else lib.kda_fwd_noalloc
        rc = fn(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A_log), _ptr(dt_bias),
                _ptr(cu_seqlens), _ptr(initial_state), _ptr(final_state), _ptr(out), ctypes.c_void_p(stream))
        if rc != KDA_OK:
            raise KdaError(rc, lib.kda_last_error().decode())
        return out, final_state
    need = int(lib.kda_fwd_workspace_size(ctypes.byref(p)))
    if workspace is None:
        workspace = _workspace(need, q.device)
    entry = {None: lib.kda_fwd, "intra": lib.kda_fwd_intra, "state": lib.kda_fwd_state}[stage]
    rc = entry(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A_log), _ptr(dt_bias),
                     _ptr(cu_seqlens), _ptr(initial_state), _ptr(final_state), _ptr(out), _ptr(workspace),
                     ctypes.c_size_t(workspace.numel()), ctypes.c_void_p(stream))
    if rc != KDA_OK:
        raise KdaError(rc, lib.kda_last_error().decode())
    return out, final_state


def bwd(q, k, v, g, beta, A_log, dt_bias, scale, d_out, lower_bound=-1.0, gate_mode=GATE_SOFTPLUS,
        initial_state=None, d_final_state=None, cu_seqlens=None, qk_l2norm=True, beta_is_prob=False,
        workspace=None, segments=0):
    """Gradients of ``fwd`` (kda_bwd) on the current HIP stream.

    Inputs as for ``fwd`` plus d_out bf16 [B,T,Hv,128] and d_final_state fp32
    [N,Hv,128,128] or None.  Returns a dict of fp32 tensors: dq, dk
    [B,T,Hqk,128], dv, dg [B,T,Hv,128], dbeta [B,T,Hv], dA_log [Hv] (None
    without A_log or with pre-gated decay), ddt_bias [Hv,128] (None with
    pre-gated decay) and dh0 [N,Hv,128,128].  ``segments`` as for ``fwd``:
    both state passes of dense input split their chains into that many
    parallel time segments (0: the library decides, 1: never).
    """
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("d_out", d_out)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous bf16 device tensor")
    B, T, Hqk, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    if d_out.shape != (B, T, Hv, V):
        raise ValueError("d_out must be [B, T, Hv, V]")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if d_final_state is not None and (d_final_state.dtype != torch.float32 or not d_final_state.is_contiguous()
                                      or tuple(d_final_state.shape) != (N, Hv, V, K)):
        raise ValueError("d_final_state must be contiguous fp32 [N, Hv, V, K]")
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    r = dict(dq=torch.empty((B, T, Hqk, K), **f32), dk=torch.empty((B, T, Hqk, K), **f32),
             dv=torch.empty((B, T, Hv, V), **f32), dg=torch.empty((B, T, Hv, K), **f32),
             dbeta=torch.empty((B, T, Hv), **f32), dh0=torch.empty((N, Hv, V, K), **f32),
             dA_log=None if (A_log is None or gate_mode == GATE_PREGATED) else torch.empty((Hv,), **f32),
             ddt_bias=None if gate_mode == GATE_PREGATED else torch.empty((Hv, K), **f32))
    p = make_params(B=B, T=T, H_qk=Hqk, H_v=Hv, K=K, V=V, num_seqs=N, scale=float(scale),
                    lower_bound=float(lower_bound), gate_mode=int(gate_mode),
                    init_state_dtype=_state_code(initial_state), final_state_dtype=STATE_NONE,
                    flags=(FLAG_QK_L2NORM if qk_l2norm else 0) | (FLAG_BETA_IS_PROB if beta_is_prob else 0),
                    segments=int(segments))
    need = int(lib.kda_bwd_workspace_size(ctypes.byref(p)))
    if workspace is None:
        workspace = _workspace(need, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.kda_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A_log), _ptr(dt_bias),
                     _ptr(cu_seqlens), _ptr(initial_state), _ptr(d_out), _ptr(d_final_state), _ptr(r["dq"]),
                     _ptr(r["dk"]), _ptr(r["dv"]), _ptr(r["dg"]), _ptr(r["dbeta"]), _ptr(r["dA_log"]),
                     _ptr(r["ddt_bias"]), _ptr(r["dh0"]), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
                     ctypes.c_void_p(stream))
    if rc != KDA_OK:
        raise KdaError(rc, lib.kda_last_error().decode())
    return r
