"""KDA oracle -- TEST INFRASTRUCTURE ONLY.

A plain fp64 token-by-token CPU evaluation of the KDA forward recurrence and
of its gradients (``kda_oracle.c``).  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the HIP product
path never does and shares no code with it.

The recurrence, its gate activations and the tensor contract follow the pages
this project is built from; ``kda_oracle.c`` cites the passages.  Every
function here is pinned: the forward by ``tests/test_oracle.py`` (closed forms,
invariants, library routines, an independent chunked formulation), the
gradients by ``tests/test_oracle_bwd.py`` (central finite differences of the
fp64 forward, and torch autograd of an independently written recurrence).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
# The mutation tests point this at a deliberately broken copy of the oracle.
_LIB_OVERRIDE = os.environ.get("KDA_ORACLE_LIB")

GATE_SOFTPLUS = 0
GATE_SAFE_SIGMOID = 1
GATE_PREGATED = 2
FLAG_QK_L2NORM = 1
FLAG_BETA_IS_PROB = 2

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP).  Returns the library path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def use_native_build() -> str:
    """For timing on the host that runs it: compile this same source with
    -O3 -march=native into a private temporary directory and use that library
    from now on (the shipped library stays portable, -O2 for any x86-64).
    Floating-point contraction stays off, so the arithmetic is the same.
    Returns the build description."""
    global _lib
    import tempfile
    flags = ["-O3", "-march=native", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c99"]
    d = tempfile.mkdtemp(prefix="kda_oracle_")
    path = os.path.join(d, "libkda_oracle_native.so")
    subprocess.check_call(["gcc", *flags, "-o", path, _SRC, "-lm"])
    global _LIB_OVERRIDE, _NATIVE
    _lib = None
    _LIB_OVERRIDE = path
    _load()
    _NATIVE = "gcc " + " ".join(flags)
    return _NATIVE


_NATIVE = None


def native_build_description() -> str:
    """How the library in use was built."""
    return _NATIVE or "gcc -O2 -fopenmp (shipped build)"


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.kda_oracle_fwd.restype = ctypes.c_int
        lib.kda_oracle_fwd.argtypes = ([ctypes.c_int] * 7 + [P] * 5 + [P, P, P] +
                                       [ctypes.c_double, ctypes.c_double, ctypes.c_int, ctypes.c_int] +
                                       [P, P, P, ctypes.c_int])
        lib.kda_oracle_gate.restype = None
        lib.kda_oracle_gate.argtypes = [ctypes.c_int, ctypes.c_int, P, ctypes.c_double,
                                        ctypes.c_double, P]
        lib.kda_oracle_l2norm.restype = None
        lib.kda_oracle_l2norm.argtypes = [ctypes.c_int, P, P]
        if hasattr(lib, "kda_oracle_bwd"):
            lib.kda_oracle_fwd_f64.restype = ctypes.c_int
            lib.kda_oracle_fwd_f64.argtypes = ([ctypes.c_int] * 7 + [P] * 5 + [P, P, P] +
                                               [ctypes.c_double, ctypes.c_double, ctypes.c_int, ctypes.c_int] +
                                               [P, P, P])
            lib.kda_oracle_bwd.restype = ctypes.c_int
            lib.kda_oracle_bwd.argtypes = ([ctypes.c_int] * 7 + [P] * 5 + [P, P, P] +
                                           [ctypes.c_double, ctypes.c_double, ctypes.c_int, ctypes.c_int] +
                                           [P, P, P] + [P] * 8 + [ctypes.c_int])
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a, name):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"{name}: expected bf16 bit patterns as uint16, got {a.dtype}")
    return a


def gate(mode: int, x, A_log: float = 0.0, lower_bound: float = -1.0) -> np.ndarray:
    """Gate activation on x = g + dt_bias (fp64)."""
    x = np.ascontiguousarray(x, dtype=np.float64).ravel()
    y = np.empty_like(x)
    _load().kda_oracle_gate(mode, x.size, _ptr(x), float(A_log), float(lower_bound), _ptr(y))
    return y


def l2norm(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64).ravel()
    y = np.empty_like(x)
    _load().kda_oracle_l2norm(x.size, _ptr(x), _ptr(y))
    return y


def fwd(q, k, v, g, beta, A_log, dt_bias, *, scale, lower_bound=-1.0,
        gate_mode=GATE_SOFTPLUS, flags=FLAG_QK_L2NORM, initial_state=None,
        cu_seqlens=None, want_out=True, want_state=True, nthreads=0):
    """Run the oracle.

    q, k : uint16 [B,T,Hqk,K]; v : uint16 [B,T,Hv,V]; g : uint16 [B,T,Hv,K];
    beta : uint16 [B,T,Hv] (bf16 bit patterns); A_log float32 [Hv] (or None);
    dt_bias float32 [Hv,K] (or None); initial_state float64-convertible
    [N,Hv,V,K] or None; cu_seqlens int64 [N+1] or None.
    Returns (out fp64 [B,T,Hv,V] or None, final_state fp64 [N,Hv,V,K] or None).
    """
    q, k, v, g, beta = (_u16(x, n) for x, n in ((q, "q"), (k, "k"), (v, "v"), (g, "g"), (beta, "beta")))
    B, T, Hqk, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    if k.shape != q.shape or g.shape != (B, T, Hv, K) or v.shape[:2] != (B, T) or beta.shape != (B, T, Hv):
        raise ValueError("oracle: inconsistent shapes")
    if cu_seqlens is not None:
        cu_seqlens = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
        N = cu_seqlens.size - 1
    else:
        N = B
    A_log = None if A_log is None else np.ascontiguousarray(A_log, dtype=np.float32)
    dt_bias = None if dt_bias is None else np.ascontiguousarray(dt_bias, dtype=np.float32)
    h0 = None if initial_state is None else np.ascontiguousarray(initial_state, dtype=np.float64)
    if h0 is not None and h0.shape != (N, Hv, V, K):
        raise ValueError("oracle: initial_state shape")
    out = np.empty((B, T, Hv, V), np.float64) if want_out else None
    hT = np.empty((N, Hv, V, K), np.float64) if want_state else None
    rc = _load().kda_oracle_fwd(B, T, Hqk, Hv, K, V, N, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                _ptr(A_log), _ptr(dt_bias), _ptr(cu_seqlens), float(scale),
                                float(lower_bound), int(gate_mode), int(flags), _ptr(h0), _ptr(hT),
                                _ptr(out), int(nthreads))
    if rc != 0:
        raise ValueError("oracle: argument error")
    return out, hT


def bf16_to_f64(a) -> np.ndarray:
    """bf16 bit patterns (uint16) -> their exact float64 values."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _f64(a, name):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a


def _shapes(q, v, g, beta, cu_seqlens):
    B, T, Hqk, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    if g.shape != (B, T, Hv, K) or v.shape[:2] != (B, T) or beta.shape != (B, T, Hv):
        raise ValueError("oracle: inconsistent shapes")
    N = B if cu_seqlens is None else np.asarray(cu_seqlens).size - 1
    return B, T, Hqk, Hv, K, V, N


def fwd_f64(q, k, v, g, beta, A_log, dt_bias, *, scale, lower_bound=-1.0, gate_mode=GATE_SOFTPLUS,
            flags=FLAG_QK_L2NORM, initial_state=None, cu_seqlens=None):
    """The forward on float64 inputs (same layouts as ``fwd``).  Returns (out, final_state)."""
    q, k, v, g, beta = (_f64(x, n) for x, n in ((q, "q"), (k, "k"), (v, "v"), (g, "g"), (beta, "beta")))
    B, T, Hqk, Hv, K, V, N = _shapes(q, v, g, beta, cu_seqlens)
    cu = None if cu_seqlens is None else np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    A_log = None if A_log is None else np.ascontiguousarray(A_log, dtype=np.float32)
    dt_bias = None if dt_bias is None else np.ascontiguousarray(dt_bias, dtype=np.float32)
    h0 = None if initial_state is None else np.ascontiguousarray(initial_state, dtype=np.float64)
    out = np.empty((B, T, Hv, V), np.float64)
    hT = np.empty((N, Hv, V, K), np.float64)
    rc = _load().kda_oracle_fwd_f64(B, T, Hqk, Hv, K, V, N, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                    _ptr(A_log), _ptr(dt_bias), _ptr(cu), float(scale), float(lower_bound),
                                    int(gate_mode), int(flags), _ptr(h0), _ptr(hT), _ptr(out))
    if rc != 0:
        raise ValueError("oracle: argument error")
    return out, hT


def bwd(q, k, v, g, beta, A_log, dt_bias, d_out, d_final_state=None, *, scale, lower_bound=-1.0,
        gate_mode=GATE_SOFTPLUS, flags=FLAG_QK_L2NORM, initial_state=None, cu_seqlens=None, nthreads=0):
    """Gradients of the forward (float64 inputs; bf16 inputs go through
    ``bf16_to_f64`` first).  d_out [B,T,Hv,V]; d_final_state [N,Hv,V,K] or None.
    Returns a dict: dq, dk [B,T,Hqk,K], dv [B,T,Hv,V], dg [B,T,Hv,K],
    dbeta [B,T,Hv], dA_log [Hv], ddt_bias [Hv,K], dh0 [N,Hv,V,K]."""
    q, k, v, g, beta = (_f64(x, n) for x, n in ((q, "q"), (k, "k"), (v, "v"), (g, "g"), (beta, "beta")))
    B, T, Hqk, Hv, K, V, N = _shapes(q, v, g, beta, cu_seqlens)
    cu = None if cu_seqlens is None else np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    A_log = None if A_log is None else np.ascontiguousarray(A_log, dtype=np.float32)
    dt_bias = None if dt_bias is None else np.ascontiguousarray(dt_bias, dtype=np.float32)
    h0 = None if initial_state is None else np.ascontiguousarray(initial_state, dtype=np.float64)
    do_ = np.ascontiguousarray(d_out, dtype=np.float64)
    dhT = None if d_final_state is None else np.ascontiguousarray(d_final_state, dtype=np.float64)
    r = dict(dq=np.empty((B, T, Hqk, K)), dk=np.empty((B, T, Hqk, K)), dv=np.empty((B, T, Hv, V)),
             dg=np.empty((B, T, Hv, K)), dbeta=np.empty((B, T, Hv)), dA_log=np.empty(Hv),
             ddt_bias=np.empty((Hv, K)), dh0=np.empty((N, Hv, V, K)))
    rc = _load().kda_oracle_bwd(B, T, Hqk, Hv, K, V, N, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                _ptr(A_log), _ptr(dt_bias), _ptr(cu), float(scale), float(lower_bound),
                                int(gate_mode), int(flags), _ptr(h0), _ptr(do_), _ptr(dhT),
                                _ptr(r["dq"]), _ptr(r["dk"]), _ptr(r["dv"]), _ptr(r["dg"]), _ptr(r["dbeta"]),
                                _ptr(r["dA_log"]), _ptr(r["ddt_bias"]), _ptr(r["dh0"]), int(nthreads))
    if rc != 0:
        raise ValueError("oracle: argument error")
    return r
