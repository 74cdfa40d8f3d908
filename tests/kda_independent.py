"""Independent fp64 formulations used to pin the oracle (CPU tests only).

Nothing here is shared with the oracle's C code: the gate activations,
normalisation and both recurrences are written again, differently, in numpy.

* ``chunked_fwd`` is the chunked WY/UT form of the same recurrence (64-token
  chunks, intra-chunk Akk/Aqk, T = (I + Akk)^-1, w/u factors, inter-chunk state
  carry) -- the decomposition the pages' kernels are organised around (fla-kda
  SKILL.md, "Code map" and "Numerical invariants").  It reaches the token
  recurrence's result exactly up to rounding, so agreement to ~1e-12 pins the
  oracle's order of operations, orientation and gating.
* ``matrix_form_fwd`` evaluates S_t = S_{t-1} Diag(e^{a_t}) (I - b_t k_t k_t^T)
  + b_t v_t k_t^T as an explicit product of matrices.
"""
from __future__ import annotations

import numpy as np
from scipy.special import expit


def widen_bf16(bits):
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def activation(mode, x, A_log, lb):
    if mode == 0:      # -exp(A_log) * softplus(x)
        return -np.exp(A_log) * np.logaddexp(0.0, x)
    if mode == 1:      # lb * sigmoid(exp(A_log) x)
        return lb * expit(np.exp(A_log) * x)
    return x           # pre-gated log-decay


def normalise_rows(x, on=True):
    if not on:
        return x
    return x / np.sqrt(np.einsum("...i,...i->...", x, x) + 1e-6)[..., None]


def _pairs(inp_like):
    B, T = inp_like["q"].shape[:2]
    cu = inp_like.get("cu_seqlens")
    if cu is None:
        return [(b, b, 0, T) for b in range(B)]
    return [(n, 0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]


def _prep(d, b, bos, eos, h, hq):
    q = widen_bf16(d["q"][b, bos:eos, hq])
    k = widen_bf16(d["k"][b, bos:eos, hq])
    v = widen_bf16(d["v"][b, bos:eos, h])
    g = widen_bf16(d["g"][b, bos:eos, h])
    bl = widen_bf16(d["beta"][b, bos:eos, h])
    x = g + (0.0 if d.get("dt_bias") is None else d["dt_bias"][h].astype(np.float64))
    A = 0.0 if d.get("A_log") is None else float(d["A_log"][h])
    a = activation(d["gate_mode"], x, A, d["lower_bound"])
    beta = bl if d.get("beta_is_prob") else expit(bl)
    on = d.get("l2norm", True)
    return normalise_rows(q, on), normalise_rows(k, on), v, a, beta


def chunked_fwd(d, chunk=64):
    """d: dict with q,k,v,g,beta (uint16), A_log, dt_bias, gate_mode, lower_bound,
    scale, optional cu_seqlens, h0 (fp64 [N,Hv,V,K]), beta_is_prob, l2norm."""
    B, T, Hqk, K = d["q"].shape
    Hv, V = d["v"].shape[2:]
    G = Hv // Hqk
    pairs = _pairs(d)
    out = np.zeros((B, T, Hv, V))
    hT = np.zeros((len(pairs), Hv, V, K))
    for n, b, bos, eos in pairs:
        for h in range(Hv):
            q, k, v, a, beta = _prep(d, b, bos, eos, h, h // G)
            S = np.zeros((V, K)) if d.get("h0") is None else d["h0"][n, h].copy()
            for c0 in range(0, eos - bos, chunk):
                c1 = min(c0 + chunk, eos - bos)
                Q, Kc, Vc, bc = q[c0:c1], k[c0:c1], v[c0:c1], beta[c0:c1]
                Gm = np.cumsum(a[c0:c1], axis=0)
                L = c1 - c0
                D = Gm[:, None, :] - Gm[None, :, :]          # Gamma_i - Gamma_j
                low = np.tril(np.ones((L, L), bool))
                E = np.where(low[:, :, None], np.exp(np.where(low[:, :, None], D, 0.0)), 0.0)
                Akk = np.einsum("ic,jc,ijc->ij", Kc, Kc, E) * bc[:, None]
                Akk = np.tril(Akk, -1)
                Aqk = np.einsum("ic,jc,ijc->ij", Q, Kc, E)
                Tm = np.linalg.inv(np.eye(L) + Akk)
                W = Tm @ (bc[:, None] * Kc * np.exp(Gm))
                Ub = Tm @ (bc[:, None] * Vc)
                U = Ub - W @ S.T
                out[b, bos + c0:bos + c1, h] = d["scale"] * ((Q * np.exp(Gm)) @ S.T + Aqk @ U)
                S = S * np.exp(Gm[-1])[None, :] + U.T @ (Kc * np.exp(Gm[-1][None, :] - Gm))
            hT[n, h] = S
    return out, hT


def matrix_form_fwd(d):
    """Token loop in the product form S_t = S_{t-1} Diag(e^a)(I - b k k^T) + b v k^T."""
    B, T, Hqk, K = d["q"].shape
    Hv, V = d["v"].shape[2:]
    G = Hv // Hqk
    pairs = _pairs(d)
    out = np.zeros((B, T, Hv, V))
    hT = np.zeros((len(pairs), Hv, V, K))
    I = np.eye(K)
    for n, b, bos, eos in pairs:
        for h in range(Hv):
            q, k, v, a, beta = _prep(d, b, bos, eos, h, h // G)
            S = np.zeros((V, K)) if d.get("h0") is None else d["h0"][n, h].copy()
            for t in range(eos - bos):
                M = np.diag(np.exp(a[t])) @ (I - beta[t] * np.outer(k[t], k[t]))
                S = S @ M + beta[t] * np.outer(v[t], k[t])
                out[b, bos + t, h] = d["scale"] * (S @ q[t])
            hT[n, h] = S
    return out, hT
