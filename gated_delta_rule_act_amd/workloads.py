"""Seeded synthetic KDA inputs.

This module only draws random numbers and rounds them to the storage dtypes;
it holds none of the KDA arithmetic, so both the HIP path and the CPU oracle
can be fed from it without sharing any of the method.

Workloads mirror the pages' call contract ("FlashKDA Delta Attention" page,
"Tensor shapes and dtypes" table): q, k, g [B,T,H,128] bf16, v [B,T,H,128]
bf16, beta [B,T,H] bf16 logits, A_log [H] fp32, dt_bias [H,K] fp32, optional
initial state [N,H,V,K], optional int64 cu_seqlens.  The named workloads are
the five shapes and distributions this project is measured on; the second
parameter of N(., .) is a standard deviation.  Draw order is fixed: lengths
(packed workload only), q, k, v, g, beta, A_log, dt_bias, initial state, each
drawn in fp32 from numpy's PCG64 and rounded to bf16 with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

GATE_SOFTPLUS = 0
GATE_SAFE_SIGMOID = 1
GATE_PREGATED = 2

FLAG_QK_L2NORM = 1
FLAG_BETA_IS_PROB = 2

STATE_NONE = 0
STATE_F32 = 1
STATE_BF16 = 2


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class KdaInputs:
    """Host copies of one call's inputs (bf16 tensors as uint16 bit patterns)."""
    q: np.ndarray            # [B,T,Hqk,K] uint16
    k: np.ndarray            # [B,T,Hqk,K] uint16
    v: np.ndarray            # [B,T,Hv,V]  uint16
    g: np.ndarray            # [B,T,Hv,K]  uint16
    beta: np.ndarray         # [B,T,Hv]    uint16
    A_log: Optional[np.ndarray]    # [Hv] float32, or None
    dt_bias: Optional[np.ndarray]  # [Hv,K] float32, or None
    scale: float
    lower_bound: float
    gate_mode: int
    cu_seqlens: Optional[np.ndarray] = None      # [N+1] int64
    initial_state: Optional[np.ndarray] = None   # [N,Hv,V,K] float32 or uint16 (bf16)
    init_state_dtype: int = STATE_NONE
    final_state_dtype: int = STATE_F32
    flags: int = FLAG_QK_L2NORM
    name: str = "custom"

    @property
    def B(self): return self.q.shape[0]
    @property
    def T(self): return self.q.shape[1]
    @property
    def Hqk(self): return self.q.shape[2]
    @property
    def Hv(self): return self.v.shape[2]
    @property
    def K(self): return self.q.shape[3]
    @property
    def V(self): return self.v.shape[3]
    @property
    def N(self): return self.B if self.cu_seqlens is None else self.cu_seqlens.size - 1

    def initial_state_f64(self) -> Optional[np.ndarray]:
        """The initial state exactly as stored, widened to fp64."""
        if self.initial_state is None:
            return None
        if self.init_state_dtype == STATE_BF16:
            return bf16_bits_to_f32(self.initial_state).astype(np.float64)
        return self.initial_state.astype(np.float64)


def _normal_bf16(rng, shape, std=1.0, mean=0.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return f32_to_bf16_bits(x)


def make_inputs(*, B, T, Hqk, Hv=None, K=128, V=128, gate_mode=GATE_SOFTPLUS, lower_bound=-1.0,
                seed=0, g_std=1.0, A_log_range=(0.0, math.log(16.0)), dt_bias_std=0.1,
                lengths=None, init_state_dtype=STATE_NONE, final_state_dtype=STATE_F32,
                h0_std=0.05, scale=None, name="custom", rng=None, qk_std=1.0, pregated_range=(-1.0, 0.0),
                beta_prob=False, with_A_log=True, with_dt_bias=True, flags=FLAG_QK_L2NORM) -> KdaInputs:
    """Draw one seeded input set.  With ``lengths`` the sequences are packed
    (B must be 1 and T is their sum) and int64 cu_seqlens is returned.  A
    generator passed as ``rng`` is used as is (``seed`` is then ignored).

    Contract variants keep the draw order: with ``gate_mode`` pre-gated, g is
    drawn U(pregated_range) as the log-space decay itself; ``beta_prob`` draws
    beta U(0, 1) as probabilities; ``qk_std`` scales q and k (for runs without
    the L2 norm); A_log and dt_bias are still drawn when ``with_A_log`` /
    ``with_dt_bias`` is false, then dropped."""
    Hv = Hqk if Hv is None else Hv
    rng = np.random.default_rng(seed) if rng is None else rng
    cu = None
    if lengths is not None:
        if B != 1:
            raise ValueError("packed sequences need B == 1")
        lengths = np.asarray(lengths, dtype=np.int64)
        cu = np.zeros(lengths.size + 1, np.int64)
        cu[1:] = np.cumsum(lengths)
        T = int(cu[-1])
    q = _normal_bf16(rng, (B, T, Hqk, K), std=qk_std)
    k = _normal_bf16(rng, (B, T, Hqk, K), std=qk_std)
    v = _normal_bf16(rng, (B, T, Hv, V))
    if gate_mode == GATE_PREGATED:
        lo, hi = pregated_range
        g = f32_to_bf16_bits(rng.uniform(lo, hi, size=(B, T, Hv, K)).astype(np.float32))
    else:
        g = _normal_bf16(rng, (B, T, Hv, K), std=g_std)
    if beta_prob:
        beta = f32_to_bf16_bits(rng.uniform(0.0, 1.0, size=(B, T, Hv)).astype(np.float32))
    else:
        beta = _normal_bf16(rng, (B, T, Hv))
    A_log = rng.uniform(A_log_range[0], A_log_range[1], size=Hv).astype(np.float32)
    dt_bias = (rng.standard_normal(size=(Hv, K), dtype=np.float32) * np.float32(dt_bias_std)).astype(np.float32)
    N = B if cu is None else cu.size - 1
    h0 = None
    if init_state_dtype != STATE_NONE:
        x = rng.standard_normal(size=(N, Hv, V, K), dtype=np.float32) * np.float32(h0_std)
        h0 = f32_to_bf16_bits(x) if init_state_dtype == STATE_BF16 else x.astype(np.float32)
    if not with_A_log or gate_mode == GATE_PREGATED:
        A_log = None
    if not with_dt_bias or gate_mode == GATE_PREGATED:
        dt_bias = None
    if beta_prob:
        flags |= FLAG_BETA_IS_PROB
    return KdaInputs(q=q, k=k, v=v, g=g, beta=beta, A_log=A_log, dt_bias=dt_bias, flags=flags,
                     scale=(1.0 / math.sqrt(K)) if scale is None else float(scale),
                     lower_bound=float(lower_bound), gate_mode=gate_mode, cu_seqlens=cu,
                     initial_state=h0, init_state_dtype=init_state_dtype,
                     final_state_dtype=final_state_dtype, name=name)


# The five measured workloads (index = seed).
WORKLOADS = {
    1: dict(name="tiny_b1_t256_h2", B=1, T=256, Hqk=2, gate_mode=GATE_SOFTPLUS),
    2: dict(name="dense_b4_t4096_h16", B=4, T=4096, Hqk=16, gate_mode=GATE_SOFTPLUS),
    3: dict(name="safe_b2_t8192_h32_lb-5", B=2, T=8192, Hqk=32, gate_mode=GATE_SAFE_SIGMOID,
            lower_bound=-5.0, A_log_range=(-4.0, 6.0), g_std=3.0, init_state_dtype=STATE_F32),
    4: dict(name="varlen_n16_h32", B=1, T=None, Hqk=32, gate_mode=GATE_SOFTPLUS,
            init_state_dtype=STATE_BF16, final_state_dtype=STATE_BF16, packed=16),
    5: dict(name="gva_t131072_hqk16_hv32_lb-1", B=1, T=131072, Hqk=16, Hv=32,
            gate_mode=GATE_SAFE_SIGMOID, lower_bound=-1.0),
    # one GPU's share of workload 5 when its 32 v-heads are split over 8 GPUs
    # (2 qk-heads with their 4 v-heads): few (sequence, head) chains, each of
    # 2,048 chunks -- the case time segments of the state chain are for
    6: dict(name="gva_share_t131072_hqk2_hv4_lb-1", B=1, T=131072, Hqk=2, Hv=4,
            gate_mode=GATE_SAFE_SIGMOID, lower_bound=-1.0),
}


# Token-recurrent (decode) workloads: one decode step, and a short-sequence
# batch, with the distributions of the safe-gate workload and fp32 state.
RECURRENT_WORKLOADS = {
    1: dict(name="decode_b64_t1_h32_lb-5", B=64, T=1, Hqk=32, gate_mode=GATE_SAFE_SIGMOID, lower_bound=-5.0,
            A_log_range=(-4.0, 6.0), g_std=3.0, init_state_dtype=STATE_F32),
    2: dict(name="short_b16_t64_h32_lb-5", B=16, T=64, Hqk=32, gate_mode=GATE_SAFE_SIGMOID, lower_bound=-5.0,
            A_log_range=(-4.0, 6.0), g_std=3.0, init_state_dtype=STATE_F32),
}


def recurrent_workload(idx: int) -> KdaInputs:
    """Draw token-recurrent workload ``idx`` (1..2) with seed = 100 + idx."""
    return make_inputs(seed=100 + idx, **RECURRENT_WORKLOADS[idx])


def workload(idx: int, **override) -> KdaInputs:
    """Draw measured workload ``idx`` (1..6) with seed = idx."""
    spec = dict(WORKLOADS[idx])
    spec.update(override)
    packed = spec.pop("packed", None)
    seed = spec.pop("seed", idx)
    rng = np.random.default_rng(seed)
    if packed:
        # lengths come first in the draw order, from the same stream
        lengths = rng.integers(64, 8192 + 1, size=packed, dtype=np.int64)
        spec["lengths"] = lengths
        spec["T"] = int(lengths.sum())
    return make_inputs(rng=rng, **spec)


def make_grads(inp: KdaInputs, seed: int, d_out_std: float = 0.1, dhT_std: Optional[float] = 0.01):
    """Seeded upstream gradients for a backward run on ``inp``: d_out as bf16
    bits [B,T,Hv,V] and d_final_state fp32 [N,Hv,V,K] (None if dhT_std is None)."""
    rng = np.random.default_rng(seed)
    d_out = _normal_bf16(rng, (inp.B, inp.T, inp.Hv, inp.V), std=d_out_std)
    dhT = None
    if dhT_std is not None:
        dhT = (rng.standard_normal(size=(inp.N, inp.Hv, inp.V, inp.K), dtype=np.float32) * np.float32(dhT_std))
    return d_out, dhT
