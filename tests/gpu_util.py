"""Helpers shared by the GPU tests: move seeded inputs to the device, run the
HIP path through the C ABI binding, run the oracle on the same inputs, and
measure errors with the tolerances the parity bar fixes."""
from __future__ import annotations

import concurrent.futures as cf
import sys

import numpy as np
import torch

import oracle
from gated_delta_rule_act_amd import kda
from gated_delta_rule_act_amd import workloads as W

# Parity bar: max |out_gpu - out_ref| <= 2e-2 on the bf16 outputs and
# ||S_gpu - S_ref||_F / ||S_ref||_F <= 1e-3 on an fp32 final state; a bf16
# final state is a bf16 output (max-abs 2e-2).  The relative RMS of the
# outputs is held to 1e-2 as well, since outputs are only ~0.05 in size.
OUT_MAX_ABS = 2e-2
STATE_REL = 1e-3
OUT_REL_RMS = 1e-2


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_dev(a: np.ndarray, dev="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def to_device(inp: W.KdaInputs, dev="cuda"):
    d = dict(q=bf16_dev(inp.q, dev), k=bf16_dev(inp.k, dev), v=bf16_dev(inp.v, dev), g=bf16_dev(inp.g, dev),
             beta=bf16_dev(inp.beta, dev),
             A_log=None if inp.A_log is None else torch.from_numpy(inp.A_log).to(dev),
             dt_bias=None if inp.dt_bias is None else torch.from_numpy(inp.dt_bias).to(dev))
    d["cu_seqlens"] = None if inp.cu_seqlens is None else torch.from_numpy(inp.cu_seqlens).to(dev)
    if inp.initial_state is None:
        d["h0"] = None
    elif inp.init_state_dtype == W.STATE_BF16:
        d["h0"] = bf16_dev(inp.initial_state, dev)
    else:
        d["h0"] = torch.from_numpy(inp.initial_state).to(dev)
    return d


def final_dtype_of(inp):
    return {W.STATE_NONE: None, W.STATE_F32: torch.float32, W.STATE_BF16: torch.bfloat16}[inp.final_state_dtype]


def run_gpu(inp: W.KdaInputs, dev_inputs=None, poison=True, segments=0, final_state=None, initial_state=None):
    d = dev_inputs or to_device(inp)
    B, T, Hv, V = inp.B, inp.T, inp.Hv, inp.V
    out = torch.empty((B, T, Hv, V), dtype=torch.bfloat16, device="cuda")
    fs = final_state
    fdt = final_dtype_of(inp)
    if fs is None and fdt is not None:
        fs = torch.empty((inp.N, Hv, V, inp.K), dtype=fdt, device="cuda")
        if poison:
            fs.fill_(float("nan"))
    if poison:
        out.fill_(float("nan"))
    h0 = d["h0"] if initial_state is None else initial_state
    o, s = kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"], d["dt_bias"], inp.scale,
                   inp.lower_bound, inp.gate_mode, initial_state=h0, cu_seqlens=d["cu_seqlens"],
                   out=out, final_state=fs, final_state_dtype=fdt,
                   qk_l2norm=bool(inp.flags & W.FLAG_QK_L2NORM), beta_is_prob=bool(inp.flags & W.FLAG_BETA_IS_PROB),
                   segments=segments)
    torch.cuda.synchronize()
    return o, s


def run_oracle(inp: W.KdaInputs, nthreads=0):
    return oracle.fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.A_log, inp.dt_bias, scale=inp.scale,
                      lower_bound=inp.lower_bound, gate_mode=inp.gate_mode, flags=inp.flags,
                      initial_state=inp.initial_state_f64(), cu_seqlens=inp.cu_seqlens, nthreads=nthreads)


def oracle_pair(inp: W.KdaInputs, n: int, h: int, h0_f64=None):
    """Oracle for one (sequence, v-head) pair on sliced inputs: (out [L,V], state [V,K])."""
    G = inp.Hv // inp.Hqk
    if inp.cu_seqlens is None:
        b, a, e = n, 0, inp.T
    else:
        b, a, e = 0, int(inp.cu_seqlens[n]), int(inp.cu_seqlens[n + 1])
    hq = h // G
    sl = lambda x, hh: np.ascontiguousarray(x[b:b + 1, a:e, hh:hh + 1])
    h0 = None if h0_f64 is None else h0_f64[n:n + 1, h:h + 1]
    o, s = oracle.fwd(sl(inp.q, hq), sl(inp.k, hq), sl(inp.v, h), sl(inp.g, h),
                      np.ascontiguousarray(inp.beta[b:b + 1, a:e, h:h + 1]),
                      None if inp.A_log is None else inp.A_log[h:h + 1],
                      None if inp.dt_bias is None else inp.dt_bias[h:h + 1], scale=inp.scale,
                      lower_bound=inp.lower_bound, gate_mode=inp.gate_mode, flags=inp.flags, initial_state=h0,
                      nthreads=1)
    return o[0, :, 0], s[0, 0]


def oracle_pairs(inp: W.KdaInputs, pairs, workers=8):
    h0 = inp.initial_state_f64()
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        futs = {p: ex.submit(oracle_pair, inp, p[0], p[1], h0) for p in pairs}
        return {p: f.result() for p, f in futs.items()}


def as_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def errors(o_gpu, o_ref, s_gpu=None, s_ref=None, state_bf16=False):
    e = {}
    e["out_max_abs"] = float(np.abs(o_gpu - o_ref).max()) if o_ref.size else 0.0
    nr = np.linalg.norm(o_ref)
    e["out_rel_rms"] = float(np.linalg.norm(o_gpu - o_ref) / nr) if nr > 0 else float(np.linalg.norm(o_gpu))
    if s_ref is not None:
        ns = np.linalg.norm(s_ref)
        e["state_rel"] = float(np.linalg.norm(s_gpu - s_ref) / ns) if ns > 0 else float(np.linalg.norm(s_gpu))
        e["state_max_abs"] = float(np.abs(s_gpu - s_ref).max())
        e["state_bf16"] = state_bf16
    return e


def assert_parity(e, what=""):
    log(f"    {what} {e}")
    assert e["out_max_abs"] <= OUT_MAX_ABS, (what, e)
    assert e["out_rel_rms"] <= OUT_REL_RMS, (what, e)
    if "state_rel" in e:
        if e["state_bf16"]:
            assert e["state_max_abs"] <= OUT_MAX_ABS, (what, e)
        else:
            assert e["state_rel"] <= STATE_REL, (what, e)
