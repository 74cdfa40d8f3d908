"""The allocation-free forward (kda_fwd_noalloc) through the C ABI: it runs
the same kernels as kda_fwd on the library's own per-GPU device array, so on
the same inputs its outputs and final state equal kda_fwd's bit for bit (and
so meet the parity bar kda_fwd is held to).  Two calls in a row, the second
smaller, check that the array's contents from one call do not leak into the
next; a call whose workspace exceeds the array is rejected before launch.
"""
import pytest
import torch

from gated_delta_rule_act_amd import kda
from gated_delta_rule_act_amd import workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def both(inp):
    d = U.to_device(inp)
    o_ref, s_ref = U.run_gpu(inp, d)
    fdt = U.final_dtype_of(inp)
    out = torch.full_like(o_ref, float("nan"))
    fs = None if s_ref is None else torch.full_like(s_ref, float("nan"))
    o, s = kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"], d["dt_bias"], inp.scale,
                   inp.lower_bound, inp.gate_mode, initial_state=d["h0"], cu_seqlens=d["cu_seqlens"], out=out,
                   final_state=fs, final_state_dtype=fdt, qk_l2norm=bool(inp.flags & W.FLAG_QK_L2NORM),
                   beta_is_prob=bool(inp.flags & W.FLAG_BETA_IS_PROB), noalloc=True)
    torch.cuda.synchronize()
    return (o, s), (o_ref, s_ref)


def test_noalloc_matches_workspace_entry_twice():
    calls = [
        # larger first: packed sequences with bf16 states
        W.make_inputs(B=1, T=None, Hqk=2, Hv=4, seed=401, lengths=[70, 1, 300, 64, 129],
                      init_state_dtype=W.STATE_BF16, final_state_dtype=W.STATE_BF16),
        # then smaller, dense, safe gate, fp32 states
        W.make_inputs(B=2, T=150, Hqk=1, Hv=2, seed=402, init_state_dtype=W.STATE_F32,
                      gate_mode=W.GATE_SAFE_SIGMOID, lower_bound=-5.0),
    ]
    for i, inp in enumerate(calls):
        U.log(f"[gpu] no-alloc call {i}: B={inp.B} T={inp.T} Hv={inp.Hv} packed={inp.cu_seqlens is not None}")
        (o, s), (o_ref, s_ref) = both(inp)
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), i
        assert torch.equal(s.view(torch.int16) if s.dtype == torch.bfloat16 else s,
                           s_ref.view(torch.int16) if s_ref.dtype == torch.bfloat16 else s_ref), i
        o_or, s_or = U.run_oracle(inp)
        U.assert_parity(U.errors(U.as_f64(o), o_or, U.as_f64(s), s_or,
                                 state_bf16=inp.final_state_dtype == W.STATE_BF16), f"no-alloc call {i}")


def test_noalloc_rejects_oversized_call():
    inp = W.make_inputs(B=2, T=8192, Hqk=16, seed=403, init_state_dtype=W.STATE_F32)
    p = kda.make_params(B=inp.B, T=inp.T, H_qk=inp.Hqk, H_v=inp.Hv, scale=inp.scale,
                        init_state_dtype=W.STATE_F32)
    assert kda.workspace_size(p) > 128 * 1024 * 1024
    d = U.to_device(inp)
    out = torch.empty((inp.B, inp.T, inp.Hv, inp.V), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kda.KdaError) as ei:
        kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"], d["dt_bias"], inp.scale, inp.lower_bound,
                inp.gate_mode, initial_state=d["h0"], out=out, noalloc=True)
    assert ei.value.status == kda.KDA_ERR_WORKSPACE
