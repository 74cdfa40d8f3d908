"""GPU parity of the token-recurrent entry (kda_fused_recurrent_fwd) against
the fp64 oracle, plus the invariants that hold for it exactly: a sequence fed
one token per call with the fp32 state carried equals one call over the whole
sequence, bit for bit; an in-place state update equals an out-of-place one;
and it agrees with the chunked entry within the parity tolerances.
"""
import math

import numpy as np
import pytest
import torch

from gated_delta_rule_act_amd import kda
from gated_delta_rule_act_amd import workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def run_rec(inp, d=None, final_state=None, initial_state=None):
    d = d or U.to_device(inp)
    out = torch.full((inp.B, inp.T, inp.Hv, inp.V), float("nan"), dtype=torch.bfloat16, device="cuda")
    fdt = U.final_dtype_of(inp)
    fs = final_state
    if fs is None and fdt is not None:
        fs = torch.full((inp.N, inp.Hv, inp.V, inp.K), float("nan"), dtype=fdt, device="cuda")
    h0 = d["h0"] if initial_state is None else initial_state
    o, s = kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"], d["dt_bias"], inp.scale,
                   inp.lower_bound, inp.gate_mode, initial_state=h0, cu_seqlens=d["cu_seqlens"], out=out,
                   final_state=fs, final_state_dtype=fdt, recurrent=True,
                   qk_l2norm=bool(inp.flags & W.FLAG_QK_L2NORM), beta_is_prob=bool(inp.flags & W.FLAG_BETA_IS_PROB))
    torch.cuda.synchronize()
    return o, s


def small(**kw):
    base = dict(B=2, T=50, Hqk=4, seed=211, init_state_dtype=W.STATE_F32)
    base.update(kw)
    return W.make_inputs(**base)


CASES = {
    "decode_softplus": dict(T=1, B=4),
    "decode_safe_lb5": dict(T=1, B=4, gate_mode=W.GATE_SAFE_SIGMOID, lower_bound=-5.0, A_log_range=(-4.0, 6.0),
                            g_std=3.0),
    "decode_pregated": dict(T=1, B=4, gate_mode=W.GATE_PREGATED, pregated_range=(-2.0, 0.0)),
    "short_softplus": dict(T=37),
    "short_safe_gva": dict(T=70, Hqk=2, Hv=6, gate_mode=W.GATE_SAFE_SIGMOID, lower_bound=-1.0),
    "no_initial_state": dict(T=65, init_state_dtype=W.STATE_NONE),
    "bf16_state": dict(T=20, init_state_dtype=W.STATE_BF16, final_state_dtype=W.STATE_BF16),
    "beta_prob_no_l2norm": dict(T=40, beta_prob=True, flags=0, qk_std=1.0 / math.sqrt(128)),
    "safe_no_A_log": dict(T=30, gate_mode=W.GATE_SAFE_SIGMOID, lower_bound=-5.0, with_A_log=False),
    "long_memory": dict(T=300, B=1, A_log_range=(-8.0, -6.0)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_recurrent_elementwise(name):
    inp = small(**CASES[name])
    U.log(f"[gpu] recurrent {name}: B={inp.B} T={inp.T} Hqk={inp.Hqk} Hv={inp.Hv} gate={inp.gate_mode}")
    o, s = run_rec(inp)
    o_ref, s_ref = U.run_oracle(inp)
    assert torch.isfinite(o.float()).all() and torch.isfinite(s.float()).all()
    U.assert_parity(U.errors(U.as_f64(o), o_ref, U.as_f64(s), s_ref,
                             state_bf16=inp.final_state_dtype == W.STATE_BF16), name)


def test_recurrent_packed():
    lengths = [1, 0, 5, 64, 130]
    inp = W.make_inputs(B=1, T=None, Hqk=2, Hv=4, seed=23, lengths=lengths, init_state_dtype=W.STATE_F32)
    U.log(f"[gpu] recurrent packed {lengths}")
    o, s = run_rec(inp)
    o_ref, s_ref = U.run_oracle(inp)
    U.assert_parity(U.errors(U.as_f64(o), o_ref, U.as_f64(s), s_ref), "recurrent packed")
    # the empty sequence returns its initial state exactly
    assert torch.equal(s[1].cpu(), torch.from_numpy(inp.initial_state[1]))


def test_token_by_token_equals_one_call():
    inp = small(T=24, B=2)
    U.log("[gpu] recurrent: token-by-token = one call")
    d = U.to_device(inp)
    o_all, s_all = run_rec(inp, d)
    state = d["h0"].clone()
    outs = []
    for t in range(inp.T):
        sl = lambda x: np.ascontiguousarray(x[:, t:t + 1])
        step = W.KdaInputs(**{**inp.__dict__, "q": sl(inp.q), "k": sl(inp.k), "v": sl(inp.v), "g": sl(inp.g),
                              "beta": sl(inp.beta)})
        ds = U.to_device(step)
        o1, state = run_rec(step, ds, initial_state=state)
        outs.append(o1)
    assert torch.equal(torch.cat(outs, dim=1).view(torch.int16), o_all.view(torch.int16))
    assert torch.equal(state, s_all)


def test_in_place_state_update():
    inp = small(T=9, B=3)
    U.log("[gpu] recurrent: in-place state")
    d = U.to_device(inp)
    o_ref, s_ref = run_rec(inp, d)
    st = d["h0"].clone()
    o, s = run_rec(inp, d, final_state=st, initial_state=st)
    assert s.data_ptr() == st.data_ptr()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(s, s_ref)


@pytest.mark.parametrize("mode", [W.GATE_SOFTPLUS, W.GATE_SAFE_SIGMOID])
def test_recurrent_matches_chunked(mode):
    inp = small(T=200, B=2, gate_mode=mode, lower_bound=-5.0 if mode == W.GATE_SAFE_SIGMOID else -1.0)
    U.log(f"[gpu] recurrent vs chunked, gate {mode}")
    d = U.to_device(inp)
    o_r, s_r = run_rec(inp, d)
    o_c, s_c = U.run_gpu(inp, d)
    assert (o_r.float() - o_c.float()).abs().max().item() <= U.OUT_MAX_ABS
    assert ((s_r - s_c).norm() / s_c.norm()).item() <= U.STATE_REL


def test_decode_batch_full_size():
    # one decode step for 64 sequences x 32 heads with fp32 state in and out,
    # sampled (sequence, head) pairs against the oracle
    inp = W.make_inputs(B=64, T=1, Hqk=32, seed=31, gate_mode=W.GATE_SAFE_SIGMOID, lower_bound=-5.0,
                        A_log_range=(-4.0, 6.0), g_std=3.0, init_state_dtype=W.STATE_F32)
    U.log("[gpu] recurrent decode B=64 H=32 T=1")
    o, s = run_rec(inp)
    assert not torch.isnan(o.float()).any() and not torch.isnan(s).any()
    refs = U.oracle_pairs(inp, [(0, 0), (17, 5), (40, 31), (63, 16)])
    for (n, h), (o_ref, s_ref) in refs.items():
        U.assert_parity(U.errors(U.as_f64(o[n, :, h]), o_ref, U.as_f64(s[n, h]), s_ref), f"decode n={n} h={h}")


def test_recurrent_packed_decode():
    # at most one token per sequence (the one-token block path), one sequence empty
    lengths = [1, 0, 1, 1]
    inp = W.make_inputs(B=1, T=None, Hqk=2, Hv=4, seed=29, lengths=lengths, init_state_dtype=W.STATE_F32)
    U.log(f"[gpu] recurrent packed decode {lengths}")
    o, s = run_rec(inp)
    o_ref, s_ref = U.run_oracle(inp)
    U.assert_parity(U.errors(U.as_f64(o), o_ref, U.as_f64(s), s_ref), "recurrent packed decode")
    assert torch.equal(s[1].cpu(), torch.from_numpy(inp.initial_state[1]))
