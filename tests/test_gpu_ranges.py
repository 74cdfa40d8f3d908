"""GPU parity over the magnitudes the call contract admits.

The FlashKDA page's "Tensor shapes and dtypes" table admits any bf16 v and
any fp32 / bf16 initial state, and with the in-kernel L2 norm any bf16 q and
k.  The recurrence is linear in (v, initial state) jointly, so scaling both
by 2^s scales the output and the final state by exactly 2^s; with the L2 norm
on, the output does not depend on the size of q and k at all.

Both HIP entries must therefore give, for v and h0 scaled by 2^s, exactly
2^s times their own unscaled results, bit for bit (the chunked path keeps its
16-bit operands at a normalised magnitude by a power-of-two exponent; the
token-recurrent path is fp32 throughout), and must match the oracle on the
scaled inputs within the parity tolerances, measured in units of 2^s.
Raw q and k scaled far up or down (beyond the fp16 range, 2^20) must still
match the oracle.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_act_amd import kda
from gated_delta_rule_act_amd import workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

SCALES = [-16, -8, 8, 16]


def scale_bf16_bits(bits: np.ndarray, s: int) -> np.ndarray:
    x = W.bf16_bits_to_f32(bits)
    y = x * np.float32(2.0 ** s)
    r = W.f32_to_bf16_bits(y)
    assert np.array_equal(W.bf16_bits_to_f32(r), y), "the scaled bf16 values must be exact"
    return r


def scaled_vh0(inp: W.KdaInputs, s: int) -> W.KdaInputs:
    h0 = inp.initial_state
    if h0 is not None:
        if inp.init_state_dtype == W.STATE_BF16:
            h0 = scale_bf16_bits(h0, s)
        else:
            h0 = (h0 * np.float32(2.0 ** s)).astype(np.float32)
    return W.KdaInputs(**{**inp.__dict__, "v": scale_bf16_bits(inp.v, s), "initial_state": h0})


def scaled_qk(inp: W.KdaInputs, s: int) -> W.KdaInputs:
    return W.KdaInputs(**{**inp.__dict__, "q": scale_bf16_bits(inp.q, s), "k": scale_bf16_bits(inp.k, s)})


def run(inp, recurrent=False, segments=0):
    if not recurrent:
        return U.run_gpu(inp, segments=segments)
    d = U.to_device(inp)
    fdt = U.final_dtype_of(inp)
    out = torch.full((inp.B, inp.T, inp.Hv, inp.V), float("nan"), dtype=torch.bfloat16, device="cuda")
    fs = torch.full((inp.N, inp.Hv, inp.V, inp.K), float("nan"), dtype=fdt, device="cuda")
    o, st = kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"], d["dt_bias"], inp.scale,
                    inp.lower_bound, inp.gate_mode, initial_state=d["h0"], cu_seqlens=d["cu_seqlens"], out=out,
                    final_state=fs, final_state_dtype=fdt, recurrent=True)
    torch.cuda.synchronize()
    return o, st


# (name, inputs, entry, forced segment count)
def cases():
    safe = dict(gate_mode=W.GATE_SAFE_SIGMOID, lower_bound=-5.0, A_log_range=(-4.0, 6.0), g_std=3.0)
    return {
        # 8 chains: 32-column V slices
        "narrow_safe_lb5": (W.make_inputs(B=2, T=300, Hqk=4, seed=301, init_state_dtype=W.STATE_F32, **safe),
                            False, 0),
        # 68 chains: 64-column V slices
        "wide_softplus": (W.make_inputs(B=17, T=150, Hqk=2, Hv=4, seed=302, init_state_dtype=W.STATE_F32),
                          False, 0),
        # one long chain cut into 4 time segments (carry, map and combine passes)
        "segments_4": (W.make_inputs(B=1, T=1100, Hqk=1, Hv=2, seed=303, init_state_dtype=W.STATE_F32, **safe),
                       False, 4),
        # packed sequences with bf16 states; v only when there is no initial state
        "packed_bf16_state": (W.make_inputs(B=1, T=None, Hqk=2, Hv=4, seed=304, lengths=[1, 63, 64, 65, 200, 130],
                                            init_state_dtype=W.STATE_BF16, final_state_dtype=W.STATE_BF16),
                              False, 0),
        "no_initial_state": (W.make_inputs(B=2, T=200, Hqk=2, seed=305), False, 0),
        "recurrent_safe_lb5": (W.make_inputs(B=3, T=40, Hqk=2, seed=306, init_state_dtype=W.STATE_F32, **safe),
                               True, 0),
    }


CASES = cases()


@pytest.mark.parametrize("name", sorted(CASES))
def test_value_and_state_scale_exactly(name):
    inp, recurrent, segments = CASES[name]
    U.log(f"[gpu] magnitude sweep {name}: B={inp.B} T={inp.T} Hv={inp.Hv} segments={segments} scales={SCALES}")
    o0, s0 = run(inp, recurrent, segments)
    assert torch.isfinite(o0.float()).all() and torch.isfinite(s0.float()).all()
    bf = inp.final_state_dtype == W.STATE_BF16
    for s in SCALES:
        inp_s = scaled_vh0(inp, s)
        o1, s1 = run(inp_s, recurrent, segments)
        f = 2.0 ** s
        # bit-exact scaling of every output and state element
        assert torch.equal(o1.float(), o0.float() * f), (name, s)
        assert torch.equal(s1.float(), s0.float() * f), (name, s)
        o_ref, s_ref = U.run_oracle(inp_s)
        U.assert_parity(U.errors(U.as_f64(o1) / f, o_ref / f, U.as_f64(s1) / f, s_ref / f, state_bf16=bf),
                        f"{name} v,h0 x 2^{s}")


@pytest.mark.parametrize("s", [-6, 6, 20])
@pytest.mark.parametrize("recurrent", [False, True])
def test_raw_qk_magnitude_under_l2norm(s, recurrent):
    # with the L2 norm on, raw q and k of any size are legal inputs; 2^20 is
    # far beyond the fp16 range, where an unnormalised 16-bit operand overflows
    inp = W.make_inputs(B=2, T=200 if not recurrent else 30, Hqk=2, seed=310, init_state_dtype=W.STATE_F32,
                        gate_mode=W.GATE_SAFE_SIGMOID, lower_bound=-5.0, A_log_range=(-4.0, 6.0), g_std=3.0)
    inp_s = scaled_qk(inp, s)
    U.log(f"[gpu] raw q, k x 2^{s}, recurrent={recurrent}")
    o, st = run(inp_s, recurrent)
    assert torch.isfinite(o.float()).all() and torch.isfinite(st).all()
    o_ref, s_ref = U.run_oracle(inp_s)
    U.assert_parity(U.errors(U.as_f64(o), o_ref, U.as_f64(st), s_ref), f"q,k x 2^{s}")
