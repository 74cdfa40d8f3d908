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
match the oracle, and so must v whose size changes from chunk to chunk by up to
2^12 over a total range of 2^88, or jumps for a single chunk by up to 2^18.  The chunked path keeps the decay factors of a
chunk in fp16 operands, so a contribution decayed within one chunk below about
2^-24 of its source is dropped; that is far below the tolerance unless v falls
by more than about 2^20 from one chunk to the next, so a fall of 2^40 is run
through the fp32 token-recurrent entry only.
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


# per 64-token chunk: the power of two that scales v
RAMP_UP = [8 * c for c in range(12)]
RAMP_DOWN = [-8 * c for c in range(12)]
MIXED = [0, 8, -4, 10, 2, -6, 6, 12, 4, -4, 8, 0]
EXTREME = [0, 20, -20, 20, -20, 0, 16, -16, 20, 0, -20, 4]
# single chunks far above their neighbours and the state
SPIKES = [0, 0, 16, 0, 0, 0, 12, 0, 0, 18, 0, 0]


def jumping_v(inp: W.KdaInputs, jumps) -> W.KdaInputs:
    v = W.bf16_bits_to_f32(inp.v).copy()
    for c in range((inp.T + 63) // 64):
        v[:, 64 * c:64 * (c + 1)] *= np.float32(2.0 ** jumps[c % len(jumps)])
    r = W.f32_to_bf16_bits(v)
    assert np.array_equal(W.bf16_bits_to_f32(r), v)
    return W.KdaInputs(**{**inp.__dict__, "v": r})


def check_tokenwise(inp, recurrent, what):
    o, st = run(inp, recurrent)
    assert torch.isfinite(o.float()).all() and torch.isfinite(st).all()
    o_ref, s_ref = U.run_oracle(inp)
    og = U.as_f64(o)
    # relative error of every (token, head) row of the output, each held to its own size
    num = np.linalg.norm(og - o_ref, axis=-1)
    den = np.linalg.norm(o_ref, axis=-1)
    rel = num / np.maximum(den, 1e-300)
    worst = float(rel[den > 0].max())
    U.log(f"    {what}: worst per-token relative error {worst:.3e}, mean {float(rel[den > 0].mean()):.3e}")
    assert worst <= 2e-2, (what, worst)
    e = U.errors(og, o_ref, U.as_f64(st), s_ref)
    assert e["state_rel"] <= U.STATE_REL, (what, e)


def jump_inputs(gate, jumps):
    extra = dict(gate_mode=W.GATE_SAFE_SIGMOID, lower_bound=-1.0) if gate == W.GATE_SAFE_SIGMOID else \
        dict(A_log_range=(-6.0, -2.0))
    base = W.make_inputs(B=2, T=64 * len(jumps) - 5, Hqk=2, seed=320, init_state_dtype=W.STATE_F32, h0_std=1e-6,
                         **extra)
    return jumping_v(base, jumps)


@pytest.mark.parametrize("recurrent", [False, True])
@pytest.mark.parametrize("pattern", ["ramp_up", "ramp_down", "mixed"])
@pytest.mark.parametrize("gate", [W.GATE_SAFE_SIGMOID, W.GATE_SOFTPLUS])
def test_value_magnitude_changes_between_chunks(gate, pattern, recurrent):
    # v changes size from chunk to chunk by up to 2^12, over a total range of
    # 2^88, so the state kernel's power-of-two exponent has to follow it chunk
    # by chunk; every output token is held to its own size and the fp32 state
    # to the usual relative bound
    jumps = {"ramp_up": RAMP_UP, "ramp_down": RAMP_DOWN, "mixed": MIXED}[pattern]
    U.log(f"[gpu] v magnitude {pattern} {jumps}, gate={gate}, recurrent={recurrent}")
    check_tokenwise(jump_inputs(gate, jumps), recurrent, pattern)


@pytest.mark.parametrize("recurrent", [False, True])
def test_single_chunk_spikes(recurrent):
    # one chunk's v 2^12 .. 2^18 above the state and the chunks around it: the
    # chunked path must scale U_c by the size of that chunk's T diag(b) V (in
    # fp16 at the size of the state, U_c would overflow); softplus decay, so
    # that the state written by a spike is still the larger part of the next
    # chunks' outputs
    U.log(f"[gpu] single-chunk spikes {SPIKES}, recurrent={recurrent}")
    check_tokenwise(jump_inputs(W.GATE_SOFTPLUS, SPIKES), recurrent, "spikes")


@pytest.mark.parametrize("gate", [W.GATE_SAFE_SIGMOID, W.GATE_SOFTPLUS])
def test_recurrent_value_magnitude_jumps_2_40(gate):
    # the token-recurrent entry is fp32 throughout: even v falling by 2^40 from
    # one chunk to the next, where the old state's decayed contribution still
    # dominates the new outputs, is reproduced token by token
    U.log(f"[gpu] recurrent, v magnitude jumps {EXTREME}, gate={gate}")
    check_tokenwise(jump_inputs(gate, EXTREME), True, "extreme jumps")
