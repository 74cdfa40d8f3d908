"""GPU parity of the segmented state chain: dense input whose per-(sequence,
head) chunk chain is cut into time segments that run in parallel (each
segment's state carried from zero and its linear map give its entry state;
then every segment emits its outputs).  Checked element by element against
the fp64 oracle, against the unsplit chain within the tolerances, and for
in-place state updates (bit-identical to out-of-place ones)."""
import pytest
import torch

from gated_delta_rule_act_amd import workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def small(**kw):
    base = dict(B=2, T=1000, Hqk=2, Hv=4, seed=401, init_state_dtype=W.STATE_F32)
    base.update(kw)
    return W.make_inputs(**base)


# (inputs, segments): 16 chunks with a 40-token tail unless stated
CASES = {
    "safe_lb5_seg4": (dict(gate_mode=W.GATE_SAFE_SIGMOID, lower_bound=-5.0, A_log_range=(-4.0, 6.0), g_std=3.0), 4),
    "softplus_seg16_one_chunk_each": (dict(B=1), 16),
    "softplus_seg3_bf16_state": (dict(T=700, init_state_dtype=W.STATE_BF16, final_state_dtype=W.STATE_BF16), 3),
    "pregated_seg5": (dict(B=1, T=1280, gate_mode=W.GATE_PREGATED, pregated_range=(-2.0, 0.0)), 5),
    "no_initial_state_seg2": (dict(T=513, init_state_dtype=W.STATE_NONE), 2),
    "no_final_state_seg6": (dict(final_state_dtype=W.STATE_NONE), 6),
    "long_memory_seg8": (dict(B=1, T=2048, A_log_range=(-8.0, -6.0)), 8),
    "more_segments_than_chunks": (dict(B=1, T=200), 7),
    "beta_prob_no_l2norm_seg4": (dict(beta_prob=True, flags=0, qk_std=1.0 / 128 ** 0.5), 4),
    # 4 chains x 24 segments = 96 jobs per launch: 64-column V slices in every pass
    "wide_slices_seg24": (dict(B=1, T=2048, gate_mode=W.GATE_SAFE_SIGMOID, lower_bound=-5.0), 24),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_segments_elementwise(name):
    kw, segments = CASES[name]
    inp = small(**kw)
    U.log(f"[gpu] segments {name}: B={inp.B} T={inp.T} Hqk={inp.Hqk} Hv={inp.Hv} gate={inp.gate_mode} "
          f"segments={segments}")
    o, s = U.run_gpu(inp, segments=segments)
    o_ref, s_ref = U.run_oracle(inp)
    assert not torch.isnan(o.float()).any(), "some output element was not written"
    if s is None:
        U.assert_parity(U.errors(U.as_f64(o), o_ref), name)
        return
    assert torch.isfinite(s.float()).all()
    U.assert_parity(U.errors(U.as_f64(o), o_ref, U.as_f64(s), s_ref,
                             state_bf16=inp.final_state_dtype == W.STATE_BF16), name)


@pytest.mark.parametrize("segments", [2, 5, 32])
def test_segments_match_unsplit(segments):
    inp = small(B=1, T=64 * 40 + 17, gate_mode=W.GATE_SAFE_SIGMOID, lower_bound=-1.0)
    U.log(f"[gpu] segments={segments} vs unsplit, T={inp.T}")
    d = U.to_device(inp)
    o1, s1 = U.run_gpu(inp, d, segments=1)
    o2, s2 = U.run_gpu(inp, d, segments=segments)
    assert (o1.float() - o2.float()).abs().max().item() <= U.OUT_MAX_ABS
    assert ((s1 - s2).norm() / s1.norm()).item() <= U.STATE_REL


@pytest.mark.parametrize("segments", [1, 4])
def test_in_place_state(segments):
    inp = small(B=2, T=900)
    U.log(f"[gpu] in-place state, segments={segments}")
    d = U.to_device(inp)
    o_ref, s_ref = U.run_gpu(inp, d, segments=segments)
    st = d["h0"].clone()
    o, s = U.run_gpu(inp, d, segments=segments, final_state=st, initial_state=st)
    assert s.data_ptr() == st.data_ptr()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(s, s_ref)


def test_packed_ignores_segments():
    lengths = [300, 0, 129, 700]
    inp = W.make_inputs(B=1, T=None, Hqk=2, Hv=4, seed=43, lengths=lengths, init_state_dtype=W.STATE_F32)
    U.log(f"[gpu] packed {lengths} with segments=8 (ignored)")
    d = U.to_device(inp)
    o1, s1 = U.run_gpu(inp, d, segments=1)
    o2, s2 = U.run_gpu(inp, d, segments=8)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(s1, s2)
