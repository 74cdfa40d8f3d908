"""Host-side tests of the C ABI (no GPU needed).

The library must load, export every function include/kda.h declares, and
reject each invalid argument with its documented status before anything is
launched.  kda_fwd_check dereferences nothing, so fake aligned addresses
stand in for device pointers.
"""
import ctypes
import os
import re

import pytest

from gated_delta_rule_act_amd import kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000  # 256-byte aligned stand-in address, never dereferenced


@pytest.fixture(scope="module")
def lib():
    return kda.load_library()


def header_functions():
    src = open(os.path.join(ROOT, "include", "kda.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert set(names) == set(kda.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code, name in kda._STATUS.items():
        assert lib.kda_status_string(code).decode() == name
    assert lib.kda_status_string(-99).decode() == "KDA_ERR_UNKNOWN"


def base_params(**kw):
    d = dict(B=2, T=300, H_qk=4, H_v=4, scale=0.125, lower_bound=-1.0, gate_mode=kda.GATE_SOFTPLUS,
             init_state_dtype=kda.STATE_F32, final_state_dtype=kda.STATE_F32)
    d.update(kw)
    return kda.make_params(**d)


def check(lib, p, ws=None, cu=None, drop=None, shift=None):
    ptrs = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, A_log=FAKE, dt_bias=FAKE, cu=cu,
                h0=FAKE if p.init_state_dtype else None, hT=FAKE if p.final_state_dtype else None,
                out=FAKE, ws=FAKE)
    for name in ((drop,) if isinstance(drop, str) else (drop or ())):
        ptrs[name] = None
    if shift:
        ptrs[shift] = ptrs[shift] + 2
    need = lib.kda_fwd_workspace_size(ctypes.byref(p))
    order = ["q", "k", "v", "g", "beta", "A_log", "dt_bias", "cu", "h0", "hT", "out", "ws"]
    args = [None if ptrs[n] is None else ctypes.c_void_p(ptrs[n]) for n in order]
    return lib.kda_fwd_check(ctypes.byref(p), *args, ctypes.c_size_t(need if ws is None else ws))


def test_valid_dense_and_packed(lib):
    assert check(lib, base_params()) == kda.KDA_OK
    p = base_params(B=1, T=1000, num_seqs=7)
    assert check(lib, p, cu=FAKE) == kda.KDA_OK


@pytest.mark.parametrize("field,bad,code", [
    ("K", 64, -2), ("V", 256, -2), ("K", 129, -2), ("H_v", 6, -2), ("B", 0, -2), ("T", -1, -2),
    ("num_seqs", 3, -2), ("gate_mode", 3, -8), ("gate_mode", -1, -8), ("flags", 4, -8), ("flags", -1, -8),
    ("init_state_dtype", 3, -3), ("final_state_dtype", -1, -3),
])
def test_shape_dtype_mode_rejections(lib, field, bad, code):
    p = base_params()
    setattr(p, field, bad)
    assert check(lib, p) == code, kda.last_error()
    assert kda.last_error() != ""


def test_launch_size_limits(lib):
    # a dispatch dimension holds fewer than 2^32 work-items: at most 2^21
    # (sequence, head) pairs (4 state workgroups of 256 each) and fewer than
    # 2^24 chunks per head (one workgroup each along x)
    assert check(lib, base_params(B=1 << 19, T=1, H_qk=4, H_v=4)) == kda.KDA_OK
    assert check(lib, base_params(B=(1 << 19) + 1, T=1, H_qk=4, H_v=4)) == -2
    assert "pairs" in kda.last_error()
    assert check(lib, base_params(B=1, T=64 * ((1 << 24) - 1), H_qk=1, H_v=1)) == kda.KDA_OK
    assert check(lib, base_params(B=1, T=64 * (1 << 24), H_qk=1, H_v=1)) == -2
    assert "chunks" in kda.last_error()


def test_gva_head_ratio(lib):
    assert check(lib, base_params(H_qk=2, H_v=6)) == kda.KDA_OK
    assert check(lib, base_params(H_qk=4, H_v=6)) == -2


def test_packed_requires_single_row(lib):
    p = base_params(B=2, T=100, num_seqs=2)
    assert check(lib, p, cu=FAKE) == -2
    p = base_params(B=1, T=100, num_seqs=0)
    assert check(lib, p, cu=FAKE) == -2


@pytest.mark.parametrize("lb,ok", [(-5.0, True), (-5.0001, False), (-4.9999, True), (0.0, False),
                                   (0.1, False), (-1e-30, True), (float("nan"), False),
                                   (float("-inf"), False)])
def test_lower_bound_range_safe_gate(lib, lb, ok):
    p = base_params(gate_mode=kda.GATE_SAFE_SIGMOID, lower_bound=lb)
    assert (check(lib, p) == kda.KDA_OK) == ok
    if not ok:
        assert check(lib, p) == -4


def test_lower_bound_ignored_for_softplus(lib):
    assert check(lib, base_params(gate_mode=kda.GATE_SOFTPLUS, lower_bound=7.0)) == kda.KDA_OK


def test_state_dtypes_must_match(lib):
    assert check(lib, base_params(init_state_dtype=1, final_state_dtype=2)) == -3
    assert check(lib, base_params(init_state_dtype=2, final_state_dtype=2)) == kda.KDA_OK
    assert check(lib, base_params(init_state_dtype=0, final_state_dtype=2)) == kda.KDA_OK
    assert check(lib, base_params(init_state_dtype=1, final_state_dtype=0)) == kda.KDA_OK


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "beta", "A_log", "out", "h0", "hT", "ws"])
def test_null_pointers(lib, name):
    # softplus gate: A_log is required
    code = check(lib, base_params(), drop=name)
    assert code == (-6 if name == "ws" else -1)


@pytest.mark.parametrize("flags", [0, 1, 2, 3])
def test_flag_combinations_accepted(lib, flags):
    assert check(lib, base_params(flags=flags)) == kda.KDA_OK


def test_optional_gate_parameters(lib):
    # dt_bias is optional for both activated gates
    assert check(lib, base_params(), drop="dt_bias") == kda.KDA_OK
    safe = dict(gate_mode=kda.GATE_SAFE_SIGMOID, lower_bound=-5.0)
    assert check(lib, base_params(**safe), drop="dt_bias") == kda.KDA_OK
    # a missing A_log means a multiplier of one for the safe gate only
    assert check(lib, base_params(**safe), drop="A_log") == kda.KDA_OK
    assert check(lib, base_params(**safe), drop=("A_log", "dt_bias")) == kda.KDA_OK
    assert check(lib, base_params(), drop="A_log") == -1


def test_pregated_contract(lib):
    pre = dict(gate_mode=kda.GATE_PREGATED)
    # the decay is given directly: no bias may accompany it, A_log is unused
    assert check(lib, base_params(**pre), drop="dt_bias") == kda.KDA_OK
    assert check(lib, base_params(**pre), drop=("dt_bias", "A_log")) == kda.KDA_OK
    assert check(lib, base_params(**pre)) == -8
    # lower_bound belongs to the safe activation and is not range-checked here
    assert check(lib, base_params(lower_bound=3.0, **pre), drop="dt_bias") == kda.KDA_OK
    # the bias rule holds for empty inputs too
    assert check(lib, base_params(T=0, **pre)) == -8


@pytest.mark.parametrize("name", ["q", "k", "v", "g", "out", "dt_bias", "h0", "hT"])
def test_misaligned(lib, name):
    assert check(lib, base_params(), shift=name) == -5


def test_workspace_too_small(lib):
    p = base_params()
    need = lib.kda_fwd_workspace_size(ctypes.byref(p))
    assert check(lib, p, ws=need) == kda.KDA_OK
    assert check(lib, p, ws=need - 1) == -6


def test_workspace_size_monotone(lib):
    size = lambda **kw: lib.kda_fwd_workspace_size(ctypes.byref(base_params(**kw)))
    # whole 64-token chunks: equal within a chunk, growing across a boundary
    assert size(T=1) == size(T=63) == size(T=64) < size(T=65) < size(T=1000) < size(T=8192)
    assert lib.kda_fwd_workspace_size(ctypes.byref(base_params(H_v=8, H_qk=4))) > \
        lib.kda_fwd_workspace_size(ctypes.byref(base_params()))
    bad = base_params(K=64)
    assert lib.kda_fwd_workspace_size(ctypes.byref(bad)) == 0


def test_empty_input_needs_no_tensors(lib):
    p = base_params(T=0)
    assert check(lib, p, drop="q") == kda.KDA_OK


def recurrent_call(lib, p, drop=None):
    ptrs = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, A_log=FAKE, dt_bias=FAKE, cu=None,
                h0=FAKE if p.init_state_dtype else None, hT=FAKE if p.final_state_dtype else None, out=FAKE)
    for name in ((drop,) if isinstance(drop, str) else (drop or ())):
        ptrs[name] = None
    order = ["q", "k", "v", "g", "beta", "A_log", "dt_bias", "cu", "h0", "hT", "out"]
    args = [None if ptrs[n] is None else ctypes.c_void_p(ptrs[n]) for n in order]
    return lib.kda_fused_recurrent_fwd(ctypes.byref(p), *args, None)


@pytest.mark.parametrize("case,code", [
    (dict(params=dict(K=64)), -2),
    (dict(params=dict(gate_mode=3)), -8),
    (dict(params=dict(gate_mode=kda.GATE_SAFE_SIGMOID, lower_bound=0.0)), -4),
    (dict(params=dict(gate_mode=kda.GATE_PREGATED)), -8),
    (dict(drop="q"), -1),
    (dict(drop="A_log"), -1),
    (dict(drop="hT"), -1),
    (dict(params=dict(init_state_dtype=1, final_state_dtype=2)), -3),
])
def test_recurrent_entry_rejects_before_launch(lib, case, code):
    # only rejections: a valid call would launch, and these tests run without a GPU
    p = base_params(**case.get("params", {}))
    assert recurrent_call(lib, p, case.get("drop")) == code, kda.last_error()


@pytest.mark.parametrize("segments,code", [(-1, -4), (257, -4), (0, 0), (1, 0), (2, 0), (256, 0)])
def test_segments_range(lib, segments, code):
    p = base_params(segments=segments)
    assert check(lib, p) == code, kda.last_error()


def segs(lib, packed=False, **kw):
    return lib.kda_fwd_segments(ctypes.byref(base_params(**kw)), int(packed))


def test_segment_plan(lib):
    # automatic: split only when the state launch has <= 128 workgroups (4 per chain)
    assert segs(lib, B=1, T=131072, H_qk=2, H_v=4) == 16
    assert segs(lib, B=1, T=131072, H_qk=16, H_v=32) == 2
    assert segs(lib, B=2, T=8192, H_qk=32, H_v=32) == 1
    assert segs(lib, B=1, T=2048, H_qk=1, H_v=1) == 2       # 32 chunks: segments of at least 16
    assert segs(lib, B=1, T=1024, H_qk=1, H_v=1) == 1
    # forced: at most one per chunk, and no empty segment
    assert segs(lib, B=1, T=200, H_qk=1, H_v=1, segments=7) == 4
    assert segs(lib, B=1, T=64 * 10, H_qk=1, H_v=1, segments=4) == 4     # 3 + 3 + 3 + 1 chunks
    assert segs(lib, B=1, T=64 * 9, H_qk=1, H_v=1, segments=6) == 5      # 2 chunks each: 5 segments
    assert segs(lib, B=2, T=4096, segments=1) == 1
    assert segs(lib, B=1, T=0, H_qk=1, H_v=1, segments=8) == 1
    # packed input never splits; invalid parameters give 0
    assert segs(lib, packed=True, B=1, T=131072, H_qk=2, H_v=4, segments=8) == 1
    assert segs(lib, B=2, T=100, segments=-3) == 0
    # segment jobs per launch stay within the pair limit
    assert segs(lib, B=1 << 18, T=64 * 8, H_qk=2, H_v=2, segments=8) == 4
    assert segs(lib, B=1 << 19, T=64 * 8, H_qk=4, H_v=4, segments=8) == 1


def test_workspace_holds_segment_scratch(lib):
    p1 = base_params(B=1, T=4096, H_qk=2, H_v=2, segments=1)
    p4 = base_params(B=1, T=4096, H_qk=2, H_v=2, segments=4)
    extra = lib.kda_fwd_workspace_size(ctypes.byref(p4)) - lib.kda_fwd_workspace_size(ctypes.byref(p1))
    assert extra == 3 * 2 * 4 * 128 * 128 * 4    # entry states, carries, maps: fp32 per (chain, segment)
    # the backward's two state passes share one scratch of the same size
    extra = lib.kda_bwd_workspace_size(ctypes.byref(p4)) - lib.kda_bwd_workspace_size(ctypes.byref(p1))
    assert extra == 3 * 2 * 4 * 128 * 128 * 4


def bwd_call(lib, p, drop=(), shift=None, ws=None, extra=None):
    ptrs = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, A_log=FAKE, dt_bias=FAKE, cu=None,
                h0=FAKE if p.init_state_dtype else None, dout=FAKE, dhT=None, dq=FAKE, dk=FAKE, dv=FAKE, dg=FAKE,
                dbeta=FAKE, dA=FAKE, ddt=FAKE, dh0=FAKE, ws=FAKE)
    ptrs.update(extra or {})
    for name in ((drop,) if isinstance(drop, str) else drop):
        ptrs[name] = None
    if shift:
        ptrs[shift] = ptrs[shift] + 2
    need = lib.kda_bwd_workspace_size(ctypes.byref(p))
    order = ["q", "k", "v", "g", "beta", "A_log", "dt_bias", "cu", "h0", "dout", "dhT", "dq", "dk", "dv", "dg",
             "dbeta", "dA", "ddt", "dh0", "ws"]
    args = [None if ptrs[n] is None else ctypes.c_void_p(ptrs[n]) for n in order]
    return lib.kda_bwd(ctypes.byref(p), *args, ctypes.c_size_t(need if ws is None else ws), None)


@pytest.mark.parametrize("case,code", [
    (dict(params=dict(K=64)), -2),
    (dict(params=dict(gate_mode=3)), -8),
    (dict(params=dict(flags=4)), -8),
    (dict(params=dict(gate_mode=kda.GATE_SAFE_SIGMOID, lower_bound=0.0)), -4),
    (dict(params=dict(gate_mode=kda.GATE_PREGATED), drop=("dA", "ddt")), -8),          # dt_bias given
    (dict(params=dict(gate_mode=kda.GATE_PREGATED), drop=("dt_bias", "dA")), -8),      # ddt_bias given
    (dict(params=dict(gate_mode=kda.GATE_PREGATED), drop=("dt_bias", "ddt")), -8),     # dA_log given
    (dict(drop="A_log"), -1),                                                          # softplus needs A_log
    (dict(params=dict(gate_mode=kda.GATE_SAFE_SIGMOID), drop="A_log"), -8),            # dA_log without A_log
    (dict(drop="q"), -1), (dict(drop="dout"), -1), (dict(drop="dq"), -1), (dict(drop="dk"), -1),
    (dict(drop="dv"), -1), (dict(drop="dg"), -1), (dict(drop="dbeta"), -1), (dict(drop="h0"), -1),
    (dict(shift="dout"), -5), (dict(shift="dg"), -5), (dict(shift="ddt"), -5),
    (dict(extra=dict(dhT=FAKE + 4)), -5), (dict(shift="dh0"), -5),
    (dict(ws=16), -6), (dict(drop="ws"), -6), (dict(shift="ws"), -5),
])
def test_bwd_entry_rejects_before_launch(lib, case, code):
    # only rejections: a valid call would launch, and these tests run without a GPU
    p = base_params(**case.get("params", {}))
    assert bwd_call(lib, p, case.get("drop", ()), case.get("shift"), case.get("ws"), case.get("extra")) == code, \
        kda.last_error()
    assert kda.last_error() != ""


def test_bwd_workspace_size(lib):
    size = lambda **kw: lib.kda_bwd_workspace_size(ctypes.byref(base_params(**kw)))
    assert size(K=64) == 0
    a, b = size(B=1, T=1000, H_qk=2, H_v=2), size(B=1, T=2000, H_qk=2, H_v=2)
    assert 0 < a < b
    # per (v-head, chunk) fp32 intermediates, plus per-v-head q/k gradient buffers with grouped heads
    mha, gva = size(B=2, T=640, H_qk=4, H_v=4), size(B=2, T=640, H_qk=2, H_v=4)
    assert gva - mha == 2 * 2 * 640 * 4 * 128 * 4
