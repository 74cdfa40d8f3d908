"""GPU parity of the backward (kda_bwd, through the C ABI) against the fp64
oracle's gradients (the token-by-token adjoint, itself pinned by finite
differences and autograd).

Bar: every element finite, and
  * per-element gradients (dq, dk, dv, dg, dbeta, dh0):
        ||g_gpu - g_ref||_F / ||g_ref||_F <= 1e-3
    -- the relative bar of the fp32 final state, since the backward computes
    in fp32 throughout;
  * the gate-parameter gradients, which are sums over every token and
    channel (dA_log per head, ddt_bias per head and channel): the error
    relative to the absolute mass of the summed terms,
        ||g_gpu - g_ref||_F <= 1e-3 * ||sum |term| ||_F,
    the usual scale for a sum's rounding, since those sums cancel (by a
    factor of ~40 at strong decay) and their own value is no scale for it.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_act_amd import kda
from gated_delta_rule_act_amd import workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

GRAD_REL = 1e-3
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dA_log", "ddt_bias", "dh0")


def run_gpu_bwd(inp, d_out, dhT, segments=0):
    d = U.to_device(inp)
    dev_dout = U.bf16_dev(d_out)
    dev_dhT = None if dhT is None else torch.from_numpy(dhT).cuda()
    r = kda.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"], d["dt_bias"], inp.scale, dev_dout,
                lower_bound=inp.lower_bound, gate_mode=inp.gate_mode, initial_state=d["h0"], d_final_state=dev_dhT,
                cu_seqlens=d["cu_seqlens"], qk_l2norm=bool(inp.flags & W.FLAG_QK_L2NORM),
                beta_is_prob=bool(inp.flags & W.FLAG_BETA_IS_PROB), segments=segments)
    torch.cuda.synchronize()
    return {n: (None if t is None else t.cpu().numpy().astype(np.float64)) for n, t in r.items()}


def run_oracle_bwd(inp, d_out, dhT):
    f = oracle.bf16_to_f64
    return oracle.bwd(f(inp.q), f(inp.k), f(inp.v), f(inp.g), f(inp.beta), inp.A_log, inp.dt_bias, f(d_out),
                      None if dhT is None else dhT.astype(np.float64), scale=inp.scale,
                      lower_bound=inp.lower_bound, gate_mode=inp.gate_mode, flags=inp.flags,
                      initial_state=inp.initial_state_f64(), cu_seqlens=inp.cu_seqlens)


def sum_masses(inp, ref):
    """Absolute masses of the terms summed into ddt_bias [Hv,K] and dA_log [Hv]:
    ddt_bias = sum_t dg and dA_log = sum_{t,c} dg * (da/dA_log) / (da/dx)."""
    dg = ref["dg"]
    m_dt = np.abs(dg).sum(axis=(0, 1))
    if inp.gate_mode == W.GATE_PREGATED or inp.A_log is None:
        return m_dt, None
    x = oracle.bf16_to_f64(inp.g) + (0.0 if inp.dt_bias is None else inp.dt_bias.astype(np.float64)[None, None])
    if inp.gate_mode == W.GATE_SAFE_SIGMOID:
        ratio = x  # (lb s'(z) z) / (lb s'(z) e^A_log), z = e^A_log x
    else:
        sp = np.maximum(x, 0) + np.log1p(np.exp(-np.abs(x)))
        ratio = sp * (1 + np.exp(-x))  # softplus(x) / sigmoid(x)
    return m_dt, np.abs(dg * ratio).sum(axis=(0, 1, 3))


def compare(gpu, ref, what, inp):
    errs = {}
    m_dt, m_A = sum_masses(inp, ref)
    for n in NAMES:
        if gpu.get(n) is None:
            continue
        a, b = gpu[n], ref[n]
        assert np.isfinite(a).all(), (what, n, "non-finite")
        if n in ("ddt_bias", "dA_log"):
            m = m_dt if n == "ddt_bias" else m_A
            nm = np.linalg.norm(m)
            errs[n] = float(np.linalg.norm(a - b) / nm) if nm > 0 else float(np.linalg.norm(a - b))
        else:
            nb = np.linalg.norm(b)
            errs[n] = float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))
    U.log(f"    {what} {errs}")
    for n, e in errs.items():
        assert e <= GRAD_REL, (what, n, e)


def small(**kw):
    base = dict(B=2, T=300, Hqk=4, seed=301, init_state_dtype=W.STATE_F32)
    base.update(kw)
    return W.make_inputs(**base)


CASES = {
    "softplus": dict(),
    "safe_lb5_extremes": dict(gate_mode=W.GATE_SAFE_SIGMOID, lower_bound=-5.0, A_log_range=(-4.0, 6.0), g_std=3.0),
    "safe_lb1_gva": dict(gate_mode=W.GATE_SAFE_SIGMOID, lower_bound=-1.0, Hqk=2, Hv=6, T=200),
    "pregated": dict(gate_mode=W.GATE_PREGATED, pregated_range=(-1.0, 0.0)),
    "softplus_no_state": dict(init_state_dtype=W.STATE_NONE, T=257),
    "bf16_state": dict(init_state_dtype=W.STATE_BF16, T=150),
    "one_token": dict(T=1, B=3),
    "exact_chunks": dict(T=128, B=1, Hqk=2),
    "long_memory": dict(A_log_range=(-8.0, -6.0), T=400, B=1),
    "strong_decay": dict(A_log_range=(3.0, 6.0), g_std=3.0, T=200),
    "no_l2norm": dict(flags=0, qk_std=1.0 / np.sqrt(128), T=260),
    "beta_prob": dict(beta_prob=True, T=200),
    "safe_no_A_log": dict(gate_mode=W.GATE_SAFE_SIGMOID, lower_bound=-5.0, with_A_log=False, g_std=3.0, T=200),
    "softplus_no_dt_bias": dict(with_dt_bias=False, T=200),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_bwd_elementwise(name):
    inp = small(**CASES[name])
    d_out, dhT = W.make_grads(inp, seed=77)
    U.log(f"[gpu] bwd {name}: B={inp.B} T={inp.T} Hqk={inp.Hqk} Hv={inp.Hv} gate={inp.gate_mode}")
    compare(run_gpu_bwd(inp, d_out, dhT), run_oracle_bwd(inp, d_out, dhT), name, inp)


def test_bwd_without_final_state_gradient():
    inp = small(T=200)
    d_out, _ = W.make_grads(inp, seed=5, dhT_std=None)
    U.log("[gpu] bwd with d_final_state = None")
    compare(run_gpu_bwd(inp, d_out, None), run_oracle_bwd(inp, d_out, None), "no dhT", inp)


def test_bwd_packed():
    lengths = [1, 63, 64, 0, 65, 200]
    inp = W.make_inputs(B=1, T=None, Hqk=2, Hv=4, seed=19, lengths=lengths, init_state_dtype=W.STATE_F32)
    d_out, dhT = W.make_grads(inp, seed=8)
    U.log(f"[gpu] bwd packed {lengths}")
    gpu = run_gpu_bwd(inp, d_out, dhT)
    compare(gpu, run_oracle_bwd(inp, d_out, dhT), "packed", inp)
    # the empty sequence passes its final-state gradient straight through
    assert np.array_equal(gpu["dh0"][3], dhT[3].astype(np.float64))


def test_bwd_empty_input():
    inp = small(T=0, B=2)
    d_out, dhT = W.make_grads(inp, seed=3)
    gpu = run_gpu_bwd(inp, d_out, dhT)
    assert np.array_equal(gpu["dh0"], dhT.astype(np.float64))
    assert not gpu["dA_log"].any() and not gpu["ddt_bias"].any()


def test_bwd_medium_sampled():
    # several chunks per sequence at the model's head count, sampled pairs
    inp = W.make_inputs(B=2, T=2048, Hqk=8, seed=23, gate_mode=W.GATE_SAFE_SIGMOID, lower_bound=-5.0,
                        A_log_range=(-4.0, 6.0), g_std=3.0, init_state_dtype=W.STATE_F32)
    d_out, dhT = W.make_grads(inp, seed=29)
    U.log("[gpu] bwd B=2 T=2048 H=8")
    gpu = run_gpu_bwd(inp, d_out, dhT)
    ref = run_oracle_bwd(inp, d_out, dhT)
    compare(gpu, ref, "medium", inp)


def test_bwd_headline_workload_sampled():
    # the bench's backward configuration (B=2, T=8192, H=32, safe gate lb=-5),
    # checked on sampled (sequence, head) pairs: every gradient of the pair's
    # v-head (dq, dk of its q/k head: grouped heads are 1 here) against the
    # oracle on that pair alone, plus finiteness of every output
    inp = W.workload(3)
    d_out, dhT = W.make_grads(inp, seed=1003)
    U.log("[gpu] bwd workload 3 full size")
    gpu = run_gpu_bwd(inp, d_out, dhT)
    for n in NAMES:
        if gpu.get(n) is not None:
            assert np.isfinite(gpu[n]).all(), n
    f = oracle.bf16_to_f64
    for n, h in ((0, 0), (1, 31), (1, 7)):
        sl = lambda a: np.ascontiguousarray(a[n:n + 1, :, h:h + 1])
        ref = oracle.bwd(f(sl(inp.q)), f(sl(inp.k)), f(sl(inp.v)), f(sl(inp.g)),
                         f(np.ascontiguousarray(inp.beta[n:n + 1, :, h:h + 1])), inp.A_log[h:h + 1],
                         inp.dt_bias[h:h + 1], f(sl(d_out)), dhT[n:n + 1, h:h + 1].astype(np.float64),
                         scale=inp.scale, lower_bound=inp.lower_bound, gate_mode=inp.gate_mode, flags=inp.flags,
                         initial_state=inp.initial_state_f64()[n:n + 1, h:h + 1])
        errs = {}
        for name, a in (("dq", gpu["dq"][n:n + 1, :, h:h + 1]), ("dk", gpu["dk"][n:n + 1, :, h:h + 1]),
                        ("dv", gpu["dv"][n:n + 1, :, h:h + 1]), ("dg", gpu["dg"][n:n + 1, :, h:h + 1]),
                        ("dbeta", gpu["dbeta"][n:n + 1, :, h:h + 1]), ("dh0", gpu["dh0"][n:n + 1, h:h + 1])):
            b = ref[name]
            errs[name] = float(np.linalg.norm(a - b) / np.linalg.norm(b))
        U.log(f"    pair n={n} h={h} {errs}")
        for name, e in errs.items():
            assert e <= GRAD_REL, (n, h, name, e)


# Time segments of both state passes (dense input): (inputs, segments)
SEG_CASES = {
    "safe_lb5_seg4": (dict(B=2, T=1000, Hqk=2, Hv=4, gate_mode=W.GATE_SAFE_SIGMOID, lower_bound=-5.0,
                           A_log_range=(-4.0, 6.0), g_std=3.0), 4),
    "softplus_seg16_one_chunk_each": (dict(B=1, T=1000, Hqk=2), 16),
    "bf16_state_seg3": (dict(B=2, T=700, init_state_dtype=W.STATE_BF16), 3),
    "pregated_seg5": (dict(B=1, T=1280, gate_mode=W.GATE_PREGATED, pregated_range=(-2.0, 0.0)), 5),
    "no_state_seg2": (dict(B=2, T=513, init_state_dtype=W.STATE_NONE), 2),
    "long_memory_seg8": (dict(B=1, T=2048, Hqk=2, A_log_range=(-8.0, -6.0)), 8),
    "more_segments_than_chunks": (dict(B=1, T=200), 7),
}


@pytest.mark.parametrize("name", sorted(SEG_CASES))
def test_bwd_segments_elementwise(name):
    kw, segments = SEG_CASES[name]
    inp = small(**kw)
    d_out, dhT = W.make_grads(inp, seed=91)
    U.log(f"[gpu] bwd segments {name}: B={inp.B} T={inp.T} Hqk={inp.Hqk} Hv={inp.Hv} segments={segments}")
    compare(run_gpu_bwd(inp, d_out, dhT, segments=segments), run_oracle_bwd(inp, d_out, dhT), name, inp)


def test_bwd_segments_without_final_state_gradient():
    inp = small(B=1, T=900)
    d_out, _ = W.make_grads(inp, seed=6, dhT_std=None)
    U.log("[gpu] bwd segments=3, d_final_state = None")
    compare(run_gpu_bwd(inp, d_out, None, segments=3), run_oracle_bwd(inp, d_out, None), "seg no dhT", inp)


@pytest.mark.parametrize("segments", [2, 5, 32])
def test_bwd_segments_match_unsplit(segments):
    inp = small(B=1, T=64 * 40 + 17, Hqk=2, gate_mode=W.GATE_SAFE_SIGMOID, lower_bound=-1.0)
    d_out, dhT = W.make_grads(inp, seed=17)
    U.log(f"[gpu] bwd segments={segments} vs unsplit, T={inp.T}")
    a = run_gpu_bwd(inp, d_out, dhT, segments=1)
    b = run_gpu_bwd(inp, d_out, dhT, segments=segments)
    for n in NAMES:
        if a.get(n) is None:
            continue
        e = float(np.linalg.norm(a[n] - b[n]) / max(np.linalg.norm(a[n]), 1e-30))
        assert e <= GRAD_REL, (n, e)


def test_bwd_long_sequence_few_heads_sampled():
    # one GPU's share of the long grouped-head workload (T=131072, 2 q/k
    # heads, 4 v-heads, safe gate lb=-1): 4 chains, so the library cuts both
    # state passes into segments.  Checked on q/k head 1 with its 2 v-heads
    # against the oracle on that group alone.
    inp = W.workload(6)
    lib_segments = kda.segments_of(kda.make_params(B=inp.B, T=inp.T, H_qk=inp.Hqk, H_v=inp.Hv, num_seqs=inp.N,
                                                   scale=inp.scale, lower_bound=inp.lower_bound,
                                                   gate_mode=inp.gate_mode, flags=inp.flags))
    assert lib_segments > 1, lib_segments
    d_out, dhT = W.make_grads(inp, seed=1006)
    U.log(f"[gpu] bwd workload 6 full size, {lib_segments} segments")
    gpu = run_gpu_bwd(inp, d_out, dhT)
    for n in NAMES:
        if gpu.get(n) is not None:
            assert np.isfinite(gpu[n]).all(), n
    f = oracle.bf16_to_f64
    hq, hv = slice(1, 2), slice(2, 4)
    ref = oracle.bwd(f(np.ascontiguousarray(inp.q[:, :, hq])), f(np.ascontiguousarray(inp.k[:, :, hq])),
                     f(np.ascontiguousarray(inp.v[:, :, hv])), f(np.ascontiguousarray(inp.g[:, :, hv])),
                     f(np.ascontiguousarray(inp.beta[:, :, hv])), inp.A_log[hv], inp.dt_bias[hv],
                     f(np.ascontiguousarray(d_out[:, :, hv])), dhT[:, hv].astype(np.float64), scale=inp.scale,
                     lower_bound=inp.lower_bound, gate_mode=inp.gate_mode, flags=inp.flags, initial_state=None)
    errs = {}
    for name, a in (("dq", gpu["dq"][:, :, hq]), ("dk", gpu["dk"][:, :, hq]), ("dv", gpu["dv"][:, :, hv]),
                    ("dg", gpu["dg"][:, :, hv]), ("dbeta", gpu["dbeta"][:, :, hv]), ("dh0", gpu["dh0"][:, hv])):
        errs[name] = float(np.linalg.norm(a - ref[name]) / np.linalg.norm(ref[name]))
    U.log(f"    group hq=1 {errs}")
    for name, e in errs.items():
        assert e <= GRAD_REL, (name, e)
