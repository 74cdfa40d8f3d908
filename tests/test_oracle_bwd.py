"""Pins of the oracle's gradients (CPU only).

The backward oracle is the token-by-token adjoint of the recurrence.  It is
pinned to things other than itself:
  * its fp64-input forward equals the bf16 forward oracle exactly on
    bf16-representable inputs (so the function being differentiated is the
    pinned forward);
  * central finite differences of that forward, element by element, on tiny
    problems (every gate mode, grouped heads, packed sequences with an empty
    one, L2 norm on and off, beta as logits or probabilities, with and
    without initial state and final-state gradient);
  * torch fp64 autograd through a recurrence written independently here.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_act_amd import workloads as W

STEP = 2.0 ** -12  # finite-difference step; A_log and dt_bias sit on a 2^-12 grid, so x +- STEP is exact in fp32


def draw(seed, B=1, T=7, Hqk=1, Hv=2, K=4, V=3, gate_mode=oracle.GATE_SOFTPLUS, flags=oracle.FLAG_QK_L2NORM,
         lengths=None, with_h0=True):
    rng = np.random.default_rng(seed)
    cu = None
    if lengths is not None:
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
        T = int(cu[-1])
    N = B if cu is None else len(lengths)
    d = dict(q=rng.normal(size=(B, T, Hqk, K)), k=rng.normal(size=(B, T, Hqk, K)), v=rng.normal(size=(B, T, Hv, V)))
    if gate_mode == oracle.GATE_PREGATED:
        d["g"] = rng.uniform(-1.0, 0.0, size=(B, T, Hv, K))
        d["A_log"], d["dt_bias"] = None, None
    else:
        d["g"] = rng.normal(size=(B, T, Hv, K))
        d["A_log"] = (np.round(rng.uniform(-1.0, 1.0, size=Hv) * 4096) / 4096).astype(np.float32)
        d["dt_bias"] = (np.round(rng.normal(size=(Hv, K)) * 0.3 * 4096) / 4096).astype(np.float32)
    d["beta"] = rng.uniform(0.05, 0.95, size=(B, T, Hv)) if flags & oracle.FLAG_BETA_IS_PROB \
        else rng.normal(size=(B, T, Hv))
    if not flags & oracle.FLAG_QK_L2NORM:
        d["q"] *= 0.4
        d["k"] *= 0.4
    d["h0"] = rng.normal(size=(N, Hv, V, K)) * 0.3 if with_h0 else None
    d["W_o"] = rng.normal(size=(B, T, Hv, V))
    d["W_s"] = rng.normal(size=(N, Hv, V, K))
    kw = dict(scale=1.0 / math.sqrt(K), lower_bound=-2.0, gate_mode=gate_mode, flags=flags, cu_seqlens=cu)
    return d, kw


def loss(d, kw):
    out, hT = oracle.fwd_f64(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"], d["dt_bias"],
                             initial_state=d["h0"], **kw)
    return float((out * d["W_o"]).sum() + (hT * d["W_s"]).sum())


def grads(d, kw):
    return oracle.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["A_log"], d["dt_bias"], d["W_o"], d["W_s"],
                      initial_state=d["h0"], **kw)


def fd_check(d, kw, rtol=2e-6, sample=None, seed=0):
    """Central differences of every input element (or of `sample` random
    elements per input) against the oracle's gradients."""
    rng = np.random.default_rng(seed)
    gr = grads(d, kw)
    names = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta")]
    if d["h0"] is not None:
        names.append(("h0", "dh0"))
    if d["A_log"] is not None:
        names += [("A_log", "dA_log"), ("dt_bias", "ddt_bias")]
    worst = 0.0
    for x, dx in names:
        arr = d[x]
        flat = arr.reshape(-1)
        idx = np.arange(flat.size) if sample is None or flat.size <= sample else \
            rng.choice(flat.size, size=sample, replace=False)
        num = np.empty(idx.size)
        for j, i in enumerate(idx):
            old = flat[i]
            flat[i] = old + STEP
            lp = loss(d, kw)
            flat[i] = old - STEP
            lm = loss(d, kw)
            flat[i] = old
            num[j] = (lp - lm) / (2 * STEP)
        ana = gr[dx].reshape(-1)[idx]
        scale = max(1.0, np.abs(num).max())
        err = np.abs(num - ana).max() / scale
        worst = max(worst, err)
        assert err <= rtol, (x, err, num[:6], ana[:6])
    return worst


FD_CASES = {
    "softplus": dict(),
    "safe": dict(gate_mode=oracle.GATE_SAFE_SIGMOID),
    "pregated": dict(gate_mode=oracle.GATE_PREGATED),
    "no_l2norm": dict(flags=0),
    "beta_prob": dict(flags=oracle.FLAG_QK_L2NORM | oracle.FLAG_BETA_IS_PROB),
    "gva3_no_h0": dict(Hqk=1, Hv=3, with_h0=False),
    "packed_with_empty": dict(lengths=[3, 0, 4], gate_mode=oracle.GATE_SAFE_SIGMOID),
    "mha_two_heads": dict(Hqk=2, Hv=2, B=2, T=5),
}


@pytest.mark.parametrize("name", sorted(FD_CASES))
def test_gradients_match_finite_differences(name):
    d, kw = draw(17 + len(name), **FD_CASES[name])
    fd_check(d, kw)


def test_gradients_across_checkpoint_blocks():
    # 600 tokens: the adjoint recomputes states from three 256-token checkpoints
    d, kw = draw(23, T=600, K=3, V=2, gate_mode=oracle.GATE_SAFE_SIGMOID)
    fd_check(d, kw, sample=40, seed=1)


def test_fwd_f64_equals_bf16_forward():
    for mode in (oracle.GATE_SOFTPLUS, oracle.GATE_SAFE_SIGMOID, oracle.GATE_PREGATED):
        inp = W.make_inputs(B=1, T=None, Hqk=2, Hv=4, K=16, V=8, seed=5, lengths=[9, 0, 20], gate_mode=mode,
                            lower_bound=-3.0, init_state_dtype=W.STATE_F32,
                            pregated_range=(-1.0, 0.0))
        kw = dict(scale=inp.scale, lower_bound=inp.lower_bound, gate_mode=mode, flags=inp.flags,
                  cu_seqlens=inp.cu_seqlens)
        o1, s1 = oracle.fwd(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.A_log, inp.dt_bias,
                            initial_state=inp.initial_state_f64(), **kw)
        f = oracle.bf16_to_f64
        o2, s2 = oracle.fwd_f64(f(inp.q), f(inp.k), f(inp.v), f(inp.g), f(inp.beta), inp.A_log, inp.dt_bias,
                                initial_state=inp.initial_state_f64(), **kw)
        assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


def torch_forward(q, k, v, g, beta, A_log, dt_bias, h0, scale, lower_bound, gate_mode, G):
    """An independent statement of the recurrence, for autograd: per v-head,
    S_t = (S_{t-1} diag(e^a))(I - b k k^T) + b v k^T and o_t = scale S_t q."""
    B, T, Hqk, K = q.shape
    Hv, V = v.shape[2], v.shape[3]
    qn = q / torch.sqrt((q * q).sum(-1, keepdim=True) + 1e-6)
    kn = k / torch.sqrt((k * k).sum(-1, keepdim=True) + 1e-6)
    x = g + dt_bias[None, None]
    if gate_mode == oracle.GATE_SOFTPLUS:
        a = -torch.exp(A_log)[None, None, :, None] * torch.nn.functional.softplus(x)
    else:
        a = lower_bound * torch.sigmoid(torch.exp(A_log)[None, None, :, None] * x)
    b = torch.sigmoid(beta)
    outs, finals = [], []
    eye = torch.eye(K, dtype=q.dtype)
    for bb in range(B):
        o_b, f_b = [], []
        for h in range(Hv):
            S = h0[bb, h]
            o_h = []
            for t in range(T):
                kk = kn[bb, t, h // G]
                S = (S * torch.exp(a[bb, t, h])[None, :]) @ (eye - b[bb, t, h] * torch.outer(kk, kk)) \
                    + b[bb, t, h] * torch.outer(v[bb, t, h], kk)
                o_h.append(scale * S @ qn[bb, t, h // G])
            o_b.append(torch.stack(o_h))
            f_b.append(S)
        outs.append(torch.stack(o_b, dim=1))
        finals.append(torch.stack(f_b))
    return torch.stack(outs), torch.stack(finals)


@pytest.mark.parametrize("gate_mode", [oracle.GATE_SOFTPLUS, oracle.GATE_SAFE_SIGMOID])
def test_gradients_match_torch_autograd(gate_mode):
    d, kw = draw(3, B=2, T=12, Hqk=2, Hv=4, K=8, V=6, gate_mode=gate_mode)
    gr = grads(d, kw)
    tt = {n: torch.tensor(np.asarray(d[n], dtype=np.float64), requires_grad=True)
          for n in ("q", "k", "v", "g", "beta", "A_log", "dt_bias", "h0")}
    out, hT = torch_forward(tt["q"], tt["k"], tt["v"], tt["g"], tt["beta"], tt["A_log"], tt["dt_bias"], tt["h0"],
                            kw["scale"], kw["lower_bound"], gate_mode, G=2)
    L = (out * torch.tensor(d["W_o"])).sum() + (hT * torch.tensor(d["W_s"])).sum()
    L.backward()
    for n, dn in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"), ("A_log", "dA_log"),
                  ("dt_bias", "ddt_bias"), ("h0", "dh0")):
        np.testing.assert_allclose(gr[dn], tt[n].grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=n)


def test_zero_write_strength_leaves_v_without_gradient():
    # beta = 0 (probabilities): values never enter the state, so dv = 0 exactly
    d, kw = draw(9, T=6, flags=oracle.FLAG_QK_L2NORM | oracle.FLAG_BETA_IS_PROB)
    d["beta"][:] = 0.0
    gr = grads(d, kw)
    assert np.all(gr["dv"] == 0.0)
    assert np.all(gr["dbeta"] != 0.0)
