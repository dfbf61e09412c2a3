"""Pins of the backward oracle (oracle/backward.py) to things other than itself.

* torch.autograd in float64 of the layer's forward, written out here from the
  forward definitions with the oracle's own routing held fixed (the top-k
  choice is a constant of the step; Shazeer et al. reading notes, section 2.1
  key points): every gradient of the hand-derived backward must match.
* Central finite differences of the oracle's own forward (float64 expert
  path, no intermediate rounding) for expert and shared-expert weights, which
  do not move the routing.
* Softmax gates: the logit gradient of a token sums to zero.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import backward as ob

SMALL = dict(T=40, d=16, F=24, E=6, k=2, act_dtype="f32")

CASES = {
    "swiglu_topk_resid": dict(act="swiglu", gate="softmax_topk", residual=True, seed=71),
    "relu_full_drops": dict(act="relu", gate="softmax_full", capacity_factor=1.0, residual=True,
                            logit_bias="zipf", seed=72),
    "swiglu_topk_drops": dict(act="swiglu", gate="softmax_topk", capacity_factor=0.8, seed=73),
    "swiglu_sigmoid_shared": dict(act="swiglu", gate="sigmoid_bias", sel_bias=True, n_shared=1, F_shared=20,
                                  seed=74),
    "swiglu_expert_choice": dict(act="swiglu", gate="expert_choice", capacity_factor=1.0, seed=75),
    "relu_hash": dict(act="relu", gate="hash", seed=76),
}


def _cfg(name):
    return workloads.Config(name, **SMALL, **CASES[name])


def _run(cfg):
    inp = workloads.make_inputs(cfg)
    fwd = oracle.forward(cfg, inp, round_intermediates=False)
    dy = workloads.make_output_grad(cfg)
    return inp, fwd, dy, ob.backward(cfg, inp, fwd, dy)


def _t(a):
    return torch.tensor(np.asarray(oracle._np(a), dtype=np.float64), dtype=torch.float64)


def _autograd(cfg, inp, fwd, dy):
    """Gradients of sum(out * dy) by torch.autograd, out written from the
    forward definitions with the oracle's routing."""
    x = _t(inp["x"]).requires_grad_()
    Wr = _t(inp["w_router"]).requires_grad_()
    b = (_t(inp["logit_bias"]) if "logit_bias" in inp else torch.zeros(cfg.E, dtype=torch.float64))
    b.requires_grad_()
    names = workloads.expert_tensor_names(cfg)
    W = {n: _t(inp[n]).requires_grad_() for n in names}
    shared = {n: _t(inp[n]).requires_grad_() for n in ("ws_gate", "ws_up", "ws_down") if n in inp}

    def mlp(v, w1, w3, w2):
        a = w1 @ v
        h = torch.nn.functional.silu(a) * (w3 @ v) if w3 is not None else torch.relu(a)
        return w2 @ h

    def expert(e, v):
        if cfg.act == "swiglu":
            return mlp(v, W["w_gate"][e], W["w_up"][e], W["w_down"][e])
        return mlp(v, W["w1"][e], None, W["w2"][e])

    ns = oracle.slots(cfg)
    idx = fwd["idx"].reshape(cfg.T, ns)
    sp = fwd["slot_pos"].reshape(cfg.T, ns)
    z = x @ Wr.T + b
    rows = []
    for t in range(cfg.T):
        sel = [(j, int(idx[t, j])) for j in range(ns) if idx[t, j] >= 0]
        es = [e for _, e in sel]
        if cfg.gate == "softmax_topk":
            g = torch.softmax(z[t, es], dim=0)
        elif cfg.gate in ("softmax_full", "expert_choice"):
            g = torch.softmax(z[t], dim=0)[es]
        elif cfg.gate == "sigmoid_bias":
            s = torch.sigmoid(z[t, es])
            g = s / s.sum()
        else:
            g = torch.ones(len(es), dtype=torch.float64)
        o = x[t] if cfg.residual else torch.zeros(cfg.d, dtype=torch.float64)
        for (j, e), gj in zip(sel, g):
            if sp[t, j] >= 0:
                o = o + gj * expert(e, x[t])
        if shared:
            o = o + mlp(x[t], shared["ws_gate"][0], shared["ws_up"][0], shared["ws_down"][0])
        rows.append(o)
    out = torch.stack(rows)
    loss = (out * _t(dy)).sum()
    leaves = [x, Wr, b] + [W[n] for n in names] + list(shared.values())
    gr = torch.autograd.grad(loss, leaves, allow_unused=True)
    res = dict(dx=gr[0], dw_router=gr[1], dlogit_bias=gr[2])
    for n, g in zip(names, gr[3:3 + len(names)]):
        res["d" + n] = g
    for n, g in zip(shared.keys(), gr[3 + len(names):]):
        res["d" + n] = g[0]
    return res, out.detach().numpy()


def _close(a, b, rtol):
    a = np.asarray(a, np.float64)
    b = np.asarray(b.detach().numpy() if isinstance(b, torch.Tensor) else b, np.float64)
    scale = max(np.abs(b).max(), 1e-30)
    return np.abs(a - b).max() / scale <= rtol


@pytest.mark.parametrize("name", list(CASES))
def test_backward_matches_autograd(name):
    cfg = _cfg(name)
    inp, fwd, dy, g = _run(cfg)
    ref, out = _autograd(cfg, inp, fwd, dy)
    # the written-out forward is the oracle's forward (fp32 router logits
    # against fp64 here: 1e-6 relative)
    assert _close(fwd["out"], out, 1e-6)
    for key, val in ref.items():
        if val is None:                     # hash gate: the router is not used
            assert key in ("dw_router", "dlogit_bias")
            assert np.abs(g[key]).max() == 0.0
            continue
        assert _close(g[key], val, 1e-6), key


def _loss(cfg, inp, dy):
    f = oracle.forward(cfg, inp, round_intermediates=False)
    return float(np.sum(f["out"] * oracle.act_to_f64(dy, "f32"))), f


@pytest.mark.parametrize("name", ["swiglu_topk_drops", "swiglu_sigmoid_shared", "relu_full_drops"])
def test_weight_gradients_match_finite_differences(name):
    cfg = _cfg(name)
    inp, fwd, dy, g = _run(cfg)
    rng = np.random.default_rng(5)
    names = list(workloads.expert_tensor_names(cfg)) + [n for n in ("ws_gate", "ws_up", "ws_down") if n in inp]
    checked = 0
    for n in names:
        W = inp[n]
        for _ in range(4):
            pos = tuple(int(rng.integers(0, s)) for s in W.shape)
            if n.startswith("ws") or int(fwd["offsets"][pos[0] + 1]) > int(fwd["offsets"][pos[0]]):
                checked += 1
            orig = W[pos].item()
            h = 1e-3
            W[pos] = orig + h
            lp, fp = _loss(cfg, inp, dy)
            up = W[pos].item()
            W[pos] = orig - h
            lm, fm = _loss(cfg, inp, dy)
            dn = W[pos].item()
            W[pos] = orig
            assert np.array_equal(fp["idx"], fwd["idx"]) and np.array_equal(fm["idx"], fwd["idx"])
            fd = (lp - lm) / (up - dn)
            key = "d" + n
            an = g[key][pos] if not n.startswith("ws") else g[key][pos[1:]]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (n, pos, fd, an)
    assert checked >= 8


@pytest.mark.parametrize("name", ["swiglu_topk_resid", "relu_full_drops", "swiglu_expert_choice"])
def test_softmax_logit_gradients_sum_to_zero(name):
    cfg = _cfg(name)
    _, _, _, g = _run(cfg)
    dz = g["dz"]
    assert np.abs(dz.sum(axis=1)).max() <= 1e-12 * max(1.0, np.abs(dz).max())
    assert np.abs(dz).max() > 0
