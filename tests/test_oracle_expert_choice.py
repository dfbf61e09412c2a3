"""Pins of the oracle's expert-choice routing (each expert takes its top-C
tokens by router probability): equal loads, a brute-force selection on the
oracle's own scores, the scores against an fp64 softmax, the all-ties case,
and the combine of tokens no expert took."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import Config


def _cfg(**kw):
    base = dict(T=96, d=64, F=64, E=6, k=2, act_dtype="f32", act="swiglu", gate="expert_choice", seed=7)
    base.update(kw)
    return Config("ec", **base)


def test_every_expert_takes_exactly_C_tokens():
    for T, E, k, cf in [(96, 6, 2, 0.0), (50, 8, 1, 1.0), (40, 4, 3, 1.5), (10, 8, 4, 4.0)]:
        cfg = _cfg(T=T, E=E, k=k, capacity_factor=cf)
        C = oracle.capacity(cfg)
        assert C == min(T, math.ceil((cf if cf > 0 else 1.0) * T * k / E))
        inp = workloads.make_inputs(cfg)
        r = oracle.route(cfg, inp["x"], inp["w_router"])
        taken = r["idx"] >= 0
        np.testing.assert_array_equal(taken.sum(axis=0), np.full(E, C))
        for e in range(E):
            assert (r["idx"][taken[:, e], e] == e).all()


def test_selection_brute_force_on_the_scores():
    cfg = _cfg()
    inp = workloads.make_inputs(cfg)
    r = oracle.route(cfg, inp["x"], inp["w_router"])
    S = r["keys"].astype(np.float64)
    C = oracle.capacity(cfg)
    for e in range(cfg.E):
        order = sorted(range(cfg.T), key=lambda t: (-S[t, e], t))
        chosen = set(order[:C])
        got = set(np.nonzero(r["idx"][:, e] >= 0)[0].tolist())
        assert got == chosen, e
        for t in chosen:
            assert r["gates"][t, e] == pytest.approx(S[t, e], rel=0, abs=0)


def test_scores_are_the_router_softmax():
    cfg = _cfg()
    inp = workloads.make_inputs(cfg)
    r = oracle.route(cfg, inp["x"], inp["w_router"])
    z = inp["x"].double().numpy() @ inp["w_router"].double().numpy().T
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(r["keys"], p, rtol=2e-6, atol=1e-9)
    np.testing.assert_allclose(r["P"], p.mean(axis=0), rtol=2e-6)


def test_all_ties_take_the_first_tokens():
    cfg = _cfg(T=20, E=4, k=1)
    inp = workloads.make_inputs(cfg)
    inp["w_router"] = torch.zeros_like(inp["w_router"])
    r = oracle.route(cfg, inp["x"], inp["w_router"])
    assert (r["keys"] == np.float32(0.25)).all()
    C = oracle.capacity(cfg)
    for e in range(cfg.E):
        np.testing.assert_array_equal(np.nonzero(r["idx"][:, e] >= 0)[0], np.arange(C))


def test_untaken_tokens_pass_through_and_stats_are_balanced():
    cfg = _cfg(T=64, E=8, k=1, residual=True)
    inp = workloads.make_inputs(cfg)
    o = oracle.forward(cfg, inp)
    taken = (o["idx"] >= 0).any(axis=1)
    assert (~taken).any(), "expected some token that no expert took"
    x = inp["x"].double().numpy()
    np.testing.assert_allclose(o["out"][~taken], x[~taken], rtol=0, atol=0)
    np.testing.assert_allclose(o["f"], 1.0 / cfg.E, rtol=1e-12)
    assert o["imbalance"] == pytest.approx(1.0)
    assert o["aux"] == pytest.approx(o["P"].sum(), rel=1e-12)
    assert o["P"].sum() == pytest.approx(1.0, rel=1e-6)


def test_balance_statistics_under_expert_choice():
    """Importance of expert e is the sum of its C largest probabilities (a
    column sort of the scores); over one sequence of all T tokens every
    expert's f is C / (T k) and the probabilities of a token sum to 1, so the
    balance term is E C / (T k) in closed form (1 when C = T k / E)."""
    for T, E, k, cf in [(96, 6, 2, 0.0), (64, 8, 1, 1.5), (40, 4, 3, 1.0)]:
        cfg = _cfg(T=T, E=E, k=k, capacity_factor=cf)
        inp = workloads.make_inputs(cfg)
        r = oracle.route(cfg, inp["x"], inp["w_router"], want_probs=True)
        C = oracle.capacity(cfg)
        b = oracle.balance(cfg, r)
        S = r["keys"].astype(np.float64)
        imp = np.array([np.sort(S[:, e])[::-1][:C].sum() for e in range(E)])
        np.testing.assert_allclose(b["importance"], imp, rtol=1e-12)
        assert b["seq_aux"] == pytest.approx(E * C / (T * k), rel=1e-6)
        assert np.isnan(b["load"]).all()
