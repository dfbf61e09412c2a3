"""Pins of the oracle's two-level (hierarchical) gate (Shazeer notes,
appendix B: a primary gate picks groups, a secondary gate picks experts inside
each picked group).  Special cases that reduce to the flat softmax top-k gate
(one group; one expert per group), a brute-force sort in fp64, gates and
probabilities that are distributions, and the whole layer against the dense
sum over groups and experts of gate products."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import oracle.brute as brute
import workloads
from workloads import Config


def _cfg(**kw):
    base = dict(T=60, d=64, F=64, E=16, k=4, act_dtype="f32", act="swiglu", gate="hierarchical", n_groups=4,
                group_top_k=2, seed=41)
    base.update(kw)
    return Config("hier", **base)


def _route(cfg, inp):
    return oracle.route(cfg, inp["x"], inp["w_router"], logit_bias=inp.get("logit_bias"),
                        w_group_router=inp["w_group_router"], want_probs=True)


def test_one_group_is_the_flat_softmax_topk_gate():
    cfg = _cfg(n_groups=1, group_top_k=1, k=3)
    inp = workloads.make_inputs(cfg)
    r = _route(cfg, inp)
    flat = cfg.replace(gate="softmax_topk", n_groups=0, group_top_k=0)
    f = oracle.route(flat, inp["x"], inp["w_router"], want_probs=True)
    np.testing.assert_array_equal(r["idx"], f["idx"])
    np.testing.assert_allclose(r["gates"], f["gates"], rtol=1e-12)
    np.testing.assert_allclose(r["P"], f["P"], rtol=1e-12)


def test_one_expert_per_group_is_top_k_of_the_primary_logits():
    cfg = _cfg(E=8, n_groups=8, group_top_k=2, k=2)
    inp = workloads.make_inputs(cfg)
    r = _route(cfg, inp)
    flat = cfg.replace(gate="softmax_topk", n_groups=0, group_top_k=0)
    f = oracle.route(flat, inp["x"], inp["w_group_router"], want_probs=True)
    np.testing.assert_array_equal(r["idx"], f["idx"])
    np.testing.assert_allclose(r["gates"], f["gates"], rtol=1e-12)
    np.testing.assert_allclose(r["P"], f["P"], rtol=1e-12)


@pytest.mark.parametrize("A,KP,k", [(4, 2, 4), (8, 3, 3), (2, 2, 8), (16, 1, 1)])
def test_brute_force_sort_and_gate_products(A, KP, k):
    cfg = _cfg(E=32, n_groups=A, group_top_k=KP, k=k)
    inp = workloads.make_inputs(cfg)
    r = _route(cfg, inp)
    z = r["logits"].astype(np.float64)
    B, KS = cfg.E // A, k // KP
    for t in range(cfg.T):
        # groups by the fp32 primary logits, descending, lower index first
        order = sorted(range(A), key=lambda g: (-float(r_zp(inp, t, g)), g))
        groups = order[:KP]
        want_idx, want_g = [], []
        ep = np.exp([float(r_zp(inp, t, g)) for g in groups] - np.max([float(r_zp(inp, t, g)) for g in groups]))
        gp = ep / ep.sum()
        for j, g in enumerate(groups):
            members = sorted(range(g * B, (g + 1) * B), key=lambda e: (-float(r["keys"][t, e]), e))[:KS]
            zs = np.array([z[t, e] for e in members])
            es = np.exp(zs - zs.max())
            gs = es / es.sum()
            want_idx += members
            want_g += list(gp[j] * gs)
        assert list(r["idx"][t]) == want_idx
        np.testing.assert_allclose(r["gates"][t], want_g, rtol=1e-12)
        assert abs(r["gates"][t].sum() - 1.0) < 1e-12
    np.testing.assert_allclose(r["probs"].sum(axis=1), 1.0, rtol=1e-12)


def r_zp(inp, t, g):
    """fp32 primary logit: the oracle's canonical fp32 dot product, read back
    through a one-expert-per-group flat routing of the same rows."""
    x = inp["x"][t:t + 1]
    w = inp["w_group_router"][g:g + 1]
    cfg = Config("one", T=1, d=x.shape[1], F=64, E=1, k=1, act_dtype="f32", act="swiglu", gate="softmax_topk")
    return oracle.route(cfg, x, w)["logits"][0, 0]


def test_layer_is_the_dense_sum_of_gate_products():
    cfg = _cfg(T=20, E=8, n_groups=2, group_top_k=2, k=4, residual=True)
    inp = workloads.make_inputs(cfg)
    o = oracle.forward(cfg, inp, round_intermediates=False)
    r = _route(cfg, inp)
    x64 = inp["x"].double().numpy()
    G = np.zeros((cfg.T, cfg.E))
    for t in range(cfg.T):
        for j in range(cfg.k):
            G[t, r["idx"][t, j]] += r["gates"][t, j]
    want = x64.copy()
    for e in range(cfg.E):
        want += G[:, e:e + 1] * brute.expert_dense(cfg, x64, inp["w_gate"][e].numpy(), inp["w_up"][e].numpy(),
                                                   inp["w_down"][e].numpy())
    np.testing.assert_allclose(o["out"], want, rtol=1e-9, atol=1e-9)
