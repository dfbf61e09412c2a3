"""Seeded random-shape sweep: 50 layers drawn from fixed seeds, each run
through the C ABI stage by stage and compared with the oracle on every
stage (routing and dispatch bit for bit, outputs within the tolerances of
tests/gpu_helpers.py).  The shapes cover one token, ragged token counts
around the 64- and 256-row tiles, d_model of 64 and 192, experts from 1 to
1024 (so that many experts stay empty), every gate family, both
activations and dtypes, capacity factors with drops, the residual and the
shared expert.  The sweep stops at the first failing case and names it.
"""
from __future__ import annotations

import random

import pytest

import oracle
import workloads
from workloads import Config
import sparse_mixture_experts_39_amd as moe
import tests.gpu_helpers as H
from tests.test_gpu_parity import check_all

pytestmark = pytest.mark.gpu

N_CASES = 50


def _draw(rng: random.Random, i: int) -> Config:
    while True:
        T = rng.choice([1, 2, 7, 63, 64, 65, 127, 255, 256, 257, 300, 511, 600])
        d = rng.choice([64, 128, 192, 256])
        F = rng.choice([64, 128, 192, 256])
        E = rng.choice([1, 2, 3, 5, 8, 16, 33, 64, 100, 256, 1024])
        gate = rng.choice(["softmax_topk", "softmax_full", "sigmoid_bias", "noisy_topk", "expert_choice", "hash",
                           "hierarchical"])
        act = rng.choice(["relu", "swiglu"])
        dt = rng.choice(["bf16", "f32"])
        k = rng.randint(1, min(E, 16))
        kw = dict(T=T, d=d, F=F, E=E, k=k, act_dtype=dt, act=act, gate=gate, seed=5000 + i,
                  residual=rng.random() < 0.5, logit_bias="zipf" if rng.random() < 0.3 else "none")
        if rng.random() < 0.4 or gate == "expert_choice":
            kw["capacity_factor"] = rng.choice([0.5, 1.0, 1.1, 1.25, 2.0])
        if gate == "sigmoid_bias":
            kw["sel_bias"] = True
        if act == "swiglu" and rng.random() < 0.2:
            kw.update(n_shared=1, F_shared=rng.choice([64, 128]))
        if gate == "hierarchical":
            groups = [g for g in range(1, min(E, 64) + 1) if E % g == 0 and E // g <= 64]
            if not groups:
                continue
            ng = rng.choice(groups)
            picks = [p for p in range(1, ng + 1) if k % p == 0 and k // p <= E // ng]
            if not picks:
                continue
            kw.update(n_groups=ng, group_top_k=rng.choice(picks))
        cfg = Config(f"sweep{i}", **kw)
        if moe.validate_config(H.bind_config(cfg)) == 0:
            return cfg


def test_seeded_random_shapes():
    rng = random.Random(20261203)
    cases = [_draw(rng, i) for i in range(N_CASES)]
    for i, cfg in enumerate(cases):
        H.log(f"[sweep {i}] {cfg}")
        inp = workloads.make_inputs(cfg)
        g = H.run_stages(cfg, H.to_device(inp))
        o = oracle.forward(cfg, inp)
        check_all(cfg, g, o)
