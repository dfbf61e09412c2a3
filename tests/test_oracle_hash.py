"""Pins of the oracle's hash routing (CS336 lecture 4 notes, section 4: a
fixed hash of the token picks its experts) and of the counter-based generator
it hashes with: Philox4x32-10 against its published known-answer vectors,
equal ids meeting equal experts, the selection against a brute-force sort of
the keys, k = E against the dense sum of every expert, balanced loads over
many distinct ids, and P equal to the selection frequencies."""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.brute as brute
import workloads
from workloads import Config

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")


def _cfg(**kw):
    base = dict(T=200, d=64, F=64, E=8, k=2, act_dtype="f32", act="swiglu", gate="hash", seed=31)
    base.update(kw)
    return Config("hash", **base)


def test_philox_known_answer_vectors():
    kat = json.load(open(GOLDEN))
    for v in kat["vectors"]:
        out = oracle.philox4x32_10([int(w, 16) for w in v["ctr"]], [int(w, 16) for w in v["key"]])
        assert [f"{int(w):08x}" for w in out] == v["out"]


def test_hash_key_is_the_top_24_bits_of_the_stream_word():
    seed, off = 0x1234_5678_9ABC, 5
    for i in (0, 1, 2, 3, 4, 7, 1 << 33, (1 << 40) + 3):
        g = i >> 2
        w = oracle.philox4x32_10([g & 0xFFFFFFFF, g >> 32, off & 0xFFFFFFFF, off >> 32],
                                 [seed & 0xFFFFFFFF, seed >> 32])[i & 3]
        assert oracle.hash_key(seed, off, i) == float(int(w) >> 8)


def test_equal_ids_meet_equal_experts_and_selection_is_the_sorted_keys():
    cfg = _cfg(T=300, E=16, k=3)
    inp = workloads.make_inputs(cfg)
    ids = inp["token_ids"].numpy()
    r = oracle.route(cfg, inp["x"], inp["w_router"], token_ids=ids, want_probs=True)
    assert len(np.unique(ids)) < len(ids), "Zipf ids should repeat"
    for u in np.unique(ids):
        rows = r["idx"][ids == u]
        assert (rows == rows[0]).all()
    for t in range(cfg.T):
        keys = [oracle.hash_key(cfg.seed, 0, int(ids[t]) * cfg.E + e) for e in range(cfg.E)]
        order = sorted(range(cfg.E), key=lambda e: (-keys[e], e))
        assert list(r["idx"][t]) == order[:cfg.k]
        np.testing.assert_array_equal(r["keys"][t], np.float32(keys))
    assert (r["gates"] == 1.0).all()
    # P is the selection frequency, 1/k per selected expert
    f = np.bincount(r["idx"].reshape(-1), minlength=cfg.E) / (cfg.T * cfg.k)
    np.testing.assert_allclose(r["P"], f, rtol=1e-12)


def test_seed_and_offset_change_the_mapping():
    cfg = _cfg(T=64, E=32, k=1)
    ids = np.arange(64, dtype=np.int32)
    x = torch.zeros(64, cfg.d)
    w = torch.zeros(cfg.E, cfg.d)
    a = oracle.route(cfg, x, w, token_ids=ids)["idx"]
    b = oracle.route(cfg.replace(seed=32), x, w, token_ids=ids)["idx"]
    c = oracle.route(cfg, x, w, token_ids=ids, noise_offset=1)["idx"]
    assert (a != b).any() and (a != c).any()


def test_distinct_ids_spread_evenly():
    """T distinct ids, top-1 of 16: each expert's count is binomial(T, 1/16);
    all 16 lie within 5 standard deviations and a chi-square over the experts
    stays below its 0.1 % critical value (37.7 at 15 degrees of freedom)."""
    T, E = 16000, 16
    cfg = _cfg(T=T, E=E, k=1)
    ids = np.arange(T, dtype=np.int32) * 7 + 3
    r = oracle.route(cfg, torch.zeros(T, cfg.d), torch.zeros(E, cfg.d), token_ids=ids)
    n = np.bincount(r["idx"].reshape(-1), minlength=E)
    mu, sd = T / E, math.sqrt(T * (1 / E) * (1 - 1 / E))
    assert np.abs(n - mu).max() < 5 * sd
    assert ((n - mu) ** 2 / mu).sum() < 37.7


def test_k_equals_E_is_the_sum_of_every_expert():
    cfg = _cfg(T=24, E=4, k=4, residual=True)
    inp = workloads.make_inputs(cfg)
    o = oracle.forward(cfg, inp, round_intermediates=False)
    x64 = inp["x"].double().numpy()
    want = x64.copy()
    for e in range(cfg.E):
        want += brute.expert_dense(cfg, x64, inp["w_gate"][e].numpy(), inp["w_up"][e].numpy(),
                                   inp["w_down"][e].numpy())
    np.testing.assert_allclose(o["out"], want, rtol=1e-9, atol=1e-9)
