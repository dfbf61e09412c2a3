"""Pins of the oracle's balance and stability statistics (router z-loss,
Shazeer's importance and load with their CV^2, the sequence-wise balance
term, the auxiliary-loss-free bias step) against closed forms, a Monte-Carlo
simulation of the load estimator's definition, and brute force on tiny
inputs."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import workloads
from workloads import Config


def _r(logits, idx, gates, probs=None, keys=None, noise_scale=None):
    logits = np.asarray(logits, np.float32)
    T, E = logits.shape
    r = dict(logits=logits, keys=np.asarray(logits if keys is None else keys, np.float32),
             idx=np.asarray(idx, np.int32), gates=np.asarray(gates, np.float64),
             probs=np.asarray(np.full((T, E), 1.0 / E) if probs is None else probs, np.float64))
    if noise_scale is not None:
        r["noise_scale"] = np.asarray(noise_scale, np.float32)
    return r


def _cfg(T, E, k, gate="softmax_topk"):
    return Config("bal", T=T, d=64, F=64, E=E, k=k, act_dtype="f32", act="swiglu", gate=gate, seed=1)


def test_z_loss_closed_forms():
    # zero logits: log sum exp = ln E
    E = 8
    b = oracle.balance(_cfg(3, E, 1), _r(np.zeros((3, E)), [[0]] * 3, [[1.0]] * 3))
    assert b["z_loss"] == pytest.approx(math.log(E) ** 2, rel=1e-12)
    # constant logits c: (c + ln E)^2
    b = oracle.balance(_cfg(2, E, 1), _r(np.full((2, E), 2.5), [[0]] * 2, [[1.0]] * 2))
    assert b["z_loss"] == pytest.approx((2.5 + math.log(E)) ** 2, rel=1e-12)
    # two experts with logits (ln 3, 0): ln(3 + 1) = ln 4
    b = oracle.balance(_cfg(1, 2, 1), _r([[math.log(3.0), 0.0]], [[0]], [[1.0]]))
    assert b["z_loss"] == pytest.approx(math.log(4.0) ** 2, rel=1e-6)
    # mean over tokens: tokens with lse 0 (one expert, logit 0) and 3
    b = oracle.balance(_cfg(2, 1, 1), _r([[0.0], [3.0]], [[0], [0]], [[1.0], [1.0]]))
    assert b["z_loss"] == pytest.approx((0.0 + 9.0) / 2.0, rel=1e-12)


def test_importance_cv2_closed_forms():
    T, E = 16, 4
    # every token on expert 0 with gate 1: importance (T, 0, 0, 0), CV^2 = E - 1
    b = oracle.balance(_cfg(T, E, 1), _r(np.zeros((T, E)), [[0]] * T, [[1.0]] * T))
    np.testing.assert_array_equal(b["importance"], [T, 0, 0, 0])
    assert b["importance_cv2"] == pytest.approx(E - 1, rel=1e-12)
    # round robin with equal gates: perfectly balanced
    idx = [[t % E] for t in range(T)]
    b = oracle.balance(_cfg(T, E, 1), _r(np.zeros((T, E)), idx, [[1.0]] * T))
    assert b["importance_cv2"] == 0.0
    # k = 2, gates (0.75, 0.25) always on experts (1, 2): importance (0, 12, 4, 0)
    b = oracle.balance(_cfg(T, E, 2), _r(np.zeros((T, E)), [[1, 2]] * T, [[0.75, 0.25]] * T))
    v = np.array([0.0, 12.0, 4.0, 0.0])
    assert b["importance_cv2"] == pytest.approx(v.var() / v.mean() ** 2, rel=1e-12)


def _kth_excluding(h, k, i):
    others = sorted((h[j] for j in range(len(h)) if j != i), reverse=True)
    return others[k - 1]


def test_load_estimator_matches_its_definition_by_simulation():
    """P(x, i) is the chance that expert i is still chosen when only its own
    noise is drawn again (Shazeer, Load(X)): simulate that draw."""
    rng = np.random.default_rng(5)
    E, k = 6, 2
    z = rng.normal(size=E).astype(np.float32)
    scale = (0.3 + rng.random(E)).astype(np.float32)
    h = (z + rng.normal(size=E).astype(np.float32) * scale).astype(np.float32)
    top = list(np.argsort(-h.astype(np.float64), kind="stable")[:k])
    b = oracle.balance(_cfg(1, E, k, "noisy_topk"),
                       _r([z], [top], [[0.5, 0.5]], keys=[h], noise_scale=[scale]))
    n = 400_000
    for i in range(E):
        thr = _kth_excluding([float(v) for v in h], k, i)
        eps = rng.normal(size=n)
        freq = np.mean(z[i] + eps * scale[i] > thr)
        sd = math.sqrt(max(freq * (1 - freq), 1e-12) / n)
        assert abs(b["load"][i] - freq) < 5 * sd + 1e-4, (i, b["load"][i], freq)


def test_load_special_cases():
    E, k = 4, 1
    z = np.array([[0.0, 0.0, 0.0, 0.0]], np.float32)
    h = np.array([[1.0, 0.5, 0.0, -0.5]], np.float32)
    # huge noise scale: every expert's chance tends to Phi(0) = 1/2
    b = oracle.balance(_cfg(1, E, k, "noisy_topk"), _r(z, [[0]], [[1.0]], keys=h, noise_scale=np.full((1, E), 1e30)))
    np.testing.assert_allclose(b["load"], 0.5, atol=1e-12)
    assert b["load_cv2"] == pytest.approx(0.0, abs=1e-20)
    # expert 0 selected with clean logit exactly at the runner-up score: Phi(0)
    z2 = np.array([[0.5, -9.0, -9.0, -9.0]], np.float32)
    b = oracle.balance(_cfg(1, E, k, "noisy_topk"), _r(z2, [[0]], [[1.0]], keys=h, noise_scale=np.ones((1, E))))
    assert b["load"][0] == pytest.approx(0.5, abs=1e-12)
    # an unselected expert whose clean logit is one scale above the winner's score: Phi(1)
    z3 = np.array([[0.0, 2.0, 0.0, 0.0]], np.float32)
    b = oracle.balance(_cfg(1, E, k, "noisy_topk"), _r(z3, [[0]], [[1.0]], keys=h, noise_scale=np.ones((1, E))))
    assert b["load"][1] == pytest.approx(0.8413447460685429, abs=1e-12)
    # k = E: every expert is always chosen
    b = oracle.balance(_cfg(1, E, E, "noisy_topk"),
                       _r(z, [[0, 1, 2, 3]], [[0.25] * 4], keys=h, noise_scale=np.ones((1, E))))
    np.testing.assert_array_equal(b["load"], 1.0)


def test_seq_aux_closed_forms_and_batch_limit():
    E, L = 2, 4
    T = 2 * L
    probs = np.zeros((T, E))
    probs[:L, 0] = 1.0
    probs[L:, 1] = 1.0
    idx = [[0]] * L + [[1]] * L
    r = _r(np.zeros((T, E)), idx, [[1.0]] * T, probs=probs)
    # each sequence is perfectly concentrated: E * (1 * 1) per sequence
    assert oracle.balance(_cfg(T, E, 1), r, seq_len=L)["seq_aux"] == pytest.approx(E, rel=1e-12)
    # over the whole batch: f = P = (1/2, 1/2) -> E * 1/2
    assert oracle.balance(_cfg(T, E, 1), r, seq_len=0)["seq_aux"] == pytest.approx(E / 2.0, rel=1e-12)
    with pytest.raises(ValueError):
        oracle.balance(_cfg(T, E, 1), r, seq_len=3)


def test_seq_aux_whole_batch_equals_batch_aux_on_a_layer():
    cfg = Config("bal_layer", T=256, d=64, F=64, E=16, k=2, act_dtype="bf16", act="relu", gate="softmax_topk",
                 seed=31)
    inp = workloads.make_inputs(cfg)
    r = oracle.route(cfg, inp["x"], inp["w_router"], want_probs=True)
    dp = oracle.dispatch(cfg, r["idx"])
    st = oracle.stats(cfg, dp["counts"], dp["kept"], r["P"], cfg.T)
    b = oracle.balance(cfg, r, seq_len=0)
    assert b["seq_aux"] == pytest.approx(st["aux"], rel=1e-12)
    # renormalised gates: importance adds up to one per token
    assert b["importance"].sum() == pytest.approx(cfg.T, rel=1e-12)


def test_update_bias_sign_rule():
    b = oracle.update_bias([1, 2, 3], [0.0, 0.0, 0.0], 0.5)
    np.testing.assert_array_equal(b, np.array([0.5, 0.0, -0.5], np.float32))
    # mean 4/3 is not an integer: the comparison is exact
    b = oracle.update_bias([1, 1, 2], [1.0, -1.0, 0.25], 0.125)
    np.testing.assert_array_equal(b, np.array([1.125, -0.875, 0.125], np.float32))
