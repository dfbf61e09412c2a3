"""Pins of the oracle's capacity reroute (Lecture29, "Inference load balance":
an expert over capacity may drop, reroute or delay): a worked example small
enough to follow by hand, no change without overflow, conservation of the
assignments, the pigeonhole case where top-1 with E*C >= T leaves nothing to
drop, and that a moved assignment only ever lands on an expert with room."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import Config


def _cfg(**kw):
    base = dict(T=8, d=64, F=64, E=3, k=1, act_dtype="f32", act="relu", gate="softmax_topk",
                capacity_factor=1.0, residual=True, reroute=True, seed=5)
    base.update(kw)
    return Config("rr", **base)


def test_worked_example():
    # T = 4 tokens, E = 3, k = 1, cf = 0.75 -> C = ceil(0.75 * 4 / 3) = 1.
    # Every token prefers expert 0; their second choices are 1, 2, 1, 2.
    cfg = _cfg(T=4, capacity_factor=0.75)
    assert oracle.capacity(cfg) == 1
    keys = np.array([[3.0, 2.0, 1.0],
                     [3.0, 1.0, 2.0],
                     [3.0, 2.0, 1.0],
                     [3.0, 1.0, 2.0]], dtype=np.float32)
    idx = np.zeros((4, 1), dtype=np.int32)
    out = oracle.reroute(cfg, keys, idx)
    # token 0 keeps expert 0; token 1 moves to its best expert with room (2);
    # token 2 to 1; token 3 finds experts 0, 1, 2 all full and stays (dropped)
    np.testing.assert_array_equal(out[:, 0], [0, 2, 1, 0])


def test_no_overflow_no_change_and_conservation():
    cfg = _cfg(T=300, E=8, k=2, capacity_factor=1.1, d=64)
    inp = workloads.make_inputs(cfg)
    r = oracle.route(cfg, inp["x"], inp["w_router"])
    out = oracle.reroute(cfg, r["keys"], r["idx"])
    assert out.shape == r["idx"].shape
    # tokens never hold one expert twice, and every slot still names an expert
    assert all(len(set(row)) == cfg.k for row in out)
    C = oracle.capacity(cfg)
    ample = cfg.replace(capacity_factor=float(cfg.E))          # C >= T k: nothing overflows
    np.testing.assert_array_equal(oracle.reroute(ample, r["keys"], r["idx"]), r["idx"])
    # after the move, the experts that still overflow are exactly the dropped ones' wish lists: none
    # of a dropped assignment's alternatives had room
    n = np.bincount(out.reshape(-1), minlength=cfg.E)
    d = oracle.dispatch(cfg, out)
    for a in np.nonzero(d["slot_pos"].reshape(-1) < 0)[0]:
        t = a // cfg.k
        others = [e for e in range(cfg.E) if e not in out[t]]
        assert all(n[e] >= C for e in others)


@pytest.mark.parametrize("T,E,cf", [(64, 4, 1.0), (101, 7, 1.0), (512, 16, 1.25)])
def test_top1_with_room_for_everyone_drops_nothing(T, E, cf):
    """k = 1 and E C >= T: whenever an assignment overflows, some other expert
    still has room (pigeonhole), so after the reroute dispatch drops none."""
    cfg = _cfg(T=T, E=E, k=1, capacity_factor=cf)
    C = oracle.capacity(cfg)
    assert E * C >= T
    inp = workloads.make_inputs(cfg)
    inp["w_router"][0] += 3.0            # pile the tokens onto expert 0
    r = oracle.route(cfg, inp["x"], inp["w_router"])
    before = oracle.dispatch(cfg, r["idx"])
    assert (before["slot_pos"] < 0).any(), "expected drops without the reroute"
    out = oracle.reroute(cfg, r["keys"], r["idx"])
    after = oracle.dispatch(cfg, out)
    assert (after["slot_pos"] >= 0).all()
    assert (after["kept"] <= C).all()


def test_moves_go_to_the_best_expert_with_room():
    cfg = _cfg(T=200, E=6, k=2, capacity_factor=1.0)
    inp = workloads.make_inputs(cfg)
    inp["w_router"][2] += 2.0
    r = oracle.route(cfg, inp["x"], inp["w_router"])
    out = oracle.reroute(cfg, r["keys"], r["idx"])
    C = oracle.capacity(cfg)
    n = np.zeros(cfg.E, dtype=np.int64)
    over = []
    for a, e in enumerate(r["idx"].reshape(-1)):
        if n[e] < C:
            n[e] += 1
        else:
            over.append(a)
    moved = [a for a in over if out.reshape(-1)[a] != r["idx"].reshape(-1)[a]]
    assert moved, "expected some rerouted assignment"
    cur = r["idx"].copy().reshape(-1)
    for a in over:
        t = a // cfg.k
        room = [e for e in range(cfg.E) if n[e] < C and e not in cur[t * cfg.k:(t + 1) * cfg.k]]
        if room:
            best = max(room, key=lambda e: (r["keys"][t, e], -e))
            assert out.reshape(-1)[a] == best
            cur[a] = best
            n[best] += 1
        else:
            assert out.reshape(-1)[a] == cur[a]
