"""Pins of the oracle's layer stages against what the pages and mathematics fix.

* Gates: softmax over the selected logits equals a full softmax followed by
  top-k renormalisation (awesome-ai-roadmap 19.3.2); gates outside S are
  exactly zero; k = 1 gives gate 1; k = E gives the full softmax; the DSV3
  bias changes selection only (19.3.4); zero noise turns the noisy gate
  into the plain top-k gate (Shazeer notes 2.2).
* Selection: the oracle's top-k equals a stable library sort of its keys;
  its fp32 logits agree with an fp64 matmul within the fp32 dot-product
  error bound.
* Dispatch: the permutation equals numpy's stable argsort by expert; the
  capacity closed form; kept = min(n, C); f, P sum to 1; uniform routing
  gives f = 1/E, I = 1, aux = 1 (CS336 notes section 9).
* Experts: E = 1, k = 1 reduces the layer to a dense SwiGLU / ReLU MLP,
  compared with torch fp64.
* Whole layer: the dense brute force (every expert on every token, mixed with
  the dense gate vector) equals the sparse oracle; with inputs on an exact
  grid (all fp32 products and sums exact) to 1e-12, otherwise within the
  fp32-router bound.  Expert relabelling leaves the output unchanged
  (Lecture29 "Myth 1", permutation symmetry).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.brute as brute
import workloads
from workloads import Config


def small(gate="softmax_topk", act="swiglu", **kw):
    base = dict(name="small", T=96, d=64, F=96, E=8, k=2, act_dtype="f32", act=act, gate=gate, seed=5)
    base.update(kw)
    return Config(**base)


def _route(cfg, inp, **kw):
    return oracle.route(cfg, inp["x"], inp["w_router"], logit_bias=inp.get("logit_bias"),
                        sel_bias=inp.get("sel_bias"), w_noise=inp.get("w_noise"),
                        noise=kw.pop("noise", inp.get("noise")), want_probs=True, **kw)


# ---------------------------------------------------------------- gates

@pytest.mark.parametrize("E,k", [(8, 2), (64, 4), (16, 1)])
def test_selected_softmax_equals_full_softmax_renormalised(E, k):
    cfg = small(E=E, k=k)
    inp = workloads.make_inputs(cfg)
    a = _route(cfg, inp)
    b = _route(cfg.replace(gate="softmax_full"), inp)
    np.testing.assert_array_equal(a["idx"], b["idx"])
    renorm = b["gates"] / b["gates"].sum(axis=1, keepdims=True)
    np.testing.assert_allclose(a["gates"], renorm, rtol=0, atol=1e-12)
    # the full-softmax gates are the router probabilities at the selected experts
    np.testing.assert_allclose(b["gates"], np.take_along_axis(b["probs"], b["idx"], 1), rtol=0, atol=0)


@pytest.mark.parametrize("gate", ["softmax_topk", "noisy_topk", "sigmoid_bias"])
def test_gates_are_a_distribution_over_the_selection(gate):
    cfg = small(gate=gate, E=32, k=4, sel_bias=(gate == "sigmoid_bias"))
    inp = workloads.make_inputs(cfg)
    r = _route(cfg, inp)
    np.testing.assert_allclose(r["gates"].sum(1), 1.0, rtol=0, atol=1e-12)
    assert (r["gates"] > 0).all()
    # slot order is key order: the first slot has the largest key
    keys = np.take_along_axis(r["keys"], r["idx"], 1)
    assert (np.diff(keys, axis=1) <= 0).all()


def test_top1_gate_is_exactly_one():
    cfg = small(k=1)
    r = _route(cfg, workloads.make_inputs(cfg))
    assert (r["gates"] == 1.0).all()


def test_k_equal_E_is_the_dense_softmax():
    cfg = small(E=8, k=8)
    inp = workloads.make_inputs(cfg)
    r = _route(cfg, inp)
    dense = np.zeros_like(r["probs"])
    np.put_along_axis(dense, r["idx"], r["gates"], 1)
    np.testing.assert_allclose(dense, r["probs"], rtol=0, atol=1e-15)
    z = r["logits"].astype(np.float64)
    ref = np.exp(z - z.max(1, keepdims=True))
    np.testing.assert_allclose(dense, ref / ref.sum(1, keepdims=True), rtol=1e-13, atol=0)


def test_zero_noise_makes_noisy_gate_the_plain_topk_gate():
    cfg = small(gate="noisy_topk", E=32, k=4)
    inp = workloads.make_inputs(cfg)
    zero = np.zeros((cfg.T, cfg.E), np.float32)
    a = _route(cfg, inp, noise=zero)
    b = _route(cfg.replace(gate="softmax_topk"), inp)
    np.testing.assert_array_equal(a["idx"], b["idx"])
    np.testing.assert_array_equal(a["gates"], b["gates"])
    np.testing.assert_array_equal(a["keys"], b["keys"])


def test_noisy_score_with_zero_noise_matrix():
    """W_noise = 0 gives softplus(0) = ln 2, so H = z + n ln 2 exactly up to
    fp32 rounding of one fma."""
    cfg = small(gate="noisy_topk", E=16, k=4)
    inp = workloads.make_inputs(cfg)
    inp["w_noise"] = torch.zeros_like(inp["w_noise"])
    r = _route(cfg, inp)
    z = r["logits"].astype(np.float64)
    H = z + inp["noise"].numpy().astype(np.float64) * math.log(2)
    assert np.abs(r["keys"] - H).max() <= 4 * np.spacing(np.abs(H).max().astype(np.float32))
    # gates are the softmax of H over the selection; probs are softmax(H)
    Hs = r["keys"].astype(np.float64)
    p = np.exp(Hs - Hs.max(1, keepdims=True))
    np.testing.assert_allclose(r["probs"], p / p.sum(1, keepdims=True), rtol=1e-13)


def test_noisy_philox_noise_is_the_oracle_stream():
    cfg = small(gate="noisy_topk", E=16, k=4, seed=99)
    inp = workloads.make_inputs(cfg)
    a = _route(cfg, inp, noise=None, seed=99, noise_offset=5)
    n = oracle.normal(99, 5, 0, cfg.T * cfg.E).reshape(cfg.T, cfg.E)
    b = _route(cfg, inp, noise=n)
    np.testing.assert_array_equal(a["keys"], b["keys"])
    np.testing.assert_array_equal(a["idx"], b["idx"])


def test_sigmoid_bias_moves_selection_not_gates():
    """A large bias on a fixed set of k experts forces that set to be chosen;
    the gates are the renormalised raw affinities, whatever the bias size."""
    cfg = small(gate="sigmoid_bias", E=16, k=3, sel_bias=True)
    inp = workloads.make_inputs(cfg)
    forced = [2, 9, 13]
    gates = []
    for big in (3.0, 7.0):
        b = np.zeros(cfg.E, np.float32)
        b[forced] = big
        inp["sel_bias"] = torch.from_numpy(b)
        r = _route(cfg, inp)
        assert (np.sort(r["idx"], 1) == forced).all()
        gates.append(np.take_along_axis(r["gates"], np.argsort(r["idx"], 1), 1))
        z = r["logits"][:, forced].astype(np.float64)
        s = 1 / (1 + np.exp(-z))
        np.testing.assert_allclose(gates[-1], s / s.sum(1, keepdims=True), rtol=1e-13)
    np.testing.assert_array_equal(gates[0], gates[1])


def test_sigmoid_zero_bias_selects_top_logits():
    cfg = small(gate="sigmoid_bias", E=32, k=4, sel_bias=True)
    inp = workloads.make_inputs(cfg)
    inp["sel_bias"] = torch.zeros(cfg.E)
    a = _route(cfg, inp)
    b = _route(cfg.replace(gate="softmax_topk"), inp)
    np.testing.assert_array_equal(np.sort(a["idx"], 1), np.sort(b["idx"], 1))


# ---------------------------------------------------------------- selection and logits

@pytest.mark.parametrize("gate", ["softmax_topk", "noisy_topk", "sigmoid_bias"])
def test_topk_equals_stable_sort_of_keys(gate):
    cfg = small(gate=gate, E=64, k=6, T=200, sel_bias=(gate == "sigmoid_bias"))
    inp = workloads.make_inputs(cfg)
    r = _route(cfg, inp)
    keys = r["keys"].astype(np.float64)
    ref = np.argsort(-keys, axis=1, kind="stable")[:, :cfg.k]
    np.testing.assert_array_equal(r["idx"], ref)


def test_ties_break_to_lower_expert_index():
    cfg = small(E=8, k=3)
    inp = workloads.make_inputs(cfg)
    inp["w_router"] = torch.zeros_like(inp["w_router"])
    r = _route(cfg, inp)
    assert (r["idx"] == np.array([0, 1, 2])).all()
    np.testing.assert_allclose(r["gates"], 1 / 3, atol=1e-15)


@pytest.mark.parametrize("act_dtype", ["f32", "bf16"])
def test_logits_within_fp32_dot_bound(act_dtype):
    cfg = small(E=16, d=512, act_dtype=act_dtype)
    inp = workloads.make_inputs(cfg)
    r = _route(cfg, inp)
    x = oracle.act_to_f64(inp["x"], act_dtype)
    W = inp["w_router"].numpy().astype(np.float64)
    exact = x @ W.T
    gamma = cfg.d * 2.0 ** -24 / (1 - cfg.d * 2.0 ** -24)
    bound = gamma * (np.abs(x) @ np.abs(W).T)
    assert (np.abs(r["logits"] - exact) <= bound).all()


def test_logit_bias_is_added_to_logits():
    cfg = workloads.get("switch").replace(T=64)
    inp = workloads.make_inputs(cfg)
    a = _route(cfg, inp)
    b = _route(cfg, {k: v for k, v in inp.items() if k != "logit_bias"})
    np.testing.assert_array_equal(a["logits"], (b["logits"] + inp["logit_bias"].numpy()[None, :]).astype(np.float32))


# ---------------------------------------------------------------- dispatch and statistics

def test_dispatch_dropless_is_stable_argsort():
    cfg = small(E=16, k=4, T=300)
    r = _route(cfg, workloads.make_inputs(cfg))
    dp = oracle.dispatch(cfg, r["idx"])
    flat = r["idx"].reshape(-1)
    np.testing.assert_array_equal(dp["perm_src"], np.argsort(flat, kind="stable"))
    np.testing.assert_array_equal(dp["counts"], np.bincount(flat, minlength=cfg.E))
    np.testing.assert_array_equal(dp["offsets"], np.concatenate([[0], np.cumsum(dp["counts"])]))
    np.testing.assert_array_equal(dp["slot_pos"].reshape(-1)[dp["perm_src"]], np.arange(dp["R"]))
    assert dp["R"] == cfg.T * cfg.k and dp["C"] == -1


def test_capacity_closed_form_and_drops():
    cfg = workloads.get("switch")
    assert oracle.capacity(cfg) == 40          # ceil(1.25 * 2048 * 1 / 64)
    assert oracle.capacity(cfg.replace(T=100)) == math.ceil(1.25 * 100 / 64)
    inp = workloads.make_inputs(cfg)
    r = _route(cfg, inp)
    dp = oracle.dispatch(cfg, r["idx"])
    C = dp["C"]
    np.testing.assert_array_equal(dp["kept"], np.minimum(dp["counts"], C))
    assert dp["kept"].sum() + (dp["slot_pos"] < 0).sum() == cfg.T * cfg.k
    assert (dp["slot_pos"] < 0).sum() > 0      # the skewed bias overflows some experts
    # kept assignments are the first C of each expert in token order
    flat = r["idx"].reshape(-1)
    order = np.argsort(flat, kind="stable")
    rank = np.empty_like(order)
    for e in range(cfg.E):
        sel = order[flat[order] == e]
        rank[sel] = np.arange(sel.size)
    kept_ref = order[rank[order] < C]
    np.testing.assert_array_equal(dp["perm_src"], kept_ref)


def test_f_P_sum_to_one_and_stats():
    cfg = workloads.get("switch").replace(T=512)
    inp = workloads.make_inputs(cfg)
    o = oracle.forward(cfg, inp)
    assert o["f"].sum() == pytest.approx(1.0, abs=1e-15)
    assert o["P"].sum() == pytest.approx(1.0, abs=1e-12)
    np.testing.assert_allclose(o["P"], o["probs"].mean(0), rtol=1e-12)
    assert o["imbalance"] == pytest.approx(o["counts"].max() / (cfg.T * cfg.k / cfg.E))
    assert o["aux"] == pytest.approx(cfg.E * float((o["f"] * o["P"]).sum()))


@pytest.mark.parametrize("case", ["k1", "k2"])
def test_load_statistics_on_a_hand_worked_selection(case):
    """Counts, capacity cut, f, drops, imbalance and the balance term worked
    out by hand for a fixed selection (capacity C = ceil(cf T k / E) with the
    first C assignments of an expert in (t, j) order kept, Lecture29
    "Inference load balance"; f_i before drops with sum 1, CS336 notes
    section 9; I = max_i n_i / mean_i n_i, Lecture29 "Myth 3"; the balance
    term E sum f_i P_i, CS336 notes section 9).  The expected values tell
    max/mean apart from max/min (an expert with no tokens), from kept counts
    in place of routed ones, and from a T / E mean in place of T k / E."""
    if case == "k1":
        cfg = small(E=4, k=1, T=8, capacity_factor=1.0)
        idx = np.array([[0], [0], [1], [0], [2], [0], [1], [0]], np.int32)
        counts, kept, dropped, imb, aux = [5, 2, 1, 0], [2, 2, 1, 0], 3, 2.5, 1.4
        f = [5 / 8, 2 / 8, 1 / 8, 0.0]
    else:
        cfg = small(E=4, k=2, T=4, capacity_factor=1.0)
        idx = np.array([[0, 1], [0, 2], [0, 1], [3, 0]], np.int32)
        counts, kept, dropped, imb, aux = [4, 2, 1, 1], [2, 2, 1, 1], 2, 2.0, 1.25
        f = [4 / 8, 2 / 8, 1 / 8, 1 / 8]
    P = np.array([0.4, 0.3, 0.2, 0.1])
    dp = oracle.dispatch(cfg, idx)
    assert dp["C"] == 2
    np.testing.assert_array_equal(dp["counts"], counts)
    np.testing.assert_array_equal(dp["kept"], kept)
    st = oracle.stats(cfg, dp["counts"], dp["kept"], P, cfg.T)
    np.testing.assert_allclose(st["f"], f, rtol=0, atol=1e-15)
    assert st["n_dropped"] == dropped
    assert st["imbalance"] == imb
    assert st["aux"] == pytest.approx(aux, abs=1e-14)


def test_uniform_routing_gives_unit_balance_terms():
    """Token t points at expert t mod E (one-hot logits), k = 1: every expert
    gets T/E tokens, so f_i = 1/E (Lecture29 routing analysis: the uniform
    baseline 1/E), I = 1, and by the cyclic symmetry P_i = 1/E, so the
    Switch balance term E sum f_i P_i equals 1 (CS336 notes section 9)."""
    E, T = 8, 64
    cfg = small(E=E, k=1, T=T, d=E)
    inp = workloads.make_inputs(cfg)
    x = torch.zeros(T, E)
    x[torch.arange(T), torch.arange(T) % E] = 3.0
    inp["x"] = x
    inp["w_router"] = torch.eye(E)
    o = oracle.forward(cfg, inp)
    np.testing.assert_array_equal(o["idx"][:, 0], np.arange(T) % E)
    np.testing.assert_allclose(o["f"], 1 / E, rtol=0, atol=0)
    np.testing.assert_allclose(o["P"], 1 / E, rtol=1e-14)
    assert o["imbalance"] == 1.0
    assert o["aux"] == pytest.approx(1.0, abs=1e-14)


# ---------------------------------------------------------------- experts

@pytest.mark.parametrize("act", ["swiglu", "relu"])
@pytest.mark.parametrize("residual", [False, True])
def test_single_expert_layer_is_the_dense_mlp(act, residual):
    cfg = small(E=1, k=1, act=act, residual=residual)
    inp = workloads.make_inputs(cfg)
    o = oracle.forward(cfg, inp, round_intermediates=False)
    x = inp["x"].double()
    if act == "swiglu":
        h = torch.nn.functional.silu(x @ inp["w_gate"][0].double().T) * (x @ inp["w_up"][0].double().T)
        y = h @ inp["w_down"][0].double().T
    else:
        y = torch.relu(x @ inp["w1"][0].double().T) @ inp["w2"][0].double().T
    if residual:
        y = y + x
    np.testing.assert_allclose(o["out"], y.numpy(), rtol=1e-12, atol=1e-12)


def test_rounded_outputs_are_bf16_values_near_exact():
    cfg = small(act_dtype="bf16", E=8, k=2)
    inp = workloads.make_inputs(cfg)
    a = oracle.forward(cfg, inp, round_intermediates=True)
    for name in ("y", "out"):
        v = torch.from_numpy(a[name]).float()
        np.testing.assert_array_equal(v.bfloat16().float().numpy(), a[name])
    # one rounding step of h and y: within a few bf16 ulps of the fp64 layer
    b = oracle.forward(cfg, inp, round_intermediates=False)
    err = np.abs(a["out"] - b["out"]).max() / np.abs(b["out"]).max()
    assert err < 2 ** -6


# ---------------------------------------------------------------- whole layer

def _grid_inputs(cfg, seed=3):
    """Values on a coarse dyadic grid so that every fp32 product and partial
    sum of the router is exact: the fp32 logits equal the fp64 ones."""
    g = np.random.default_rng(seed)
    inp = workloads.make_inputs(cfg)
    inp["x"] = torch.from_numpy(g.integers(-4, 5, (cfg.T, cfg.d)).astype(np.float32) / 8)
    inp["w_router"] = torch.from_numpy(g.integers(-4, 5, (cfg.E, cfg.d)).astype(np.float32) / 8
                                       + g.integers(0, 1024, (cfg.E, 1)) / 2 ** 14)
    return inp


@pytest.mark.parametrize("gate", ["softmax_topk", "softmax_full"])
def test_brute_force_equals_sparse_oracle_exactly_on_grid(gate):
    cfg = small(gate=gate, E=8, k=2, T=64, d=32, F=48)
    inp = _grid_inputs(cfg)
    o = oracle.forward(cfg, inp, round_intermediates=False)
    b = brute.forward(cfg, inp)
    np.testing.assert_array_equal(o["idx"], b["S"])
    np.testing.assert_allclose(o["out"], b["out"], rtol=0, atol=1e-12 * np.abs(b["out"]).max())


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("switch", {"T": 512}),
    ("noisy", {"T": 128, "E": 32, "d": 64, "F": 128}),
    ("dsv3", {"T": 64, "E": 32, "d": 64, "F": 32, "F_shared": 48, "k": 4}),
    ("mixtral", {"T": 64, "d": 64, "F": 96}),
])
def test_brute_force_equals_sparse_oracle(name, kw):
    """Random inputs: the oracle's fp32 router logits differ from the brute
    force's fp64 ones by the fp32 dot-product bound, which moves the gates by
    ~1e-7 relative; selections agree."""
    cfg = workloads.get(name).replace(**kw)
    inp = workloads.make_inputs(cfg)
    o = oracle.forward(cfg, inp, round_intermediates=False)
    b = brute.forward(cfg, inp)
    np.testing.assert_array_equal(o["idx"], b["S"])
    scale = np.abs(b["out"]).max()
    np.testing.assert_allclose(o["out"], b["out"], rtol=0, atol=1e-5 * scale)


def test_dropped_assignments_pass_the_residual_through():
    cfg = workloads.get("switch").replace(T=512)
    inp = workloads.make_inputs(cfg)
    o = oracle.forward(cfg, inp)
    dropped = (o["slot_pos"] < 0).all(1)
    assert dropped.any()
    np.testing.assert_array_equal(o["out"][dropped], inp["x"].numpy()[dropped].astype(np.float64))


def test_expert_relabelling_leaves_layer_unchanged():
    cfg = small(E=8, k=2, T=80)
    inp = workloads.make_inputs(cfg)
    o = oracle.forward(cfg, inp)
    pi = np.random.default_rng(1).permutation(cfg.E)       # new label j holds old expert pi[j]
    perm = {k: (v[torch.from_numpy(pi)] if k in ("w_router", "w_gate", "w_up", "w_down") else v)
            for k, v in inp.items()}
    p = oracle.forward(cfg, perm)
    np.testing.assert_array_equal(pi[p["idx"]], o["idx"])
    np.testing.assert_array_equal(p["out"], o["out"])
    np.testing.assert_array_equal(p["gates"], o["gates"])
