"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small and mid-size layers are compared element by element on every stage;
the full-size Mixtral-, DeepSeek-V3- and Shazeer-shaped layers are compared
bit-exactly on routing and dispatch over all tokens and on sampled expert rows
and output tokens, which the oracle computes one by one.  Tolerances are the
ones stated in tests/gpu_helpers.py.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import Config
import sparse_mixture_experts_39_amd as moe
import tests.gpu_helpers as H

pytestmark = pytest.mark.gpu

MID = {
    # several tiles in every dimension and ragged tails everywhere
    "rag_bf16_swiglu": Config("rag_bf16_swiglu", T=1000, d=256, F=512, E=16, k=3, act_dtype="bf16",
                              act="swiglu", gate="softmax_topk", seed=11),
    "rag_bf16_relu_cap": Config("rag_bf16_relu_cap", T=777, d=192, F=320, E=6, k=2, act_dtype="bf16",
                                act="relu", gate="softmax_full", capacity_factor=1.0, residual=True, seed=12),
    "sigmoid_shared": Config("sigmoid_shared", T=300, d=128, F=128, E=64, k=8, act_dtype="bf16", act="swiglu",
                             gate="sigmoid_bias", n_shared=1, F_shared=192, sel_bias=True, seed=13),
    "noisy_small": Config("noisy_small", T=500, d=64, F=128, E=40, k=4, act_dtype="bf16", act="relu",
                          gate="noisy_topk", seed=14),
    # noisy gate with 2 E = 40 router columns (33 .. 63 columns)
    "noisy_40_cols": Config("noisy_40_cols", T=300, d=128, F=64, E=20, k=3, act_dtype="f32", act="relu",
                            gate="noisy_topk", seed=41),
    "f32_swiglu_mid": Config("f32_swiglu_mid", T=600, d=320, F=448, E=12, k=2, act_dtype="f32", act="swiglu",
                             gate="softmax_topk", seed=15),
    "many_experts": Config("many_experts", T=2000, d=64, F=64, E=1024, k=16, act_dtype="bf16", act="relu",
                           gate="softmax_topk", seed=16),
    # fewer than half a round of tiles on 256 CUs and K long enough: both
    # GEMMs cut every tile into K ranges and add them in the fixup kernel
    "split_k_bf16": Config("split_k_bf16", T=1024, d=1024, F=1024, E=4, k=2, act_dtype="bf16", act="swiglu",
                           gate="softmax_topk", seed=17),
    "split_k_f32": Config("split_k_f32", T=512, d=512, F=512, E=4, k=2, act_dtype="f32", act="swiglu",
                          gate="softmax_topk", seed=18),
    "split_k_relu_cap": Config("split_k_relu_cap", T=900, d=768, F=640, E=5, k=2, act_dtype="bf16", act="relu",
                               gate="softmax_full", capacity_factor=1.0, seed=19),
    # about 128 rows per expert with a long up reduction (K = d = 2048): the
    # up projection takes 256-row tiles (remainder tiles included), the down
    # projection (K = 256) 128-row tiles
    "k2048_avg128": Config("k2048_avg128", T=512, d=2048, F=256, E=8, k=2, act_dtype="bf16", act="swiglu",
                           gate="softmax_topk", seed=27),
    # 256 x 256 tiles without split: every accumulator goes through the
    # LDS-staged epilogue
    "tiles_256_bf16": Config("tiles_256_bf16", T=2048, d=256, F=256, E=2, k=1, act_dtype="bf16", act="swiglu",
                             gate="softmax_topk", seed=23),
    # expert choice: every expert takes its C top tokens, E slots per token
    "ec_bf16_swiglu": Config("ec_bf16_swiglu", T=1000, d=256, F=512, E=16, k=2, act_dtype="bf16", act="swiglu",
                             gate="expert_choice", capacity_factor=1.0, residual=True, seed=24),
    "ec_f32_relu": Config("ec_f32_relu", T=333, d=128, F=192, E=12, k=3, act_dtype="f32", act="relu",
                          gate="expert_choice", capacity_factor=1.5, logit_bias="zipf", seed=25),
    "ec_many_experts_shared": Config("ec_many_experts_shared", T=700, d=64, F=64, E=256, k=8, act_dtype="bf16",
                                     act="swiglu", gate="expert_choice", n_shared=1, F_shared=128, seed=26),
    # hash routing: experts from a hash of Zipf token ids, outputs summed
    "hash_bf16_swiglu": Config("hash_bf16_swiglu", T=1000, d=256, F=512, E=16, k=2, act_dtype="bf16", act="swiglu",
                               gate="hash", residual=True, seed=28),
    "hash_f32_top1_cap": Config("hash_f32_top1_cap", T=333, d=128, F=192, E=12, k=1, act_dtype="f32", act="relu",
                                gate="hash", capacity_factor=1.25, residual=True, seed=29),
    "hash_k_equals_E": Config("hash_k_equals_E", T=130, d=128, F=128, E=4, k=4, act_dtype="bf16", act="swiglu",
                              gate="hash", seed=30),
    # two-level gate: groups first, then experts inside each picked group
    "hier_bf16_relu": Config("hier_bf16_relu", T=1000, d=256, F=256, E=64, k=4, act_dtype="bf16", act="relu",
                             gate="hierarchical", n_groups=8, group_top_k=2, seed=31),
    "hier_f32_swiglu_bias": Config("hier_f32_swiglu_bias", T=333, d=128, F=192, E=24, k=3, act_dtype="f32",
                                   act="swiglu", gate="hierarchical", n_groups=3, group_top_k=3,
                                   logit_bias="zipf", capacity_factor=1.5, residual=True, seed=32),
    "hier_wide": Config("hier_wide", T=300, d=64, F=64, E=1024, k=16, act_dtype="bf16", act="relu",
                        gate="hierarchical", n_groups=32, group_top_k=4, seed=33),
    # capacity reroute: overflowing assignments move to the token's next expert with room
    "reroute_top2_zipf": Config("reroute_top2_zipf", T=1000, d=256, F=256, E=8, k=2, act_dtype="bf16",
                                act="swiglu", gate="softmax_topk", capacity_factor=1.0, logit_bias="zipf",
                                residual=True, reroute=True, seed=34),
    "reroute_sigmoid_k4": Config("reroute_sigmoid_k4", T=700, d=128, F=128, E=32, k=4, act_dtype="bf16",
                                 act="swiglu", gate="sigmoid_bias", sel_bias=True, capacity_factor=1.0,
                                 residual=True, reroute=True, seed=35),
    "reroute_hash_f32": Config("reroute_hash_f32", T=512, d=64, F=128, E=16, k=3, act_dtype="f32", act="relu",
                               gate="hash", capacity_factor=0.9, residual=True, reroute=True, seed=36),
    # rows wider than one block's registers (4160 16-byte chunks): dispatch
    # falls back to scatter + copy, combine runs in column passes
    "wide_rows": Config("wide_rows", T=70, d=33280, F=64, E=4, k=2, act_dtype="bf16", act="relu",
                        gate="softmax_topk", residual=True, seed=38),
    # expert choice with more than 256 (and 512) slots per token: dispatch
    # ranks in two passes, combine reads the slot rows unstaged
    "ec_wide_slots": Config("ec_wide_slots", T=150, d=64, F=64, E=600, k=2, act_dtype="bf16", act="relu",
                            gate="expert_choice", capacity_factor=1.0, residual=True, seed=39),
    # more than 64 experts: ranked lists of 16, then the full scan once they are used up
    "reroute_many_experts": Config("reroute_many_experts", T=900, d=64, F=64, E=200, k=2, act_dtype="bf16",
                                   act="relu", gate="softmax_full", capacity_factor=1.0, logit_bias="zipf",
                                   residual=True, reroute=True, seed=37),
}


def full_oracle(cfg, inp, noise="input", noise_offset=0):
    return oracle.forward(cfg, inp, noise=noise, noise_offset=noise_offset)


def check_all(cfg, g, o):
    T = cfg.T
    H.compare_route(cfg, g, o, T)
    H.compare_dispatch(cfg, g, o)
    R = o["R"]
    np.testing.assert_array_equal(H.bytes_of(g["x_perm"][:R]), o["x_perm"].view(np.int16 if cfg.act_dtype == "bf16" else np.int32),
                                  err_msg="x_perm bytes")
    if R:
        H.assert_close_rel(H.as_f64(g["y_perm"][:R]), o["y"], cfg.act_dtype, "y_perm")
    if cfg.n_shared:
        H.assert_close_rel(H.as_f64(g["shared"]), o["shared"], cfg.act_dtype, "shared expert")
    return H.assert_close_rel(H.as_f64(g["out"]), o["out"], cfg.act_dtype, "out")


@pytest.mark.parametrize("name", ["tiny", "switch"])
def test_small_configs_every_stage(name):
    cfg = workloads.get(name)
    H.log(f"[parity] {name} T={cfg.T}")
    inp = workloads.make_inputs(cfg)
    g = H.run_stages(cfg, H.to_device(inp))
    o = full_oracle(cfg, inp)
    err = check_all(cfg, g, o)
    H.log(f"[parity] {name} out rel err {err:.2e}")


@pytest.mark.parametrize("name", list(MID))
def test_mid_configs_every_stage(name):
    cfg = MID[name]
    H.log(f"[parity] {name}")
    inp = workloads.make_inputs(cfg)
    g = H.run_stages(cfg, H.to_device(inp))
    o = full_oracle(cfg, inp)
    err = check_all(cfg, g, o)
    H.log(f"[parity] {name} out rel err {err:.2e}")


def test_noisy_builtin_philox_stream_matches_oracle():
    """In-kernel Philox4x32-10 + Box-Muller + canonical softplus: scores equal
    the oracle's bit for bit, hence the same selection."""
    cfg = MID["noisy_small"]
    inp = workloads.make_inputs(cfg)
    g = H.run_stages(cfg, H.to_device(inp), noise_input=False, noise_offset=7)
    o = full_oracle(cfg, inp, noise="philox", noise_offset=7)
    check_all(cfg, g, o)


# moe_layer_forward gathers the up projection's rows from x (the stage calls
# read the dispatch's x_perm copy): small tiles, 256 x 256 ping-pong tiles with
# split-K units, remainder tiles, expert choice, hash routing and fp32.
LAYER_EQ = ["sigmoid_shared", "split_k_bf16", "k2048_avg128", "tiles_256_bf16", "rag_bf16_swiglu", "ec_bf16_swiglu",
            "hash_bf16_swiglu", "f32_swiglu_mid", "split_k_relu_cap"]


@pytest.mark.parametrize("name", LAYER_EQ)
def test_layer_forward_equals_stages_and_is_deterministic(name):
    cfg = MID[name]
    inp = workloads.make_inputs(cfg)
    d = H.to_device(inp)
    g = H.run_stages(cfg, d)
    out1, st1 = H.run_layer(cfg, d)
    out2, st2 = H.run_layer(cfg, d)
    np.testing.assert_array_equal(H.bytes_of(out1), H.bytes_of(g["out"]))
    np.testing.assert_array_equal(H.bytes_of(out1), H.bytes_of(out2))
    for k in st1:
        np.testing.assert_array_equal(st1[k].numpy(), st2[k].numpy())


# ---------------------------------------------------------------- edge cases

EDGE = {
    "one_token": dict(T=1),
    "all_ties": dict(zero_router=True),
    "single_expert": dict(E=1, k=1),
    "k_equals_E": dict(E=4, k=4),
    "capacity_one": dict(capacity_factor=0.01, residual=True),
    "d64": dict(d=64, F=64),
    "ragged_T": dict(T=257),
}


EC_EDGE = {
    "ec_one_token": dict(T=1),
    "ec_all_ties": dict(zero_router=True),
    "ec_every_token": dict(capacity_factor=100.0),       # C = T: every expert takes every token
    "ec_single_expert": dict(E=1, k=1),
    "ec_ragged_T": dict(T=1031, E=5, k=2),
}


@pytest.mark.parametrize("case", list(EC_EDGE))
def test_expert_choice_edge_cases(case):
    kw = dict(EC_EDGE[case])
    zero_router = kw.pop("zero_router", False)
    cfg = Config("ec_edge", T=130, d=128, F=192, E=8, k=2, act_dtype="bf16", act="swiglu", gate="expert_choice",
                 capacity_factor=1.0, residual=True, seed=27).replace(**kw)
    H.log(f"[edge] {case}")
    inp = workloads.make_inputs(cfg)
    if zero_router:
        inp["w_router"] = torch.zeros_like(inp["w_router"])     # every expert takes tokens 0..C-1
    g = H.run_stages(cfg, H.to_device(inp))
    o = full_oracle(cfg, inp)
    check_all(cfg, g, o)
    C = oracle.capacity(cfg)
    np.testing.assert_array_equal(g["stats"]["counts"].numpy(), np.full(cfg.E, C))
    if zero_router:
        taken = g["idx"].numpy() >= 0
        assert taken[:C].all() and not taken[C:].any()


@pytest.mark.parametrize("case", list(EDGE))
def test_edge_cases(case):
    kw = dict(EDGE[case])
    zero_router = kw.pop("zero_router", False)
    cfg = Config("edge", T=130, d=128, F=192, E=8, k=2, act_dtype="bf16", act="swiglu", gate="softmax_topk",
                 seed=21).replace(**kw)
    H.log(f"[edge] {case}")
    inp = workloads.make_inputs(cfg)
    if zero_router:
        inp["w_router"] = torch.zeros_like(inp["w_router"])     # every token on experts 0..k-1
    g = H.run_stages(cfg, H.to_device(inp))
    o = full_oracle(cfg, inp)
    check_all(cfg, g, o)
    if zero_router:
        assert (g["stats"]["counts"].numpy()[cfg.k:] == 0).all()


def test_empty_batch():
    cfg = Config("empty", T=0, d=128, F=128, E=8, k=2, act_dtype="bf16", act="swiglu", gate="softmax_topk", seed=1)
    inp = workloads.make_inputs(cfg.replace(T=1))
    d = H.to_device(inp)
    d["x"] = d["x"][:0]
    g = H.run_stages(cfg, d)
    assert g["out"].shape == (0, 128)
    assert (g["offsets"].numpy() == 0).all()
    assert (g["stats"]["counts"].numpy() == 0).all()
    assert int(g["stats"]["n_dropped"][0]) == 0


# Router products at few columns (one wave per block, K chunks of 128 through
# a ring of LDS slots when d is a multiple of 128): every column count class,
# both dtypes, fewer chunks than ring slots and more (with a ragged last
# round), a ragged last block of tokens; and two shapes of the many-column
# kernel.  The scores must be bit-identical.
ROUTER_SHAPES = [(2, "bf16", 384), (3, "f32", 1152), (4, "bf16", 1152), (5, "f32", 384), (8, "bf16", 1152),
                 (8, "f32", 384), (12, "bf16", 384), (16, "bf16", 1152), (16, "f32", 1152), (32, "bf16", 384),
                 (8, "bf16", 320), (64, "bf16", 384), (96, "f32", 384),
                 # 33 .. 63 columns (a gap of the few-column kernels, found by the random-shape sweep)
                 (33, "f32", 128), (40, "bf16", 1152), (63, "bf16", 320)]


@pytest.mark.parametrize("E,dt,d", ROUTER_SHAPES)
def test_router_dots_shapes(E, dt, d):
    cfg = Config(f"dots_{E}_{dt}_{d}", T=777, d=d, F=64, E=E, k=min(2, E), act_dtype=dt, act="relu",
                 gate="softmax_topk", seed=40 + E)
    H.log(f"[dots] E={E} {dt} d={d}")
    inp = workloads.make_inputs(cfg)
    g = H.run_stages(cfg, H.to_device(inp))
    o = oracle.route(cfg, inp["x"], inp["w_router"])
    o["status"] = 0
    H.compare_route(cfg, g, o, cfg.T)


# Dispatch against the oracle's stable counting sort at larger sizes: 16384
# assignments and one more, one expert, capacity drops under a skewed router
# (most assignments of the busiest experts dropped), four slots per token.
DISPATCH_CASES = {
    "disp_e8_k2": dict(T=4096, E=8, k=2),
    "disp_e16_full": dict(T=16384, E=16, k=1),
    "disp_e16_over": dict(T=16385, E=16, k=1),
    "disp_e16_cap_zipf": dict(T=16384, E=16, k=1, capacity_factor=1.25, logit_bias="zipf"),
    "disp_e12_k4_cap_zipf": dict(T=4096, E=12, k=4, capacity_factor=1.1, logit_bias="zipf"),
    "disp_e5_k3_cap": dict(T=1000, E=5, k=3, capacity_factor=1.0),
    "disp_e1": dict(T=700, E=1, k=1),
}


@pytest.mark.parametrize("name", list(DISPATCH_CASES))
def test_dispatch_sizes_and_drops(name):
    kw = DISPATCH_CASES[name]
    cfg = Config(name, d=64, F=64, act_dtype="bf16", act="relu", gate="softmax_topk", residual=True, seed=50, **kw)
    H.log(f"[dispatch] {name}")
    inp = workloads.make_inputs(cfg)
    g = H.run_stages(cfg, H.to_device(inp))
    o = oracle.route(cfg, inp["x"], inp["w_router"], logit_bias=inp.get("logit_bias"))
    o.update(oracle.dispatch(cfg, o["idx"]))
    o.update(oracle.stats(cfg, o["counts"], o["kept"], o["P"], cfg.T))
    o["status"] = 0
    H.compare_route(cfg, g, o, cfg.T)
    H.compare_dispatch(cfg, g, o)


# Capacity factors whose product with T k / E is an integer (C = 44, 600 and
# 2 exactly by the printed formula) and which a binary float32 factor would
# round up by one; a Zipf logit bias makes the busiest experts overflow, so
# the drop masks decide at exactly C.
CAPACITY_BOUNDARY = {
    "cap_1p1_T2560_E64_k1": (dict(T=2560, E=64, k=1, capacity_factor=1.1), 44),
    "cap_1p2_T4000_E16_k2": (dict(T=4000, E=16, k=2, capacity_factor=1.2), 600),
    "cap_0p1_T160_E8_k1": (dict(T=160, E=8, k=1, capacity_factor=0.1), 2),
}


@pytest.mark.parametrize("name", list(CAPACITY_BOUNDARY))
def test_capacity_on_integer_boundaries_drops_bit_exact(name):
    kw, C_formula = CAPACITY_BOUNDARY[name]
    cfg = Config(name, d=64, F=64, act_dtype="bf16", act="relu", gate="softmax_topk", residual=True,
                 logit_bias="zipf", seed=51, **kw)
    H.log(f"[capacity] {name}")
    assert oracle.capacity(cfg) == C_formula == moe.capacity(H.bind_config(cfg))
    inp = workloads.make_inputs(cfg)
    g = H.run_stages(cfg, H.to_device(inp))
    o = full_oracle(cfg, inp)
    check_all(cfg, g, o)
    kept = g["stats"]["kept"].numpy()
    assert kept.max() == C_formula and int(g["stats"]["n_dropped"][0]) > 0


# Expert row counts that put every kind of remainder after 256-row tiles:
# none, 1 and 64 (these go to a 64-row remainder tile of the same launch), 65,
# 128, 129 and 255 (a whole, padded 256-row tile), and experts smaller than one
# tile, on either side of the 64-row threshold.  The caller hands
# the offsets straight to moe_expert_ffn; every row is checked.
REM_COUNTS = [256, 257, 320, 321, 384, 385, 511, 0, 1, 64, 100, 128, 129, 577]


@pytest.mark.parametrize("act", ["swiglu", "relu"])
def test_expert_ffn_remainder_tiles(act):
    E = len(REM_COUNTS)
    cfg = Config("rem_" + act, T=2700, d=512, F=512, E=E, k=2, act_dtype="bf16", act=act,
                 gate="softmax_topk", seed=31)
    c = H.bind_config(cfg)
    R = moe.max_rows(c)
    assert sum(REM_COUNTS) <= R and R // E >= 384     # 256-row tiles are chosen for this average
    inp = workloads.make_inputs(cfg)
    d = H.to_device(inp)
    x_perm = torch.cat([d["x"], d["x"]])[:R].contiguous()
    off = np.concatenate([[0], np.cumsum(REM_COUNTS)]).astype(np.int32)
    offsets = torch.from_numpy(off).to("cuda")
    y_perm = torch.zeros((R, cfg.d), dtype=torch.bfloat16, device="cuda")
    H.log(f"[rem] {act}: expert_ffn with counts {REM_COUNTS}")
    moe.moe_expert_ffn(c, x_perm, offsets, moe.weights_from(c, d), y_perm, moe.workspace(c))
    torch.cuda.synchronize()
    xp = x_perm.cpu()
    y = y_perm.cpu()
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        ref = oracle.expert_ffn(cfg, xp[lo:hi], *oracle.expert_weights(cfg, inp, e))
        H.assert_close_rel(H.as_f64(y[lo:hi]), ref, "bf16", f"expert {e} ({hi - lo} rows)")


# Reductions of 1, 2 and 3 K slices (64 bf16 values each) through 256 x 256
# tiles, whose two wave groups take turns loading and multiplying: the
# shortest prologues and drains of that schedule.  (d, F) puts the short K
# on the up projection (K = d, N = F) or on the down projection (K = F,
# N = d = 256); the other product and every expert row are checked too.
@pytest.mark.parametrize("d,F", [(64, 256), (128, 256), (192, 256), (256, 64), (256, 128), (256, 192)])
@pytest.mark.parametrize("act", ["swiglu", "relu"])
def test_expert_ffn_short_reductions(d, F, act):
    E = len(REM_COUNTS)
    cfg = Config(f"shortk_{act}_{d}_{F}", T=2700, d=d, F=F, E=E, k=2, act_dtype="bf16", act=act,
                 gate="softmax_topk", seed=33)
    c = H.bind_config(cfg)
    R = moe.max_rows(c)
    assert sum(REM_COUNTS) <= R and R // E >= 384     # 256-row tiles are chosen for this average
    inp = workloads.make_inputs(cfg)
    dv = H.to_device(inp)
    x_perm = torch.cat([dv["x"], dv["x"]])[:R].contiguous()
    off = np.concatenate([[0], np.cumsum(REM_COUNTS)]).astype(np.int32)
    offsets = torch.from_numpy(off).to("cuda")
    y_perm = torch.zeros((R, d), dtype=torch.bfloat16, device="cuda")
    H.log(f"[short-k] {act} d={d} F={F}: expert_ffn with counts {REM_COUNTS}")
    moe.moe_expert_ffn(c, x_perm, offsets, moe.weights_from(c, dv), y_perm, moe.workspace(c))
    torch.cuda.synchronize()
    xp = x_perm.cpu()
    y = y_perm.cpu()
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        ref = oracle.expert_ffn(cfg, xp[lo:hi], *oracle.expert_weights(cfg, inp, e))
        H.assert_close_rel(H.as_f64(y[lo:hi]), ref, "bf16", f"expert {e} ({hi - lo} rows)")


@pytest.mark.parametrize("act", ["swiglu", "relu"])
def test_expert_gemms_unaligned_outputs_bitwise(act):
    """Outputs whose rows cannot be stored 16 bytes at a time (the buffer
    starts 2 bytes past a 16-byte boundary) go through the direct-store
    instantiation of the grouped GEMM instead of the LDS-staged one; both
    must write the same bits."""
    E = len(REM_COUNTS)
    cfg = Config("unal_" + act, T=2700, d=512, F=512, E=E, k=2, act_dtype="bf16", act=act,
                 gate="softmax_topk", seed=32)
    c = H.bind_config(cfg)
    R = moe.max_rows(c)
    inp = workloads.make_inputs(cfg)
    d = H.to_device(inp)
    w = moe.weights_from(c, d)
    ws = moe.workspace(c)
    x_perm = torch.cat([d["x"], d["x"]])[:R].contiguous()
    off = np.concatenate([[0], np.cumsum(REM_COUNTS)]).astype(np.int32)
    offsets = torch.from_numpy(off).to("cuda")
    kept = int(off[-1])

    def unaligned(rows, cols):
        t = torch.full((rows * cols + 1,), float("nan"), dtype=torch.bfloat16, device="cuda")[1:].view(rows, cols)
        assert t.data_ptr() % 16 == 2
        return t

    H.log(f"[unaligned] {act}: expert_up / expert_down, aligned and 2-byte-offset outputs")
    h_a = torch.zeros((R, cfg.F), dtype=torch.bfloat16, device="cuda")
    y_a = torch.zeros((R, cfg.d), dtype=torch.bfloat16, device="cuda")
    moe.moe_expert_up(c, x_perm, offsets, w, h_a, ws)
    moe.moe_expert_down(c, h_a, offsets, w, y_a, ws)
    h_u, y_u = unaligned(R, cfg.F), unaligned(R, cfg.d)
    moe.moe_expert_up(c, x_perm, offsets, w, h_u, ws)
    moe.moe_expert_down(c, h_a, offsets, w, y_u, ws)
    torch.cuda.synchronize()
    assert torch.equal(h_a[:kept].view(torch.int16), h_u[:kept].view(torch.int16)), "h differs"
    assert torch.equal(y_a[:kept].view(torch.int16), y_u[:kept].view(torch.int16)), "y differs"


def test_nonfinite_input_sets_device_status():
    cfg = Config("nan", T=64, d=64, F=64, E=8, k=2, act_dtype="f32", act="relu", gate="softmax_topk", seed=2)
    inp = workloads.make_inputs(cfg)
    inp["x"][5, 3] = float("nan")
    g = H.run_stages(cfg, H.to_device(inp))
    assert int(g["stats"]["device_status"][0]) == 1
    o = oracle.route(cfg, inp["x"], inp["w_router"])
    assert o["status"] == 1
    np.testing.assert_array_equal(g["idx"].numpy(), o["idx"])


# ---------------------------------------------------------------- full sizes, sampled

def _sampled_full_size(name, n_tokens=12, rows_per_expert=2, max_experts=24, noise_input=True):
    cfg = workloads.get(name)
    H.log(f"[full] {name}: drawing inputs on the GPU")
    dinp = workloads.make_inputs(cfg, device="cuda")
    g = H.run_stages(cfg, dinp, noise_input=noise_input)
    H.log(f"[full] {name}: GPU path done, oracle route/dispatch over all {cfg.T} tokens")
    x = dinp["x"].cpu()
    o = oracle.route(cfg, x, dinp["w_router"].cpu(),
                     logit_bias=dinp["logit_bias"].cpu() if "logit_bias" in dinp else None,
                     sel_bias=dinp["sel_bias"].cpu() if "sel_bias" in dinp else None,
                     w_noise=dinp["w_noise"].cpu() if "w_noise" in dinp else None,
                     noise=dinp["noise"].cpu() if (noise_input and "noise" in dinp) else None,
                     token_ids=dinp["token_ids"].cpu() if "token_ids" in dinp else None,
                     w_group_router=dinp["w_group_router"].cpu() if "w_group_router" in dinp else None)
    if cfg.reroute:
        o["idx"] = oracle.reroute(cfg, o["keys"], o["idx"])
    o.update(oracle.dispatch(cfg, o["idx"]))
    o.update(oracle.stats(cfg, o["counts"], o["kept"], o["P"], cfg.T))
    o["status"] = 0
    H.compare_route(cfg, g, o, cfg.T)
    H.compare_dispatch(cfg, g, o)
    R = o["R"]
    xp = oracle.gather_rows(cfg, x, o["perm_src"])
    np.testing.assert_array_equal(H.bytes_of(g["x_perm"][:R]), xp.view(np.int16 if cfg.act_dtype == "bf16" else np.int32))
    H.log(f"[full] {name}: routing and dispatch bit-exact; sampling expert rows")
    rng = np.random.default_rng(0)
    off = o["offsets"]
    experts = [e for e in range(cfg.E) if off[e + 1] > off[e]]
    experts = sorted(rng.choice(experts, size=min(max_experts, len(experts)), replace=False).tolist())

    def weights(e):
        return oracle.expert_weights(cfg, {k: v for k, v in dinp.items() if k.startswith("w")}, e)

    y_ref, y_got = [], []
    for e in experts:
        lo, hi = int(off[e]), int(off[e + 1])
        rows = sorted(set([lo, hi - 1] + rng.integers(lo, hi, size=rows_per_expert).tolist()))
        y_ref.append(oracle.expert_ffn(cfg, xp[rows], *weights(e)))
        y_got.append(H.as_f64(g["y_perm"][rows]))
    err_y = H.assert_close_rel(np.concatenate(y_got), np.concatenate(y_ref), cfg.act_dtype, "sampled y_perm")
    H.log(f"[full] {name}: sampled y rel err {err_y:.2e}; sampling output tokens")
    tokens = np.sort(rng.choice(cfg.T, size=n_tokens, replace=False)).astype(np.int32)
    sp = o["slot_pos"][tokens]
    need = sorted(set(int(r) for r in sp.reshape(-1) if r >= 0))
    compact = {r: i for i, r in enumerate(need)}
    y_c = np.zeros((len(need), cfg.d))
    ends = off[1:]
    for r in need:
        e = int(np.searchsorted(ends, r, side="right"))
        y_c[compact[r]] = oracle.expert_ffn(cfg, xp[[r]], *weights(e))[0]
    sp_c = np.where(sp >= 0, np.vectorize(lambda r: compact.get(int(r), -1))(sp), -1).astype(np.int32)
    shared = None
    if cfg.n_shared:
        shared = oracle.expert_ffn(cfg, x[torch.from_numpy(tokens).long()], *oracle.shared_weights(dinp),
                                   F=cfg.F_shared)
        H.assert_close_rel(H.as_f64(g["shared"][torch.from_numpy(tokens).long()]), shared, cfg.act_dtype,
                           "sampled shared expert")
    out_ref = oracle.combine(cfg, sp_c, o["gates"][tokens], y_c, x[torch.from_numpy(tokens).long()],
                             shared=shared)
    err = H.assert_close_rel(H.as_f64(g["out"][torch.from_numpy(tokens).long()]), out_ref, cfg.act_dtype,
                             "sampled out")
    H.log(f"[full] {name}: sampled out rel err {err:.2e}")


def test_full_size_mixtral_sampled():
    _sampled_full_size("mixtral", max_experts=8, rows_per_expert=3)


def test_full_size_dsv3_sampled():
    _sampled_full_size("dsv3", n_tokens=6, max_experts=16, rows_per_expert=1)


def test_full_size_noisy_sampled():
    _sampled_full_size("noisy", n_tokens=24, max_experts=32, rows_per_expert=2)


def test_full_size_mixtral_expert_choice_sampled():
    _sampled_full_size("mixtral_ec", max_experts=8, rows_per_expert=3)


def test_full_size_mixtral_hash_sampled():
    _sampled_full_size("mixtral_hash", max_experts=8, rows_per_expert=3)


def test_full_size_hierarchical_sampled():
    _sampled_full_size("hier", n_tokens=24, max_experts=32, rows_per_expert=2)


def test_full_size_switch_reroute():
    _sampled_full_size("switch_reroute", n_tokens=32, max_experts=16, rows_per_expert=2)


def test_full_size_noisy_philox_routing():
    _sampled_full_size("noisy", n_tokens=8, max_experts=8, rows_per_expert=1, noise_input=False)
