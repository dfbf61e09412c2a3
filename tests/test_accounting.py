"""Closed forms of parameter and storage accounting against the pages' numbers
(tests/golden/pages_numbers.json holds each number with its citation)."""
import json
import math
import os

import pytest

from oracle import accounting as acc

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


def _mixtral():
    m = GOLD["mixtral"]
    d, F = 4096, 14336
    P_e = acc.expert_params(d, F, "swiglu")
    P_s = acc.layer_shared_params(d, m["n_query_heads"], m["n_kv_heads"], m["n_experts"])
    return m, P_e, P_s


def test_mixtral_total_minus_active_is_the_idle_experts():
    """P_total - P_active = N (E - k) P_e, free of embeddings and shared parts."""
    m, P_e, P_s = _mixtral()
    diff = acc.total_params(0, m["n_layers"], P_s, m["n_experts"], P_e) - \
        acc.active_params(0, m["n_layers"], P_s, m["top_k"], P_e)
    assert diff == m["n_layers"] * (m["n_experts"] - m["top_k"]) * P_e
    assert abs(diff / 1e9 - (m["total_params_B"] - m["active_params_B"])) <= 0.1


def test_mixtral_total_and_active_admit_one_embedding_size():
    """Both printed figures (rounded to 0.1B) are met by a common embedding
    count; the vocabulary is not on the pages, so only existence is checked."""
    m, P_e, P_s = _mixtral()
    N = m["n_layers"]
    body_total = N * (P_s + m["n_experts"] * P_e)
    body_active = N * (P_s + m["top_k"] * P_e)
    lo = max(m["total_params_B"] * 1e9 - 0.05e9 - body_total, m["active_params_B"] * 1e9 - 0.05e9 - body_active, 0)
    hi = min(m["total_params_B"] * 1e9 + 0.05e9 - body_total, m["active_params_B"] * 1e9 + 0.05e9 - body_active)
    assert lo <= hi
    # and the layer body alone rounds to the pages' 47B / 13B class
    assert round(body_total / 1e9) == 46 and round(body_active / 1e9) == 13


def test_expert_fraction_of_active_path():
    m, P_e, P_s = _mixtral()
    rho = acc.expert_fraction(P_s, m["top_k"], P_e)
    assert 0.85 < rho < 0.95
    assert rho == pytest.approx(2 * P_e / (P_s + 2 * P_e))


def test_shazeer_expert_shape_is_one_million_parameters():
    s = GOLD["shazeer"]
    p = acc.expert_params(s["expert_in"], s["expert_hidden"], "relu")
    assert p == 512 * 1024 + 1024 * 512 == 1_048_576
    assert round(p / 1e6, 1) == s["expert_params_M"]


def test_shazeer_batch_shrinkage_and_sparsity():
    s = GOLD["shazeer"]
    assert round(acc.avg_rows_per_expert(s["batch"], s["k"], s["n_experts_hier"]), 3) == s["rows_per_expert"]
    assert round(100 * (1 - s["k"] / s["sparsity_experts"]), 3) == s["sparsity_pct"]
    total = s["mt_expert_params_M"] * 1e6 * s["mt_experts"] * s["mt_layers"]
    assert round(total / 1e9, 2) == s["mt_expert_total_B"]


def test_deepseek_storage_and_activation_rate():
    v = GOLD["deepseek_v3"]
    P = v["total_params_B"] * 1e9
    assert acc.storage_bytes(P, 16) / 1e12 == pytest.approx(v["storage_16bit_TB"])
    assert acc.storage_bytes(P, 8) / 1e9 == pytest.approx(v["storage_8bit_GB"])
    assert acc.storage_bytes(P, 4) / 1e9 == pytest.approx(v["storage_4bit_GB"])
    assert round(100 * v["active_params_B"] / v["total_params_B"], 1) == v["activation_rate_pct"]


def test_deepseek_layer_shape_of_the_workload():
    """One DSV3-shaped MoE layer: 256 routed SwiGLU experts of d_ff 2048 at
    d = 7168 (the workload's shape), top-8 + 1 shared active."""
    v = GOLD["deepseek_v3"]
    P_e = acc.expert_params(7168, 2048, "swiglu")
    routed = v["routed_experts"] * P_e
    active = (v["top_k"] + v["shared_experts"]) * P_e
    assert routed == 11_274_289_152
    assert active == 396_361_728
    # stored in bf16 the routed experts of one layer take about 22.6 GB of HBM
    assert acc.storage_bytes(routed + P_e, 16) / 1e9 == pytest.approx(22.64, abs=0.01)


def test_uniform_share():
    assert 100 / 8 == GOLD["uniform_routing_share_pct_E8"]
