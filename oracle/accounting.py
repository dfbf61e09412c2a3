"""Parameter and storage accounting of sparse MoE models (closed forms).

TEST INFRASTRUCTURE ONLY (see the oracle package docstring).

CS25 "Lecture29" notes, section "Formula page and parameter table":
    P_total  ~ P_embed + N (P_s + E P_e)
    P_active ~ P_embed + N (P_s + k P_e)
with P_s the per-layer shared parameters (attention, router, norms) and P_e
the parameters of one expert MLP.  A SwiGLU expert has three d x d_ff
matrices (W1, W3 up, W2 down; section "Dense baseline"); a one-hidden-layer
ReLU expert has two (Shazeer notes, section 2.2: [512x1024]+[1024x512]).
Weight storage is P * bits / 8 bytes (awesome-ai-roadmap 19.4 table).
"""
from __future__ import annotations


def expert_params(d: int, d_ff: int, act: str) -> int:
    return (3 if act == "swiglu" else 2) * d * d_ff


def attention_params_gqa(d: int, n_q_heads: int, n_kv_heads: int) -> int:
    """Wq, Wo: d x d; Wk, Wv: d x (n_kv * head_dim) (Lecture29, section
    "MHA, MQA and GQA": GQA shares one K/V head among a group of query heads)."""
    hd = d // n_q_heads
    return 2 * d * d + 2 * d * n_kv_heads * hd


def layer_shared_params(d: int, n_q_heads: int, n_kv_heads: int, E: int) -> int:
    """Attention + router (E x d) + the two RMSNorm gains (d each)."""
    return attention_params_gqa(d, n_q_heads, n_kv_heads) + E * d + 2 * d


def total_params(P_embed: int, N: int, P_s: int, E: int, P_e: int) -> int:
    return P_embed + N * (P_s + E * P_e)


def active_params(P_embed: int, N: int, P_s: int, k: int, P_e: int) -> int:
    return P_embed + N * (P_s + k * P_e)


def expert_fraction(P_s: int, k: int, P_e: int) -> float:
    """rho = k P_e / (P_s + k P_e): share of a layer's active parameters that
    sit in the experts (Lecture29, section "Myth 2")."""
    return k * P_e / (P_s + k * P_e)


def storage_bytes(params: float, bits: int) -> float:
    return params * bits / 8.0


def avg_rows_per_expert(batch: int, k: int, n_experts: int) -> float:
    """k b / n: the batch-shrinkage count of Shazeer notes, section 2.3."""
    return k * batch / n_experts
