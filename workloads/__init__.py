"""Seeded synthetic workloads for the sparse token-choice MoE FFN layer.

This module holds the nine layer shapes and a deterministic input generator.
It contains none of the layer's arithmetic: it only draws tensors.  Both the
HIP path and the CPU oracle take their inputs from here, and nothing here
imports either of them.

Shapes and distributions follow the layer configurations studied on the pages:

* ``tiny``     top-2 of 8 SwiGLU experts, fp32 (the Mixtral routing rule of
               "Lecture29", section "Top-two routing", at toy size).
* ``switch``   top-1 of 64 ReLU experts 512->1024->512, fp32, capacity
               factor 1.25 with overflow dropped to the residual ("Switch
               Transformers" lesson, points (3) and the token-drop answer).
* ``noisy``    Shazeer noisy top-4 of 256 ReLU experts 512->1024->512, bf16
               ("Outrageously Large Neural Networks" reading notes, section 2.2
               symbol tables and the 1M-parameter expert shape).
* ``mixtral``  Mixtral-8x7B-shaped layer: d=4096, d_ff=14336, top-2 of 8
               SwiGLU experts, bf16 ("Lecture29", sections "Top-two routing"
               and "Mixtral 8x7B").
* ``dsv3``     DeepSeek-V3-shaped layer: d=7168, 256 routed SwiGLU experts of
               d_ff 2048 plus one shared expert, sigmoid affinity with a
               selection-only bias, top-8 ("awesome-ai-roadmap" ch. 19,
               sections 19.3.4 and 19.5; CS336 lecture 4 notes, section 12).
* ``mixtral_ec`` the Mixtral-shaped layer routed by expert choice: each of
               the 8 experts takes the T k / E = 1024 tokens of highest router
               probability (CS336 lecture 4 notes, section 4; "awesome-ai-
               roadmap" 19.6.1), so every expert GEMM has the same M.
* ``mixtral_hash`` the Mixtral-shaped layer routed by a hash of Zipf(1.1)
               token ids, top-2 with the outputs summed (CS336 lecture 4
               notes, section 4, hash routing).
* ``hier``     the Shazeer-shaped layer (256 ReLU experts 512->1024->512,
               bf16) under a two-level gate: 16 groups of 16 experts, 2
               groups then 2 experts each, k = 4 ("Outrageously Large Neural
               Networks" reading notes, appendix B hierarchical MoE and the
               2 x 2 remark).
* ``switch_reroute`` the Switch workload with capacity overflow rerouted to
               each token's next expert with room instead of dropped
               (Lecture29, "Inference load balance": drop, reroute or delay).

Distributions: x ~ N(0,1); every weight ~ N(0, 1/fan_in); the DeepSeek-style
selection bias ~ N(0, 0.1) read as a variance; the Switch logit bias is
b_e = -1.1*ln(1 + pi(e)) for a seeded permutation pi, so that softmax(b) alone
is a Zipf(1.1) law over experts.  Weights of bf16 configs are drawn in fp32
and rounded to bf16 (round-to-nearest-even).  The router (and the noise-scale
matrix) are always fp32.

Values depend on the device the generator runs on (torch's CPU and GPU
generators differ), so a test that compares two paths draws once and hands
the same tensors to both.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch

__all__ = ["Config", "CONFIGS", "get", "make_inputs", "make_output_grad", "expert_tensor_names"]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    T: int                      # tokens per call
    d: int                      # d_model
    F: int                      # expert d_ff
    E: int                      # routed experts
    k: int                      # top-k
    act_dtype: str              # "f32" | "bf16": activations and expert weights
    act: str                    # "relu" | "swiglu"
    gate: str                   # "softmax_topk" | "softmax_full" | "noisy_topk" | "sigmoid_bias" | "expert_choice"
                                #  | "hash" | "hierarchical"
    capacity_factor: float = 0.0  # <= 0: dropless
    residual: bool = False
    n_shared: int = 0
    F_shared: int = 0
    logit_bias: str = "none"    # "none" | "zipf"
    sel_bias: bool = False
    seed: int = 0
    n_groups: int = 0           # hierarchical gate: groups of E / n_groups experts
    group_top_k: int = 0        # hierarchical gate: groups picked per token
    reroute: bool = False       # capacity overflow moves to the token's next expert instead of dropping

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.act_dtype == "f32" else torch.bfloat16


CONFIGS: Dict[str, Config] = {
    "tiny": Config("tiny", T=256, d=128, F=256, E=8, k=2, act_dtype="f32",
                   act="swiglu", gate="softmax_topk", seed=1001),
    "switch": Config("switch", T=2048, d=512, F=1024, E=64, k=1, act_dtype="f32",
                     act="relu", gate="softmax_full", capacity_factor=1.25,
                     residual=True, logit_bias="zipf", seed=1002),
    "noisy": Config("noisy", T=8192, d=512, F=1024, E=256, k=4, act_dtype="bf16",
                    act="relu", gate="noisy_topk", seed=1003),
    "mixtral": Config("mixtral", T=4096, d=4096, F=14336, E=8, k=2, act_dtype="bf16",
                      act="swiglu", gate="softmax_topk", seed=1004),
    "dsv3": Config("dsv3", T=4096, d=7168, F=2048, E=256, k=8, act_dtype="bf16",
                   act="swiglu", gate="sigmoid_bias", n_shared=1, F_shared=2048,
                   sel_bias=True, seed=1005),
    "mixtral_ec": Config("mixtral_ec", T=4096, d=4096, F=14336, E=8, k=2, act_dtype="bf16",
                         act="swiglu", gate="expert_choice", capacity_factor=1.0, seed=1006),
    "mixtral_hash": Config("mixtral_hash", T=4096, d=4096, F=14336, E=8, k=2, act_dtype="bf16",
                           act="swiglu", gate="hash", seed=1007),
    "hier": Config("hier", T=8192, d=512, F=1024, E=256, k=4, act_dtype="bf16", act="relu",
                   gate="hierarchical", n_groups=16, group_top_k=2, seed=1008),
    "switch_reroute": Config("switch_reroute", T=2048, d=512, F=1024, E=64, k=1, act_dtype="f32",
                             act="relu", gate="softmax_full", capacity_factor=1.25, residual=True,
                             logit_bias="zipf", reroute=True, seed=1002),
}


def get(name: str) -> Config:
    return CONFIGS[name]


def expert_tensor_names(cfg: Config):
    """Names of the per-expert weight tensors, in draw order."""
    if cfg.act == "swiglu":
        return ("w_gate", "w_up", "w_down")
    return ("w1", "w2")


def _normal(shape, std: float, gen: torch.Generator, device, out_dtype) -> torch.Tensor:
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t if out_dtype == torch.float32 else t.to(out_dtype)


def _expert_stack(E: int, rows: int, cols: int, gen, device, dtype) -> torch.Tensor:
    """[E][rows][cols] weights ~ N(0, 1/cols), drawn one expert at a time."""
    out = torch.empty((E, rows, cols), dtype=dtype, device=device)
    std = 1.0 / math.sqrt(cols)
    for e in range(E):
        out[e].copy_(_normal((rows, cols), std, gen, device, dtype))
    return out


def make_inputs(cfg: Config, device="cpu", with_noise: Optional[bool] = None) -> Dict[str, torch.Tensor]:
    """Draw every tensor of one layer call, deterministically from ``cfg.seed``.

    Returns a dict with ``x`` [T][d], ``w_router`` [E][d] fp32 and, as the
    config asks, ``w_noise`` [E][d] fp32, ``noise`` [T][E] fp32 (standard
    normal draws for the noisy gate, used when the caller passes the noise
    in), ``logit_bias`` [E], ``sel_bias`` [E], the expert stacks
    (``w_gate``/``w_up`` [E][F][d] and ``w_down`` [E][d][F] for SwiGLU,
    ``w1`` [E][F][d] and ``w2`` [E][d][F] for ReLU) and the shared expert
    (``ws_gate``/``ws_up`` [S][Fs][d], ``ws_down`` [S][d][Fs]); for the hash
    gate ``token_ids`` [T] int32, for the hierarchical gate ``w_group_router``
    [n_groups][d] fp32.
    Weight layouts are [out][in] (the reduction dimension is contiguous).
    """
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(cfg.seed)
    dt = cfg.torch_dtype
    T, d, F, E = cfg.T, cfg.d, cfg.F, cfg.E
    inp: Dict[str, torch.Tensor] = {}
    inp["x"] = _normal((T, d), 1.0, gen, device, dt)
    inp["w_router"] = _normal((E, d), 1.0 / math.sqrt(d), gen, device, torch.float32)
    if cfg.gate == "noisy_topk":
        inp["w_noise"] = _normal((E, d), 1.0 / math.sqrt(d), gen, device, torch.float32)
    if cfg.logit_bias == "zipf":
        perm = torch.randperm(E, generator=gen, device=device)
        inp["logit_bias"] = (-1.1 * torch.log1p(perm.to(torch.float64))).to(torch.float32)
    if cfg.sel_bias:
        inp["sel_bias"] = _normal((E,), math.sqrt(0.1), gen, device, torch.float32)
    if cfg.act == "swiglu":
        inp["w_gate"] = _expert_stack(E, F, d, gen, device, dt)
        inp["w_up"] = _expert_stack(E, F, d, gen, device, dt)
        inp["w_down"] = _expert_stack(E, d, F, gen, device, dt)
    else:
        inp["w1"] = _expert_stack(E, F, d, gen, device, dt)
        inp["w2"] = _expert_stack(E, d, F, gen, device, dt)
    if cfg.n_shared:
        S, Fs = cfg.n_shared, cfg.F_shared
        inp["ws_gate"] = _expert_stack(S, Fs, d, gen, device, dt)
        inp["ws_up"] = _expert_stack(S, Fs, d, gen, device, dt)
        inp["ws_down"] = _expert_stack(S, d, Fs, gen, device, dt)
    if with_noise is None:
        with_noise = cfg.gate == "noisy_topk"
    if with_noise:
        inp["noise"] = _normal((T, E), 1.0, gen, device, torch.float32)
    if cfg.gate == "hierarchical":
        inp["w_group_router"] = _normal((cfg.n_groups, d), 1.0 / math.sqrt(d), gen, device, torch.float32)
    if cfg.gate == "hash":
        # token ids with a Zipf(1.1) law over a 32000-id vocabulary, so that
        # frequent ids repeat (CS336 notes section 4: under a Zipf law a word
        # like "the" can dominate one expert)
        ranks = torch.arange(1, 32001, dtype=torch.float64, device=device)
        w = ranks.pow(-1.1)
        inp["token_ids"] = torch.multinomial(w / w.sum(), T, replacement=True, generator=gen).to(torch.int32)
    return inp


def make_output_grad(cfg: Config, device="cpu") -> torch.Tensor:
    """The gradient dL/dout [T][d] of one backward call: standard normal in
    the activation dtype, from its own stream (seed + 7919) so the forward
    inputs do not change."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(cfg.seed + 7919)
    return _normal((cfg.T, cfg.d), 1.0, gen, device, cfg.torch_dtype)
