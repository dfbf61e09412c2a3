"""Brute-force dense evaluation of the MoE layer in numpy fp64.

TEST INFRASTRUCTURE ONLY (see the oracle package docstring).

This is the layer written the way the pages state it, with no permutation at
all: every expert is evaluated on every token and the outputs are mixed with
the dense gate vector G(x), which is zero outside the selected set
(CS25 "Lecture29" notes, section "Top-two routing": y = sum over all E experts
of g_i(x) Expert_i(x); Shazeer notes, section 2.2: G(x) is a sparse
n-dimensional vector and E_i need not be computed where G(x)_i = 0).
Capacity drops are applied by walking the tokens in order and zeroing a gate
once its expert has accepted C assignments.

It uses fp64 throughout (logits included) and its own selection, so it shares
nothing with the C oracle beyond the inputs.  Meant for tiny inputs only.
"""
from __future__ import annotations

import math
from typing import Dict

import numpy as np

from . import _np, act_to_f64


def _softplus(v):
    return np.logaddexp(0.0, v)


def dense_gates(cfg, x64, w_router, *, logit_bias=None, sel_bias=None, w_noise=None, noise=None):
    """Returns (G [T][E] dense gates before drops, S [T][k] selected experts in
    slot order, key [T][E] fp64 selection scores)."""
    W = _np(w_router).astype(np.float64)
    z = x64 @ W.T
    if logit_bias is not None:
        z = z + _np(logit_bias).astype(np.float64)[None, :]
    if cfg.gate == "noisy_topk":
        zn = x64 @ _np(w_noise).astype(np.float64).T
        key = z + _np(noise).astype(np.float64) * _softplus(zn)
    elif cfg.gate == "sigmoid_bias":
        s = 1.0 / (1.0 + np.exp(-z))
        key = s + (_np(sel_bias).astype(np.float64)[None, :] if sel_bias is not None else 0.0)
    else:
        key = z
    T, E = z.shape
    k = cfg.k
    S = np.empty((T, k), dtype=np.int64)
    G = np.zeros((T, E), dtype=np.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-key[t, e], e))
        sel = order[:k]
        S[t] = sel
        if cfg.gate == "softmax_full":
            w = np.exp(z[t] - z[t].max())
            w = w / w.sum()
            for e in sel:
                G[t, e] = w[e]
        elif cfg.gate == "sigmoid_bias":
            s = 1.0 / (1.0 + np.exp(-z[t, sel]))
            for e, v in zip(sel, s / s.sum()):
                G[t, e] = v
        else:
            src = key[t] if cfg.gate == "noisy_topk" else z[t]
            masked = np.full(E, -np.inf)
            masked[sel] = src[sel]
            w = np.exp(masked - masked.max())
            G[t] = w / w.sum()
    return G, S, key


def expert_dense(cfg, x64, w1, w3, w2):
    """Expert applied to all rows, fp64 (SwiGLU or ReLU)."""
    a = x64 @ act_to_f64(w1, cfg.act_dtype).T
    if cfg.act == "swiglu":
        u = x64 @ act_to_f64(w3, cfg.act_dtype).T
        h = a / (1.0 + np.exp(-a)) * u
    else:
        h = np.maximum(a, 0.0)
    return h @ act_to_f64(w2, cfg.act_dtype).T


def forward(cfg, inputs, noise=None) -> Dict[str, np.ndarray]:
    x64 = act_to_f64(inputs["x"], cfg.act_dtype)
    T = x64.shape[0]
    G, S, key = dense_gates(cfg, x64, inputs["w_router"], logit_bias=inputs.get("logit_bias"),
                            sel_bias=inputs.get("sel_bias"), w_noise=inputs.get("w_noise"),
                            noise=noise if noise is not None else inputs.get("noise"))
    if cfg.capacity_factor > 0:
        C = math.ceil(cfg.capacity_factor * T * cfg.k / cfg.E)
        taken = np.zeros(cfg.E, dtype=np.int64)
        for t in range(T):
            for e in S[t]:
                if taken[e] >= C:
                    G[t, e] = 0.0
                taken[e] += 1
    out = np.zeros((T, cfg.d), dtype=np.float64)
    if cfg.residual:
        out += x64
    for e in range(cfg.E):
        if cfg.act == "swiglu":
            w1, w3, w2 = inputs["w_gate"][e], inputs["w_up"][e], inputs["w_down"][e]
        else:
            w1, w3, w2 = inputs["w1"][e], None, inputs["w2"][e]
        ye = expert_dense(cfg, x64, _np(w1), None if w3 is None else _np(w3), _np(w2))
        out += G[:, e:e + 1] * ye
    if cfg.n_shared:
        out += expert_dense(cfg, x64, _np(inputs["ws_gate"][0]), _np(inputs["ws_up"][0]),
                            _np(inputs["ws_down"][0]))
    return dict(out=out, G=G, S=S, key=key)
