"""CPU oracle for the backward pass of the sparse MoE FFN layer.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only ``tests/``, the
smoke check and the benchmark's CPU-baseline leg may use it.

The layer is trained by ordinary backpropagation through the experts each
token was sent to: the top-k choice is a constant of the step, a masked
(unselected) logit has probability exactly zero and receives zero gradient,
and the selected positions pass a nonzero gradient to the router matrix
(Shazeer et al. reading notes, section 2.1 key points 1 and 2; CS25
"Lecture29" notes, Q&A "Gradient flow and training cost": the gating and
expert operations on the selected path stay differentiable; Switch
Transformers lesson: with one expert the router still learns through the gate
probability that scales the expert output).  This module writes that chain
rule out in numpy float64, stage by stage, from the forward definitions:

  out_t  = [residual] x_t + [shared] S(x_t) + sum_j g_tj  y_{e_tj}(x_t)
  y_e(x) = W2_e h,  h = SiLU(a) * u (SwiGLU) or relu(a) (ReLU),
           a = W1_e x, u = W3_e x
  z_t    = W_r x_t + b   (router logits; the gates g are functions of z)

Given dL/dout = dY it returns dL/dx, the router gradients dL/dW_r and dL/db,
and the expert (and shared expert) weight gradients.  Gate families:
  softmax over the selected logits:  dz_i = g_i (dg_i - sum_j g_j dg_j)
      on the selected experts, 0 elsewhere;
  full softmax p read at the selected experts (and expert choice, whose
      gate of a taken (t, e) is p_te):  dz = p * (dp - <p, dp>), dp_e the
      sum of dg over the slots that hold e;
  sigmoid with selection-only bias: g_i = s_i / sum_sel s, s = sigmoid(z):
      ds_i = (dg_i - sum_j g_j dg_j) / sum_sel s, dz_i = ds_i s_i (1 - s_i);
      the selection bias gets no gradient (it never enters g);
  hash routing: gates are constants, the router gets nothing.
dg_tj = <dY_t, y_{e_tj}(x_t)> for a kept slot and 0 for a dropped one (its
output is zero whatever the gate).
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from . import _np, act_to_f64, expert_weights, shared_weights, slots

SUPPORTED_GATES = ("softmax_topk", "softmax_full", "sigmoid_bias", "expert_choice", "hash")


def _sigmoid(v: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-v))


def expert_backward(cfg, xr: np.ndarray, dyr: np.ndarray, w1, w3, w2) -> Dict[str, np.ndarray]:
    """One expert MLP on rows xr [n][d] with output gradient dyr [n][d].
    w1/w3 [F][d], w2 [d][F] (w3 None for ReLU).  Returns dx [n][d] and the
    weight gradients in the weights' own layouts."""
    W1 = act_to_f64(w1, _dt(cfg))
    W2 = act_to_f64(w2, _dt(cfg))
    a = xr @ W1.T
    if cfg.act == "swiglu":
        W3 = act_to_f64(w3, _dt(cfg))
        u = xr @ W3.T
        sg = _sigmoid(a)
        h = a * sg * u
    else:
        W3 = None
        h = np.maximum(a, 0.0)
    dh = dyr @ W2                       # y = h W2^T
    dw2 = dyr.T @ h
    if cfg.act == "swiglu":
        da = dh * u * sg * (1.0 + a * (1.0 - sg))   # d SiLU(a) / da = s (1 + a (1 - s))
        du = dh * a * sg
        dx = da @ W1 + du @ W3
        return dict(dx=dx, dw1=da.T @ xr, dw3=du.T @ xr, dw2=dw2)
    da = dh * (a > 0.0)
    return dict(dx=da @ W1, dw1=da.T @ xr, dw3=None, dw2=dw2)


def _dt(cfg) -> str:
    return getattr(cfg, "act_dtype", "f32")


def router_backward(cfg, idx: np.ndarray, gates: np.ndarray, logits: np.ndarray, dg: np.ndarray) -> np.ndarray:
    """dL/dz [T][E] from dL/dg [T][slots] for the gate family of cfg."""
    T, E = logits.shape[0], cfg.E
    z = logits.astype(np.float64)
    dz = np.zeros((T, E), np.float64)
    if cfg.gate == "hash":
        return dz
    for t in range(T):
        sel = [(j, int(idx[t, j])) for j in range(idx.shape[1]) if idx[t, j] >= 0]
        if cfg.gate == "softmax_topk":
            g = np.array([gates[t, j] for j, _ in sel])
            d = np.array([dg[t, j] for j, _ in sel])
            c = float(np.dot(g, d))
            for (j, e), gj, dj in zip(sel, g, d):
                dz[t, e] += gj * (dj - c)
        elif cfg.gate in ("softmax_full", "expert_choice"):
            p = np.exp(z[t] - z[t].max())
            p /= p.sum()
            dp = np.zeros(E)
            for j, e in sel:
                dp[e] += dg[t, j]
            dz[t] = p * (dp - np.dot(p, dp))
        elif cfg.gate == "sigmoid_bias":
            s = _sigmoid(z[t])
            ssum = sum(s[e] for _, e in sel)
            g = np.array([s[e] / ssum for _, e in sel])
            d = np.array([dg[t, j] for j, _ in sel])
            c = float(np.dot(g, d))
            for (j, e), dj in zip(sel, d):
                dz[t, e] += (dj - c) / ssum * s[e] * (1.0 - s[e])
        else:
            raise NotImplementedError(f"backward of the {cfg.gate} gate")
    return dz


def backward(cfg, inputs, fwd, dy) -> Dict[str, object]:
    """Gradients of the whole layer for output gradient dy [T][d], given the
    oracle forward ``fwd`` of the same inputs (its routing is the constant
    selection).  Returns fp64 arrays: dx [T][d]; dw_router [E][d];
    dlogit_bias [E]; dw_gate / dw_up / dw_down (or dw1 / dw2 for ReLU) per
    expert in the weight layouts; dws_* for the shared expert; and the
    intermediate dg [T][slots] and dz [T][E]."""
    if cfg.gate not in SUPPORTED_GATES:
        raise NotImplementedError(f"backward of the {cfg.gate} gate")
    if getattr(cfg, "reroute", False):
        raise NotImplementedError("backward after a capacity reroute")
    dt = _dt(cfg)
    x = act_to_f64(inputs["x"], dt)
    dY = act_to_f64(dy, dt)
    T, d, E = x.shape[0], cfg.d, cfg.E
    ns = slots(cfg)
    idx = _np(fwd["idx"], np.int32).reshape(T, ns)
    gates = _np(fwd["gates"], np.float64).reshape(T, ns)
    slot_pos = _np(fwd["slot_pos"], np.int32).reshape(T, ns)
    off = _np(fwd["offsets"], np.int32)
    perm_src = _np(fwd["perm_src"], np.int32)
    y = _np(fwd["y"], np.float64)
    x_perm = act_to_f64(fwd["x_perm"], dt)

    # per kept row r of assignment (t, j): output gradient g_tj dY_t, and the
    # gate gradient <dY_t, y_r>
    dg = np.zeros((T, ns), np.float64)
    R = int(off[E])
    dyp = np.zeros((R, d), np.float64)
    for r in range(R):
        a = int(perm_src[r])
        t, j = divmod(a, ns)
        dyp[r] = gates[t, j] * dY[t]
        dg[t, j] = float(np.dot(dY[t], y[r]))

    dxp = np.zeros((R, d), np.float64)
    grads = {}
    names = ("dw_gate", "dw_up", "dw_down") if cfg.act == "swiglu" else ("dw1", None, "dw2")
    F = cfg.F
    gw1 = np.zeros((E, F, d))
    gw3 = np.zeros((E, F, d)) if cfg.act == "swiglu" else None
    gw2 = np.zeros((E, d, F))
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi <= lo:
            continue
        w1, w3, w2 = expert_weights(cfg, inputs, e)
        b = expert_backward(cfg, x_perm[lo:hi], dyp[lo:hi], w1, w3, w2)
        dxp[lo:hi] = b["dx"]
        gw1[e] = b["dw1"]
        gw2[e] = b["dw2"]
        if gw3 is not None:
            gw3[e] = b["dw3"]
    grads[names[0]] = gw1
    if names[1]:
        grads[names[1]] = gw3
    grads[names[2]] = gw2

    # token gradient: residual, routed experts in slot order, shared expert,
    # router
    dx = np.zeros((T, d), np.float64)
    if cfg.residual:
        dx += dY
    for t in range(T):
        for j in range(ns):
            r = int(slot_pos[t, j])
            if r >= 0:
                dx[t] += dxp[r]
    if cfg.n_shared:
        s1, s3, s2 = shared_weights(inputs)
        b = expert_backward(cfg, x, dY, s1, s3, s2)
        dx += b["dx"]
        grads.update(dws_gate=b["dw1"], dws_up=b["dw3"], dws_down=b["dw2"])
    if cfg.gate == "hash":
        dz = np.zeros((T, E))
    else:
        dz = router_backward(cfg, idx, gates, _np(fwd["logits"], np.float32), dg)
        Wr = _np(inputs["w_router"], np.float64)
        dx += dz @ Wr
    grads.update(dx=dx, dw_router=dz.T @ x, dlogit_bias=dz.sum(axis=0), dg=dg, dz=dz)
    return grads
