"""CPU oracle for the sparse token-choice MoE FFN layer forward.

TEST INFRASTRUCTURE ONLY: only ``tests/``, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product path (the HIP library
and its binding) never imports, links or calls anything here, and this package
imports nothing from it.

The arithmetic lives in ``oracle.c`` (plain C, compiled with gcc, OpenMP over
tokens and rows).  This module only marshals numpy arrays through ctypes and
strings the stages together in the order the pages give them:
route -> dispatch (permute by expert) -> experts -> combine (CS25
"Lecture29" notes, section "Top-two routing", minimal pseudocode;
awesome-ai-roadmap ch. 19, section 19.3.2).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

GATES = {"softmax_topk": 0, "softmax_full": 1, "noisy_topk": 2, "sigmoid_bias": 3, "expert_choice": 4, "hash": 5, "hierarchical": 6}
ACTS = {"relu": 0, "swiglu": 1}
MAP_FN = {"exp": 0, "log": 1, "log1p": 2, "softplus": 3, "sigmoid": 4, "sin": 5, "cos": 6}


class _Cfg(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int32), ("d", ctypes.c_int32), ("F", ctypes.c_int32),
        ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("act_bf16", ctypes.c_int32),
        ("act", ctypes.c_int32), ("gate", ctypes.c_int32),
        ("capacity_factor", ctypes.c_double), ("residual", ctypes.c_int32),
        ("n_shared", ctypes.c_int32), ("F_shared", ctypes.c_int32),
        ("round_intermediates", ctypes.c_int32), ("pad_", ctypes.c_int32),
        ("seed", ctypes.c_uint64), ("noise_offset", ctypes.c_uint64),
        ("n_groups", ctypes.c_int32), ("group_k", ctypes.c_int32),
    ]


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (no fast-math, no fp contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-fvisibility=hidden", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        L.oc_exp.restype = ctypes.c_float
        L.oc_exp.argtypes = [ctypes.c_float]
        L.oc_map_f32.argtypes = [ctypes.c_int32, P, P, ctypes.c_int64]
        L.oc_normal.restype = ctypes.c_float
        L.oc_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64]
        L.oc_hash_key.restype = ctypes.c_float
        L.oc_hash_key.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64]
        L.oc_normal_batch.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, P]
        L.oc_philox4x32_10.argtypes = [P, P, P]
        L.oc_route.restype = ctypes.c_int
        L.oc_route.argtypes = [ctypes.POINTER(_Cfg)] + [P] * 16
        L.oc_capacity.restype = ctypes.c_int64
        L.oc_capacity.argtypes = [ctypes.POINTER(_Cfg)]
        L.oc_reroute.restype = ctypes.c_int64
        L.oc_reroute.argtypes = [ctypes.POINTER(_Cfg), P, P]
        L.oc_dispatch.restype = ctypes.c_int64
        L.oc_dispatch.argtypes = [ctypes.POINTER(_Cfg)] + [P] * 6
        L.oc_gather_rows.argtypes = [ctypes.POINTER(_Cfg), P, P, ctypes.c_int64, P]
        L.oc_expert_ffn.argtypes = [ctypes.POINTER(_Cfg), ctypes.c_int32, P, ctypes.c_int64, P, P, P, P]
        L.oc_combine.argtypes = [ctypes.POINTER(_Cfg), P, ctypes.c_int64, P, P, P, P, P, P]
        L.oc_stats.argtypes = [ctypes.POINTER(_Cfg), P, P, P, P, P, P, P]
        L.oc_balance.restype = ctypes.c_int
        L.oc_balance.argtypes = [ctypes.POINTER(_Cfg), ctypes.c_int32] + [P] * 12
        L.oc_update_bias.argtypes = [ctypes.c_int32, P, ctypes.c_float, P]
        L.oc_ec_capacity.restype = ctypes.c_int64
        L.oc_ec_capacity.argtypes = [ctypes.POINTER(_Cfg)]
        L.oc_route_ec.restype = ctypes.c_int
        L.oc_route_ec.argtypes = [ctypes.POINTER(_Cfg), P, P, P, P, P, P, P, P]
        _lib = L
    return _lib


# --------------------------------------------------------------------------
# array marshalling
# --------------------------------------------------------------------------

def _np(a, dtype=None) -> Optional[np.ndarray]:
    """torch tensor / numpy array -> contiguous host numpy array.  bf16 tensors
    become uint16 arrays holding the raw bits."""
    if a is None:
        return None
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach()
            if a.device.type != "cpu":
                a = a.cpu()
            if a.dtype == torch.bfloat16:
                a = a.contiguous().view(torch.int16).numpy().view(np.uint16)
            else:
                a = a.contiguous().numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(a)
    if dtype is not None and a.dtype != dtype:
        a = a.astype(dtype)
    return a


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _act_dtype(cfg) -> str:
    return getattr(cfg, "act_dtype", "f32")


def make_cfg(cfg, *, round_intermediates: bool = True, seed: Optional[int] = None,
             noise_offset: int = 0, T: Optional[int] = None) -> _Cfg:
    c = _Cfg()
    c.T = cfg.T if T is None else T
    c.d, c.F, c.E, c.k = cfg.d, cfg.F, cfg.E, cfg.k
    c.act_bf16 = 1 if _act_dtype(cfg) == "bf16" else 0
    c.act = ACTS[cfg.act]
    c.gate = GATES[cfg.gate]
    c.capacity_factor = float(cfg.capacity_factor)
    c.residual = 1 if cfg.residual else 0
    c.n_shared, c.F_shared = cfg.n_shared, cfg.F_shared
    c.round_intermediates = 1 if round_intermediates else 0
    c.seed = cfg.seed if seed is None else seed
    c.noise_offset = noise_offset
    c.n_groups = getattr(cfg, "n_groups", 0)
    c.group_k = getattr(cfg, "group_top_k", 0)
    return c


def act_to_f64(a, act_dtype: str) -> np.ndarray:
    """Activation-dtype array (fp32, or bf16 bits as uint16) -> fp64 values."""
    a = _np(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


# --------------------------------------------------------------------------
# scalar functions and the noise stream
# --------------------------------------------------------------------------

def map_f32(fn: str, x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty_like(x)
    lib().oc_map_f32(MAP_FN[fn], _ptr(x), _ptr(y), x.size)
    return y


def normal(seed: int, offset: int, first: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    lib().oc_normal_batch(seed, offset, first, n, _ptr(out))
    return out


def philox4x32_10(ctr: Sequence[int], key: Sequence[int]) -> np.ndarray:
    c = np.asarray(ctr, dtype=np.uint32)
    kk = np.asarray(key, dtype=np.uint32)
    out = np.empty(4, dtype=np.uint32)
    lib().oc_philox4x32_10(_ptr(c), _ptr(kk), _ptr(out))
    return out


# --------------------------------------------------------------------------
# stages
# --------------------------------------------------------------------------

def hash_key(seed: int, offset: int, i: int) -> float:
    """Hash-routing key of flat element i = token_id * E + expert."""
    return float(lib().oc_hash_key(seed, offset, i))


def route(cfg, x, w_router, *, logit_bias=None, sel_bias=None, w_noise=None, noise=None,
          seed: Optional[int] = None, noise_offset: int = 0, want_probs: bool = False,
          token_ids=None, w_group_router=None) -> Dict[str, np.ndarray]:
    """Router logits, scores, top-k indices, gates and P for all tokens.
    ``noise`` [T][E] fp32, or None to draw it from the Philox stream.
    Expert choice returns E slots per token (idx -1 where the expert did not
    take the token) and its scores S as ``keys``."""
    xa = _np(x)
    T = xa.shape[0]
    if cfg.gate == "expert_choice":
        c = make_cfg(cfg, T=T)
        E = cfg.E
        idx = np.empty((T, E), dtype=np.int32)
        gates = np.empty((T, E), dtype=np.float64)
        S = np.empty((T, E), dtype=np.float32)
        z = np.empty((T, E), dtype=np.float32)
        P = np.empty(E, dtype=np.float64)
        rc = lib().oc_route_ec(ctypes.byref(c), _ptr(xa), _ptr(_np(w_router, np.float32)),
                               _ptr(_np(logit_bias, np.float32)), _ptr(idx), _ptr(gates), _ptr(S), _ptr(z),
                               _ptr(P))
        if rc != 0:
            raise ValueError("oracle route rejected the configuration")
        out = dict(idx=idx, gates=gates, keys=S, logits=z, P=P, status=0)
        if want_probs:
            out["probs"] = S.astype(np.float64)
        return out
    c = make_cfg(cfg, seed=seed, noise_offset=noise_offset, T=T)
    wr = _np(w_router, np.float32)
    lb = _np(logit_bias, np.float32)
    sb = _np(sel_bias, np.float32)
    wn = _np(w_noise, np.float32)
    nz = _np(noise, np.float32)
    E, k = cfg.E, cfg.k
    idx = np.empty((T, k), dtype=np.int32)
    gates = np.empty((T, k), dtype=np.float64)
    keys = np.empty((T, E), dtype=np.float32)
    logits = np.empty((T, E), dtype=np.float32)
    probs = np.empty((T, E), dtype=np.float64) if want_probs else None
    P = np.empty(E, dtype=np.float64)
    status = np.zeros(1, dtype=np.int32)
    nscale = np.empty((T, E), dtype=np.float32) if cfg.gate == "noisy_topk" else None
    rc = lib().oc_route(ctypes.byref(c), _ptr(xa), _ptr(wr), _ptr(lb), _ptr(sb), _ptr(wn), _ptr(nz),
                        _ptr(idx), _ptr(gates), _ptr(keys), _ptr(logits), _ptr(probs), _ptr(P), _ptr(status),
                        _ptr(nscale), _ptr(_np(token_ids, np.int32)), _ptr(_np(w_group_router, np.float32)))
    if rc != 0:
        raise ValueError("oracle route rejected the configuration")
    out = dict(idx=idx, gates=gates, keys=keys, logits=logits, P=P, status=int(status[0]))
    if want_probs:
        out["probs"] = probs
    if nscale is not None:
        out["noise_scale"] = nscale
    return out


def capacity(cfg, T: Optional[int] = None) -> int:
    c = make_cfg(cfg, T=T)
    if cfg.gate == "expert_choice":
        return int(lib().oc_ec_capacity(ctypes.byref(c)))
    return int(lib().oc_capacity(ctypes.byref(c)))


def slots(cfg) -> int:
    """Selection slots per token: k for token choice, E for expert choice."""
    return cfg.E if cfg.gate == "expert_choice" else cfg.k


def _slot_cfg(cfg):
    # dispatch / combine see one slot per (token, expert) under expert
    # choice, and no capacity cut (the selection already took C per expert)
    if cfg.gate == "expert_choice":
        return cfg.replace(k=cfg.E, capacity_factor=0.0)
    return cfg


def reroute(cfg, keys, idx) -> np.ndarray:
    """Capacity reroute of the route's selection (a new idx array): the
    assignments past an expert's capacity move, in (t, j) order, to their
    token's best other expert with room."""
    idx = np.array(_np(idx, np.int32), dtype=np.int32, copy=True)
    keys = _np(keys, np.float32)
    c = make_cfg(cfg, T=idx.shape[0])
    lib().oc_reroute(ctypes.byref(c), _ptr(keys), _ptr(idx))
    return idx


def dispatch(cfg, idx, T: Optional[int] = None) -> Dict[str, np.ndarray]:
    idx = _np(idx, np.int32)
    T = idx.shape[0] if T is None else T
    C = capacity(cfg, T)
    cfg = _slot_cfg(cfg)
    c = make_cfg(cfg, T=T)
    E, k = cfg.E, cfg.k
    counts = np.empty(E, np.int32)
    kept = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm_src = np.full(T * k, -1, np.int32)
    slot_pos = np.empty(T * k, np.int32)
    R = lib().oc_dispatch(ctypes.byref(c), _ptr(idx), _ptr(counts), _ptr(kept), _ptr(offsets),
                          _ptr(perm_src), _ptr(slot_pos))
    return dict(counts=counts, kept=kept, offsets=offsets, perm_src=perm_src[:R].copy(),
                slot_pos=slot_pos.reshape(T, k), R=int(R), C=C)


def gather_rows(cfg, x, perm_src) -> np.ndarray:
    xa = _np(x)
    ps = _np(perm_src, np.int32)
    R = ps.shape[0]
    out = np.empty((R, cfg.d), dtype=xa.dtype)
    c = make_cfg(_slot_cfg(cfg), T=xa.shape[0])
    lib().oc_gather_rows(ctypes.byref(c), _ptr(xa), _ptr(ps), R, _ptr(out))
    return out


def expert_ffn(cfg, a_rows, w1, w3, w2, *, F: Optional[int] = None,
               round_intermediates: bool = True) -> np.ndarray:
    """One expert on rows a_rows [n][d]; w1/w3 [F][d], w2 [d][F] (w3 None for ReLU)."""
    a = _np(a_rows)
    n = a.shape[0]
    F = cfg.F if F is None else F
    c = make_cfg(cfg, round_intermediates=round_intermediates)
    w1a, w3a, w2a = _np(w1), _np(w3), _np(w2)
    y = np.empty((n, cfg.d), dtype=np.float64)
    if n:
        lib().oc_expert_ffn(ctypes.byref(c), F, _ptr(a), n, _ptr(w1a), _ptr(w3a), _ptr(w2a), _ptr(y))
    return y


def combine(cfg, slot_pos, gates, y, x, shared=None, tokens=None,
            round_intermediates: bool = True) -> np.ndarray:
    sp = _np(slot_pos, np.int32)
    T = sp.shape[0]
    g = _np(gates, np.float64)
    ya = _np(y, np.float64)
    xa = _np(x)
    sh = _np(shared, np.float64)
    tok = _np(tokens, np.int32)
    ntok = T if tok is None else tok.shape[0]
    c = make_cfg(_slot_cfg(cfg), round_intermediates=round_intermediates, T=T)
    out = np.empty((ntok, cfg.d), dtype=np.float64)
    lib().oc_combine(ctypes.byref(c), _ptr(tok), ntok, _ptr(sp), _ptr(g), _ptr(ya), _ptr(xa), _ptr(sh), _ptr(out))
    return out


def stats(cfg, counts, kept, P, T: int) -> Dict[str, object]:
    c = make_cfg(cfg, T=T)
    counts = _np(counts, np.int32)
    kept = _np(kept, np.int32)
    P = _np(P, np.float64)
    f = np.empty(cfg.E, np.float64)
    nd = np.zeros(1, np.int64)
    imb = np.zeros(1, np.float64)
    aux = np.zeros(1, np.float64)
    lib().oc_stats(ctypes.byref(c), _ptr(counts), _ptr(kept), _ptr(P), _ptr(f), _ptr(nd), _ptr(imb), _ptr(aux))
    return dict(f=f, n_dropped=int(nd[0]), imbalance=float(imb[0]), aux=float(aux[0]))


def balance(cfg, r, seq_len: int = 0) -> Dict[str, object]:
    """Router z-loss, importance and load (with their CV^2) and the
    sequence-wise balance term from the outputs of route(..., want_probs=True)."""
    T = r["idx"].shape[0]
    c = make_cfg(cfg, T=T)
    E = cfg.E
    imp = np.empty(E, np.float64)
    load = np.full(E, np.nan, np.float64)
    z = np.zeros(1, np.float64)
    icv = np.zeros(1, np.float64)
    lcv = np.full(1, np.nan, np.float64)
    sa = np.zeros(1, np.float64)
    ns = r.get("noise_scale")
    rc = lib().oc_balance(ctypes.byref(c), int(seq_len), _ptr(_np(r["logits"], np.float32)),
                          _ptr(_np(r["keys"], np.float32)), _ptr(None if ns is None else _np(ns, np.float32)),
                          _ptr(_np(r["probs"], np.float64)), _ptr(_np(r["idx"], np.int32)),
                          _ptr(_np(r["gates"], np.float64)), _ptr(z), _ptr(imp), _ptr(icv), _ptr(load),
                          _ptr(lcv), _ptr(sa))
    if rc != 0:
        raise ValueError("seq_len must divide T")
    return dict(z_loss=float(z[0]), importance=imp, importance_cv2=float(icv[0]), load=load,
                load_cv2=float(lcv[0]), seq_aux=float(sa[0]))


def update_bias(counts, bias, gamma: float) -> np.ndarray:
    """The auxiliary-loss-free bias step b += gamma * sign(mean count - count)."""
    counts = _np(counts, np.int32)
    b = np.array(_np(bias, np.float32), dtype=np.float32, copy=True)
    lib().oc_update_bias(int(counts.shape[0]), _ptr(counts), ctypes.c_float(gamma), _ptr(b))
    return b


# --------------------------------------------------------------------------
# whole layer
# --------------------------------------------------------------------------

def expert_weights(cfg, inputs, e: int):
    """(w1, w3, w2) host arrays of routed expert e (w3 None for ReLU)."""
    if cfg.act == "swiglu":
        return _np(inputs["w_gate"][e]), _np(inputs["w_up"][e]), _np(inputs["w_down"][e])
    return _np(inputs["w1"][e]), None, _np(inputs["w2"][e])


def shared_weights(inputs):
    return _np(inputs["ws_gate"][0]), _np(inputs["ws_up"][0]), _np(inputs["ws_down"][0])


def forward(cfg, inputs, *, round_intermediates: bool = True, noise: str = "input",
            noise_offset: int = 0) -> Dict[str, object]:
    """Whole layer on the CPU, every token.  ``noise`` selects where the noisy
    gate's Gaussian draws come from: "input" (inputs["noise"]) or "philox"."""
    x = _np(inputs["x"])
    T = x.shape[0]
    nz = inputs.get("noise") if (cfg.gate == "noisy_topk" and noise == "input") else None
    r = route(cfg, x, inputs["w_router"], logit_bias=inputs.get("logit_bias"),
              sel_bias=inputs.get("sel_bias"), w_noise=inputs.get("w_noise"), noise=nz,
              noise_offset=noise_offset, want_probs=True, token_ids=inputs.get("token_ids"),
              w_group_router=inputs.get("w_group_router"))
    if getattr(cfg, "reroute", False):
        r["idx"] = reroute(cfg, r["keys"], r["idx"])
    dp = dispatch(cfg, r["idx"], T=T)
    x_perm = gather_rows(cfg, x, dp["perm_src"])
    R = dp["R"]
    y = np.zeros((R, cfg.d), dtype=np.float64)
    off = dp["offsets"]
    for e in range(cfg.E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            w1, w3, w2 = expert_weights(cfg, inputs, e)
            y[lo:hi] = expert_ffn(cfg, x_perm[lo:hi], w1, w3, w2, round_intermediates=round_intermediates)
    shared = None
    if cfg.n_shared:
        s1, s3, s2 = shared_weights(inputs)
        shared = expert_ffn(cfg, x, s1, s3, s2, F=cfg.F_shared, round_intermediates=round_intermediates)
    out = combine(cfg, dp["slot_pos"], r["gates"], y, x, shared=shared,
                  round_intermediates=round_intermediates)
    st = stats(cfg, dp["counts"], dp["kept"], r["P"], T)
    res = dict(r)
    res.update(dp)
    res.update(st)
    res.update(x_perm=x_perm, y=y, shared=shared, out=out)
    return res
