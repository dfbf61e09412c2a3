"""Python binding of libmoe.so, the MI355X (gfx950) sparse token-choice MoE layer.

Argument marshalling only: every function takes torch device tensors, checks
their dtype, shape and contiguity, and calls the C entry point of the same
name (include/moe.h) with raw device pointers and the current HIP stream.
All arithmetic runs in the library's HIP kernels.  There is no fallback: if
libmoe.so is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

__all__ = [
    "MoeConfig", "MoeWeights", "MoeStats", "MoeError", "lib", "config", "weights_from", "alloc_stats",
    "workspace", "max_rows", "capacity", "validate_config", "workspace_size",
    "moe_route", "moe_dispatch", "moe_expert_ffn", "moe_expert_up", "moe_expert_down", "moe_shared_expert",
    "moe_combine", "moe_layer_forward", "MoeSaved", "MoeGrads", "backward_workspace_size", "backward_workspace",
    "moe_layer_backward", "moe_expert_up_train", "moe_dispatch_noalloc",
    "EXPORTED_SYMBOLS", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_F32, MOE_BF16 = 0, 1
ACTS = {"relu": 0, "swiglu": 1}
GATES = {"softmax_topk": 0, "softmax_full": 1, "noisy_topk": 2, "sigmoid_bias": 3, "expert_choice": 4, "hash": 5, "hierarchical": 6}
MOE_F_ADD_RESIDUAL, MOE_F_NOISE_INPUT, MOE_F_REROUTE = 1, 2, 4
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported configuration", 3: "workspace missing or too small",
          4: "HIP launch failed"}

EXPORTED_SYMBOLS = (
    "moe_validate_config", "moe_workspace_size", "moe_max_rows", "moe_capacity", "moe_route_slots",
    "moe_last_hip_error",
    "moe_status_string", "moe_route", "moe_dispatch", "moe_expert_ffn", "moe_expert_up", "moe_expert_down",
    "moe_shared_expert", "moe_combine", "moe_layer_forward", "moe_update_bias",
    "moe_backward_workspace_size", "moe_layer_backward", "moe_expert_up_train", "moe_dispatch_noalloc",
)


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, hip: int = 0):
        msg = f"{fn}: {STATUS.get(status, status)}"
        if status == 4:
            msg += f" (hip error {hip})"
        super().__init__(msg)
        self.status = status


class MoeConfig(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int32), ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
        ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("n_shared", ctypes.c_int32),
        ("d_ff_shared", ctypes.c_int32), ("act_dtype", ctypes.c_int32), ("act", ctypes.c_int32),
        ("gate", ctypes.c_int32), ("capacity_factor", ctypes.c_double), ("flags", ctypes.c_uint32),
        ("seed", ctypes.c_uint64), ("noise_offset", ctypes.c_uint64),
        ("seq_len", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("n_groups", ctypes.c_int32), ("group_top_k", ctypes.c_int32),
    ]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_router", "logit_bias", "sel_bias", "w_noise", "noise", "w_gate", "w_up", "w_down",
        "ws_gate", "ws_up", "ws_down", "token_ids", "w_group_router")]


class MoeStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "counts", "kept", "f", "P", "n_dropped", "imbalance", "aux", "device_status",
        "z_loss", "importance", "importance_cv2", "load", "load_cv2", "seq_aux")]


class MoeSaved(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "topk_idx", "topk_gate", "expert_offsets", "perm_src", "slot_pos", "x_perm", "y_perm", "pre_act")]


class MoeGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "dx", "dw_router", "dlogit_bias", "dw_gate", "dw_up", "dw_down", "dws_gate", "dws_up", "dws_down")]


_lib = None


def lib():
    """Load libmoe.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        P, C = ctypes.c_void_p, ctypes.POINTER(MoeConfig)
        L.moe_validate_config.restype = ctypes.c_int
        L.moe_validate_config.argtypes = [C]
        L.moe_workspace_size.restype = ctypes.c_int
        L.moe_workspace_size.argtypes = [C, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_max_rows.restype = ctypes.c_int64
        L.moe_max_rows.argtypes = [C]
        L.moe_capacity.restype = ctypes.c_int64
        L.moe_capacity.argtypes = [C]
        L.moe_route_slots.restype = ctypes.c_int32
        L.moe_route_slots.argtypes = [C]
        L.moe_last_hip_error.restype = ctypes.c_int32
        L.moe_last_hip_error.argtypes = []
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [ctypes.c_int]
        W, S = ctypes.POINTER(MoeWeights), ctypes.POINTER(MoeStats)
        sz = ctypes.c_size_t
        L.moe_route.restype = ctypes.c_int
        L.moe_route.argtypes = [C, P, W, P, P, P, S, P, sz, P]
        L.moe_dispatch.restype = ctypes.c_int
        L.moe_dispatch.argtypes = [C, P, P, P, P, P, P, S, P, sz, P]
        L.moe_dispatch_noalloc.restype = ctypes.c_int
        L.moe_dispatch_noalloc.argtypes = [C, P, P, P, P, P, P, S, P]
        L.moe_expert_ffn.restype = ctypes.c_int
        L.moe_expert_ffn.argtypes = [C, P, P, W, P, P, sz, P]
        L.moe_expert_up.restype = ctypes.c_int
        L.moe_expert_up.argtypes = [C, P, P, W, P, P, sz, P]
        L.moe_expert_down.restype = ctypes.c_int
        L.moe_expert_down.argtypes = [C, P, P, W, P, P, sz, P]
        L.moe_shared_expert.restype = ctypes.c_int
        L.moe_shared_expert.argtypes = [C, P, W, P, P, sz, P]
        L.moe_combine.restype = ctypes.c_int
        L.moe_combine.argtypes = [C, P, P, P, P, P, P, P]
        L.moe_layer_forward.restype = ctypes.c_int
        L.moe_layer_forward.argtypes = [C, W, P, P, S, P, sz, P]
        L.moe_update_bias.restype = ctypes.c_int
        L.moe_update_bias.argtypes = [C, P, ctypes.c_float, P, P]
        L.moe_expert_up_train.restype = ctypes.c_int
        L.moe_expert_up_train.argtypes = [C, P, P, W, P, P, P, sz, P]
        L.moe_backward_workspace_size.restype = ctypes.c_int
        L.moe_backward_workspace_size.argtypes = [C, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_layer_backward.restype = ctypes.c_int
        L.moe_layer_backward.argtypes = [C, W, P, P, ctypes.POINTER(MoeSaved), ctypes.POINTER(MoeGrads), P, sz, P]
        _lib = L
    return _lib


# ---------------------------------------------------------------- marshalling

def config(*, T: int, d_model: int, d_ff: int, n_experts: int, top_k: int, act_dtype: str = "bf16",
           act: str = "swiglu", gate: str = "softmax_topk", capacity_factor: float = 0.0,
           residual: bool = False, n_shared: int = 0, d_ff_shared: int = 0, noise_input: bool = False,
           seed: int = 0, noise_offset: int = 0, seq_len: int = 0, n_groups: int = 0,
           group_top_k: int = 0, reroute: bool = False) -> MoeConfig:
    c = MoeConfig()
    c.T, c.d_model, c.d_ff, c.n_experts, c.top_k = T, d_model, d_ff, n_experts, top_k
    c.n_shared, c.d_ff_shared = n_shared, d_ff_shared
    c.act_dtype = MOE_BF16 if act_dtype == "bf16" else MOE_F32
    c.act = ACTS[act]
    c.gate = GATES[gate]
    c.capacity_factor = capacity_factor
    c.flags = ((MOE_F_ADD_RESIDUAL if residual else 0) | (MOE_F_NOISE_INPUT if noise_input else 0) |
               (MOE_F_REROUTE if reroute else 0))
    c.seed, c.noise_offset = seed, noise_offset
    c.seq_len = seq_len
    c.n_groups, c.group_top_k = n_groups, group_top_k
    return c


def _dt(c: MoeConfig) -> torch.dtype:
    return torch.bfloat16 if c.act_dtype == MOE_BF16 else torch.float32


def _ptr(t: Optional[torch.Tensor], dtype: Optional[torch.dtype] = None, shape=None, name: str = "tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn: str, rc: int):
    if rc != 0:
        raise MoeError(fn, rc, lib().moe_last_hip_error())


def weights_from(c: MoeConfig, t: Dict[str, torch.Tensor]) -> MoeWeights:
    """MoeWeights from a dict of device tensors named as in include/moe.h
    (ReLU experts may use ``w1``/``w2`` for ``w_gate``/``w_down``)."""
    dt, E, d, F = _dt(c), c.n_experts, c.d_model, c.d_ff
    w = MoeWeights()
    w.w_router = _ptr(t.get("w_router"), torch.float32, (E, d), "w_router")
    w.logit_bias = _ptr(t.get("logit_bias"), torch.float32, (E,), "logit_bias")
    w.sel_bias = _ptr(t.get("sel_bias"), torch.float32, (E,), "sel_bias")
    w.w_noise = _ptr(t.get("w_noise"), torch.float32, (E, d), "w_noise")
    w.noise = _ptr(t.get("noise"), torch.float32, (c.T, E), "noise")
    w.w_gate = _ptr(t.get("w_gate", t.get("w1")), dt, (E, F, d), "w_gate")
    w.w_up = _ptr(t.get("w_up"), dt, (E, F, d), "w_up")
    w.w_down = _ptr(t.get("w_down", t.get("w2")), dt, (E, d, F), "w_down")
    w.token_ids = _ptr(t.get("token_ids"), torch.int32, (c.T,), "token_ids")
    w.w_group_router = _ptr(t.get("w_group_router"), torch.float32, (c.n_groups, d), "w_group_router")
    if c.n_shared:
        Fs = c.d_ff_shared
        w.ws_gate = _ptr(t["ws_gate"].reshape(Fs, d) if "ws_gate" in t else None, dt, (Fs, d), "ws_gate")
        w.ws_up = _ptr(t["ws_up"].reshape(Fs, d) if "ws_up" in t else None, dt, (Fs, d), "ws_up")
        w.ws_down = _ptr(t["ws_down"].reshape(d, Fs) if "ws_down" in t else None, dt, (d, Fs), "ws_down")
    return w


def alloc_stats(c: MoeConfig, device="cuda", balance: bool = False) -> Dict[str, torch.Tensor]:
    """Device buffers for moe_stats; balance=True adds the balance and
    stability statistics (z_loss, importance, load, their CV^2, seq_aux),
    which makes moe_route run their kernels."""
    E = c.n_experts
    i32, f32 = dict(dtype=torch.int32, device=device), dict(dtype=torch.float32, device=device)
    st = dict(counts=torch.zeros(E, **i32), kept=torch.zeros(E, **i32), f=torch.zeros(E, **f32),
              P=torch.zeros(E, **f32), n_dropped=torch.zeros(1, **i32), imbalance=torch.zeros(1, **f32),
              aux=torch.zeros(1, **f32), device_status=torch.zeros(1, **i32))
    if balance:
        st.update(z_loss=torch.zeros(1, **f32), importance=torch.zeros(E, **f32),
                  importance_cv2=torch.zeros(1, **f32), load=torch.full((E,), float("nan"), **f32),
                  load_cv2=torch.full((1,), float("nan"), **f32), seq_aux=torch.zeros(1, **f32))
    return st


def _stats_struct(st: Optional[Dict[str, torch.Tensor]]) -> Optional[MoeStats]:
    if st is None:
        return None
    s = MoeStats()
    for name, _ in MoeStats._fields_:
        t = st.get(name)
        setattr(s, name, None if t is None else _ptr(t, name=name))
    return s


def _sref(s: Optional[MoeStats]):
    return None if s is None else ctypes.byref(s)


def validate_config(c: MoeConfig) -> int:
    return lib().moe_validate_config(ctypes.byref(c))


def workspace_size(c: MoeConfig) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_workspace_size", lib().moe_workspace_size(ctypes.byref(c), ctypes.byref(n)))
    return int(n.value)


def max_rows(c: MoeConfig) -> int:
    return int(lib().moe_max_rows(ctypes.byref(c)))


def capacity(c: MoeConfig) -> int:
    return int(lib().moe_capacity(ctypes.byref(c)))


def route_slots(c: MoeConfig) -> int:
    """Selection slots per token: top_k, or n_experts under expert choice."""
    return int(lib().moe_route_slots(ctypes.byref(c)))


def workspace(c: MoeConfig, device="cuda") -> torch.Tensor:
    return torch.empty(max(workspace_size(c), 1), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- stages

def moe_route(c: MoeConfig, x, w: MoeWeights, topk_idx, topk_gate, scores=None, stats=None, ws=None, stream=None):
    T, E, k, d = c.T, c.n_experts, route_slots(c), c.d_model
    st = _stats_struct(stats)
    rc = lib().moe_route(ctypes.byref(c), _ptr(x, _dt(c), (T, d), "x"), ctypes.byref(w),
                         _ptr(topk_idx, torch.int32, (T, k), "topk_idx"),
                         _ptr(topk_gate, torch.float32, (T, k), "topk_gate"),
                         _ptr(scores, torch.float32, (T, E), "scores"), _sref(st),
                         _ptr(ws, torch.uint8, name="ws"), ws.numel() if ws is not None else 0, _stream(stream))
    _check("moe_route", rc)


def moe_dispatch(c: MoeConfig, x, topk_idx, x_perm, expert_offsets, perm_src, slot_pos, stats=None, ws=None,
                 stream=None):
    T, E, k, d = c.T, c.n_experts, route_slots(c), c.d_model
    R = max_rows(c)
    st = _stats_struct(stats)
    rc = lib().moe_dispatch(ctypes.byref(c), _ptr(x, _dt(c), (T, d), "x"),
                            _ptr(topk_idx, torch.int32, (T, k), "topk_idx"),
                            _ptr(x_perm, _dt(c), (R, d), "x_perm"),
                            _ptr(expert_offsets, torch.int32, (E + 1,), "expert_offsets"),
                            _ptr(perm_src, torch.int32, (R,), "perm_src"),
                            _ptr(slot_pos, torch.int32, (T, k), "slot_pos"), _sref(st),
                            _ptr(ws, torch.uint8, name="ws"), ws.numel() if ws is not None else 0, _stream(stream))
    _check("moe_dispatch", rc)


def moe_dispatch_noalloc(c: MoeConfig, x, topk_idx, x_perm, expert_offsets, perm_src, slot_pos, stats=None,
                         stream=None):
    """moe_dispatch with the library's static device scratch instead of a
    workspace (nothing is allocated; calls on one GPU must not overlap)."""
    T, E, k, d = c.T, c.n_experts, route_slots(c), c.d_model
    R = max_rows(c)
    st = _stats_struct(stats)
    rc = lib().moe_dispatch_noalloc(ctypes.byref(c), _ptr(x, _dt(c), (T, d), "x"),
                                    _ptr(topk_idx, torch.int32, (T, k), "topk_idx"),
                                    _ptr(x_perm, _dt(c), (R, d), "x_perm"),
                                    _ptr(expert_offsets, torch.int32, (E + 1,), "expert_offsets"),
                                    _ptr(perm_src, torch.int32, (R,), "perm_src"),
                                    _ptr(slot_pos, torch.int32, (T, k), "slot_pos"), _sref(st), _stream(stream))
    _check("moe_dispatch_noalloc", rc)


def moe_expert_ffn(c: MoeConfig, x_perm, expert_offsets, w: MoeWeights, y_perm, ws=None, stream=None):
    R, d, E = max_rows(c), c.d_model, c.n_experts
    rc = lib().moe_expert_ffn(ctypes.byref(c), _ptr(x_perm, _dt(c), (R, d), "x_perm"),
                              _ptr(expert_offsets, torch.int32, (E + 1,), "expert_offsets"), ctypes.byref(w),
                              _ptr(y_perm, _dt(c), (R, d), "y_perm"),
                              _ptr(ws, torch.uint8, name="ws"), ws.numel() if ws is not None else 0, _stream(stream))
    _check("moe_expert_ffn", rc)


def moe_expert_up(c: MoeConfig, x_perm, expert_offsets, w: MoeWeights, h, ws=None, stream=None):
    R, d, E, F = max_rows(c), c.d_model, c.n_experts, c.d_ff
    rc = lib().moe_expert_up(ctypes.byref(c), _ptr(x_perm, _dt(c), (R, d), "x_perm"),
                             _ptr(expert_offsets, torch.int32, (E + 1,), "expert_offsets"), ctypes.byref(w),
                             _ptr(h, _dt(c), (R, F), "h"),
                             _ptr(ws, torch.uint8, name="ws"), ws.numel() if ws is not None else 0, _stream(stream))
    _check("moe_expert_up", rc)


def moe_expert_up_train(c: MoeConfig, x_perm, expert_offsets, w: MoeWeights, h, pre_act, ws=None, stream=None):
    """moe_expert_up that also stores the pre-activations [a | u] (SwiGLU) or a
    (ReLU) for the backward."""
    R, d, E, F = max_rows(c), c.d_model, c.n_experts, c.d_ff
    ig = 2 if c.act == ACTS["swiglu"] else 1
    rc = lib().moe_expert_up_train(ctypes.byref(c), _ptr(x_perm, _dt(c), (R, d), "x_perm"),
                                   _ptr(expert_offsets, torch.int32, (E + 1,), "expert_offsets"), ctypes.byref(w),
                                   _ptr(h, _dt(c), (R, F), "h"), _ptr(pre_act, _dt(c), (R, ig * F), "pre_act"),
                                   _ptr(ws, torch.uint8, name="ws"), ws.numel() if ws is not None else 0,
                                   _stream(stream))
    _check("moe_expert_up_train", rc)


def moe_expert_down(c: MoeConfig, h, expert_offsets, w: MoeWeights, y_perm, ws=None, stream=None):
    R, d, E, F = max_rows(c), c.d_model, c.n_experts, c.d_ff
    rc = lib().moe_expert_down(ctypes.byref(c), _ptr(h, _dt(c), (R, F), "h"),
                               _ptr(expert_offsets, torch.int32, (E + 1,), "expert_offsets"), ctypes.byref(w),
                               _ptr(y_perm, _dt(c), (R, d), "y_perm"),
                               _ptr(ws, torch.uint8, name="ws"), ws.numel() if ws is not None else 0,
                               _stream(stream))
    _check("moe_expert_down", rc)


def moe_shared_expert(c: MoeConfig, x, w: MoeWeights, shared_out, ws=None, stream=None):
    T, d = c.T, c.d_model
    rc = lib().moe_shared_expert(ctypes.byref(c), _ptr(x, _dt(c), (T, d), "x"), ctypes.byref(w),
                                 _ptr(shared_out, _dt(c), (T, d), "shared_out"),
                                 _ptr(ws, torch.uint8, name="ws"), ws.numel() if ws is not None else 0,
                                 _stream(stream))
    _check("moe_shared_expert", rc)


def moe_combine(c: MoeConfig, y_perm, slot_pos, topk_gate, residual, shared_out, out, stream=None):
    T, d, k = c.T, c.d_model, route_slots(c)
    R = max_rows(c)
    rc = lib().moe_combine(ctypes.byref(c), _ptr(y_perm, _dt(c), (R, d), "y_perm"),
                           _ptr(slot_pos, torch.int32, (T, k), "slot_pos"),
                           _ptr(topk_gate, torch.float32, (T, k), "topk_gate"),
                           _ptr(residual, _dt(c), (T, d), "residual"),
                           _ptr(shared_out, _dt(c), (T, d), "shared_out"),
                           _ptr(out, _dt(c), (T, d), "out"), _stream(stream))
    _check("moe_combine", rc)


def moe_layer_forward(c: MoeConfig, w: MoeWeights, x, out, stats=None, ws=None, stream=None):
    T, d = c.T, c.d_model
    st = _stats_struct(stats)
    rc = lib().moe_layer_forward(ctypes.byref(c), ctypes.byref(w), _ptr(x, _dt(c), (T, d), "x"),
                                 _ptr(out, _dt(c), (T, d), "out"), _sref(st),
                                 _ptr(ws, torch.uint8, name="ws"), ws.numel() if ws is not None else 0,
                                 _stream(stream))
    _check("moe_layer_forward", rc)


def moe_update_bias(c: MoeConfig, counts, gamma: float, sel_bias, stream=None):
    """sel_bias += gamma * sign(mean(counts) - counts), in place on the device."""
    E = c.n_experts
    rc = lib().moe_update_bias(ctypes.byref(c), _ptr(counts, torch.int32, (E,), "counts"), ctypes.c_float(gamma),
                               _ptr(sel_bias, torch.float32, (E,), "sel_bias"), _stream(stream))
    _check("moe_update_bias", rc)


# ---------------------------------------------------------------- backward

def backward_workspace_size(c: MoeConfig) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_backward_workspace_size", lib().moe_backward_workspace_size(ctypes.byref(c), ctypes.byref(n)))
    return int(n.value)


def backward_workspace(c: MoeConfig, device="cuda") -> torch.Tensor:
    return torch.empty(max(backward_workspace_size(c), 1), dtype=torch.uint8, device=device)


def moe_layer_backward(c: MoeConfig, w: MoeWeights, x, dy, saved: Dict[str, torch.Tensor],
                       grads: Dict[str, torch.Tensor], ws=None, stream=None):
    """Backward of the layer.  ``saved`` holds the forward's stage outputs
    (topk_idx, topk_gate, expert_offsets, perm_src, slot_pos, x_perm, y_perm);
    ``grads`` the output tensors to write (dx required; dw_router,
    dlogit_bias, dw_gate / dw_up / dw_down, dws_gate / dws_up / dws_down
    optional)."""
    T, d, E, F, dt = c.T, c.d_model, c.n_experts, c.d_ff, _dt(c)
    k, R = route_slots(c), max_rows(c)
    sv = MoeSaved()
    sv.topk_idx = _ptr(saved.get("topk_idx"), torch.int32, (T, k), "topk_idx")
    sv.topk_gate = _ptr(saved.get("topk_gate"), torch.float32, (T, k), "topk_gate")
    sv.expert_offsets = _ptr(saved.get("expert_offsets"), torch.int32, (E + 1,), "expert_offsets")
    sv.perm_src = _ptr(saved.get("perm_src"), torch.int32, (R,), "perm_src")
    sv.slot_pos = _ptr(saved.get("slot_pos"), torch.int32, (T, k), "slot_pos")
    sv.x_perm = _ptr(saved.get("x_perm"), dt, (R, d), "x_perm")
    sv.y_perm = _ptr(saved.get("y_perm"), dt, (R, d), "y_perm")
    ig = 2 if c.act == ACTS["swiglu"] else 1
    sv.pre_act = _ptr(saved.get("pre_act"), dt, (R, ig * F), "pre_act")
    g = MoeGrads()
    g.dx = _ptr(grads.get("dx"), dt, (T, d), "dx")
    g.dw_router = _ptr(grads.get("dw_router"), torch.float32, (E, d), "dw_router")
    g.dlogit_bias = _ptr(grads.get("dlogit_bias"), torch.float32, (E,), "dlogit_bias")
    g.dw_gate = _ptr(grads.get("dw_gate"), dt, (E, F, d), "dw_gate")
    g.dw_up = _ptr(grads.get("dw_up"), dt, (E, F, d), "dw_up")
    g.dw_down = _ptr(grads.get("dw_down"), dt, (E, d, F), "dw_down")
    Fs = c.d_ff_shared
    g.dws_gate = _ptr(grads.get("dws_gate"), dt, (Fs, d), "dws_gate")
    g.dws_up = _ptr(grads.get("dws_up"), dt, (Fs, d), "dws_up")
    g.dws_down = _ptr(grads.get("dws_down"), dt, (d, Fs), "dws_down")
    rc = lib().moe_layer_backward(ctypes.byref(c), ctypes.byref(w), _ptr(x, dt, (T, d), "x"),
                                  _ptr(dy, dt, (T, d), "dy"), ctypes.byref(sv), ctypes.byref(g),
                                  _ptr(ws, torch.uint8, name="ws"), ws.numel() if ws is not None else 0,
                                  _stream(stream))
    _check("moe_layer_backward", rc)
