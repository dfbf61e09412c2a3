#!/usr/bin/env python3
"""Benchmark of the MoE layer forward on one MI355X.

One step = one pass of the whole layer over one batch of synthetic tokens:
route -> dispatch -> grouped GEMM up -> grouped GEMM down (-> shared expert)
-> combine, each stage a call of the C ABI on the current stream, inputs and
weights resident in HBM.  HIP events between the stage calls time every stage
inside the timed region; the whole-step throughput comes from the wall clock
around K steps bracketed by device synchronisation.

Prints one JSON line (see the keys below).  Default workload: the
Mixtral-8x7B-shaped layer (T=4096, d=4096, d_ff=14336, 8 experts, top-2,
SwiGLU, bf16).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0                        # MI355X HBM3E
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
METRIC = "MoE layer tokens/s + grouped-GEMM % MFMA peak, Mixtral-shaped layer, 1 GPU"


def log(msg):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def workload_desc(cfg):
    s = (f"{cfg.name}: T={cfg.T} d_model={cfg.d} d_ff={cfg.F} experts={cfg.E} top_k={cfg.k} "
         f"{cfg.act} {cfg.gate} {cfg.act_dtype}")
    if cfg.capacity_factor > 0:
        s += f" capacity_factor={cfg.capacity_factor}"
    if cfg.n_shared:
        s += f" shared_expert d_ff={cfg.F_shared}"
    return s


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ("ffn.hip", "device_common.h"):
        with open(os.path.join(ROOT, "sparse_mixture_experts_39_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(path, workload, stage):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or
    None when there is none for this workload / stage or the GEMM source has
    changed since the counters were taken.  The summary carries lines
    'key: value' for workload, stage, source_sha256 and hbm_bytes_per_launch."""
    if not path or not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and line.strip().startswith("- "):
            k, v = line.strip()[2:].split(":", 1)
            kv[k.strip().strip("`")] = v.strip().strip("`")
    if kv.get("workload") != workload or kv.get("stage") != stage:
        return None
    if kv.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(cfg, dinp, target_s):
    """The oracle as it stands, on the host cores, on the first Ts tokens of
    the same workload (whole layer, every weight); Ts is sized so the run
    takes about target_s seconds."""
    import oracle
    host = {k: v.cpu() for k, v in dinp.items()}
    cores = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)

    def run(ts):
        sub = dict(host)
        sub["x"] = host["x"][:ts].contiguous()
        if "noise" in sub:
            sub["noise"] = host["noise"][:ts].contiguous()
        c = cfg.replace(T=ts)
        t0 = time.perf_counter()
        oracle.forward(c, sub, noise="philox")
        return time.perf_counter() - t0

    # two probes give the per-token slope and the fixed per-call cost (the
    # oracle converts every weight to fp64 on each call), then one run sized
    # for target_s; the second probe is large enough (128 tokens) that the
    # slope holds at the sized run, where small per-expert row counts no
    # longer hide the per-row cost
    n1, n2 = min(16, cfg.T), min(128, cfg.T)
    t1 = run(n1)
    if cfg.T <= n1 or t1 >= target_s:
        ts, t = n1, t1
    else:
        t2 = run(n2)
        if n2 == cfg.T or t2 >= target_s:
            ts, t = n2, t2
        else:
            slope = max((t2 - t1) / (n2 - n1), 1e-6)
            fixed = max(t1 - n1 * slope, 0.0)
            ts = int(min(cfg.T, max(n2, (target_s - fixed) / slope)))
            t = run(ts) if ts > n2 else t2
    return {"value": ts / t, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {ts} of the {cfg.T} tokens, whole layer (route, dispatch, experts, combine) "
                      f"with all weights, {t:.1f} s of oracle time"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="mixtral")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle time of the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--balance-stats", action="store_true",
                    help="also request the balance statistics (z-loss, importance, load, seq_aux) from the route stage")
    ap.add_argument("--traffic-file", default=os.path.join(ROOT, "profiles", "mixtral_expert_up_hbm_traffic.md"),
                    help="rocprofv3 counter summary giving the dominant kernel's HBM bytes per launch")
    ap.add_argument("--pass", dest="which", choices=("forward", "backward"), default="forward",
                    help="forward (default): the layer forward, stage by stage; backward: moe_layer_backward on the "
                         "saved tensors of one forward (a separate JSON line with its own metric)")
    ap.add_argument("--peaks", action="store_true",
                    help="only measure the achievable ceilings (register-only bf16 MFMA rate for both MFMA shapes, "
                         "device copy rate) and print them as one JSON line")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (counter calibration)")
    args = ap.parse_args()

    if args.peaks:
        from sparse_mixture_experts_39_amd import peaks
        res = peaks.measure_all()
        res["device"] = __import__("torch").cuda.get_device_name(0)
        print(json.dumps(res))
        return

    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 3}))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs the layer on one GPU only; multi-GPU runs are not part of it "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    import sparse_mixture_experts_39_amd as moe

    cfg = workloads.get(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"bench: drawing {workload_desc(cfg)} on {torch.cuda.get_device_name(0)}")
    dinp = workloads.make_inputs(cfg, device=dev, with_noise=False)
    c = moe.config(T=cfg.T, d_model=cfg.d, d_ff=cfg.F, n_experts=cfg.E, top_k=cfg.k, act_dtype=cfg.act_dtype,
                   act=cfg.act, gate=cfg.gate, capacity_factor=cfg.capacity_factor, residual=cfg.residual,
                   n_shared=cfg.n_shared, d_ff_shared=cfg.F_shared, seed=cfg.seed, n_groups=cfg.n_groups,
                   group_top_k=cfg.group_top_k, reroute=cfg.reroute)
    w = moe.weights_from(c, dinp)
    ws = moe.workspace(c)
    st = moe.alloc_stats(c, balance=args.balance_stats)
    T, E, k, d, F = c.T, c.n_experts, moe.route_slots(c), c.d_model, c.d_ff
    R = moe.max_rows(c)
    dt = dinp["x"].dtype
    i32 = dict(dtype=torch.int32, device=dev)
    idx = torch.empty((T, k), **i32)
    gates = torch.empty((T, k), dtype=torch.float32, device=dev)
    x_perm = torch.empty((R, d), dtype=dt, device=dev)
    H = torch.empty((R, F), dtype=dt, device=dev)
    y_perm = torch.empty((R, d), dtype=dt, device=dev)
    offsets = torch.empty((E + 1,), **i32)
    perm_src = torch.empty((R,), **i32)
    slot_pos = torch.empty((T, k), **i32)
    shared = torch.empty((T, d), dtype=dt, device=dev) if cfg.n_shared else None
    out = torch.empty((T, d), dtype=dt, device=dev)
    x = dinp["x"]
    if args.which == "backward":
        return bench_backward(args, cfg, c, dinp, w, ws, st, moe, torch)
    stages = ["route", "dispatch", "expert_up", "expert_down"] + (["shared_expert"] if shared is not None else []) + ["combine"]

    def step(ev):
        ev[0].record()
        moe.moe_route(c, x, w, idx, gates, None, st, ws)
        ev[1].record()
        moe.moe_dispatch(c, x, idx, x_perm, offsets, perm_src, slot_pos, st, ws)
        ev[2].record()
        moe.moe_expert_up(c, x_perm, offsets, w, H, ws)
        ev[3].record()
        moe.moe_expert_down(c, H, offsets, w, y_perm, ws)
        ev[4].record()
        i = 5
        if shared is not None:
            moe.moe_shared_expert(c, x, w, shared, ws)
            ev[i].record()
            i += 1
        moe.moe_combine(c, y_perm, slot_pos, gates, x if cfg.residual else None, shared, out)
        ev[i].record()

    nev = len(stages) + 1
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps + args.warmup)]
    for i in range(args.warmup):
        step(events[i])
    torch.cuda.synchronize()
    log(f"bench: {args.warmup} warmup steps done, timing {args.steps}")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[args.warmup + i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    stage_ms = {s: 0.0 for s in stages}
    for i in range(args.steps):
        ev = events[args.warmup + i]
        for j, s in enumerate(stages):
            stage_ms[s] += ev[j].elapsed_time(ev[j + 1]) / args.steps

    kept = int(st["kept"].sum().item())
    es = 2 if cfg.act_dtype == "bf16" else 4
    gemm_mult = 2 if cfg.act == "swiglu" else 1
    flops_up = 2.0 * kept * d * F * gemm_mult
    flops_down = 2.0 * kept * F * d
    counts = st["kept"].cpu()
    active = int((counts > 0).sum().item())
    w_up_bytes = active * gemm_mult * F * d * es
    w_down_bytes = active * d * F * es
    up_bytes = w_up_bytes + kept * d * es + kept * F * es          # weights + x_perm rows + h rows
    down_bytes = w_down_bytes + kept * F * es + kept * d * es
    if shared is not None:
        fs = cfg.F_shared
        flops_sh = 2.0 * T * d * fs * 3
        sh_bytes = 3 * d * fs * es + 2 * T * d * es + 2 * T * fs * es
    peak_f = PEAK_MFMA_TFLOPS[cfg.act_dtype]

    def roof(name, flops, nbytes):
        t = stage_ms[name] * 1e-3
        mfma_t, hbm_t = flops / (peak_f * 1e12), nbytes / (PEAK_HBM_GBS * 1e9)
        if mfma_t >= hbm_t:
            a = flops / t / 1e12
            return {"bound": "mfma", "achieved": a, "peak": peak_f, "unit": "TFLOP/s", "frac": a / peak_f}
        a = nbytes / t / 1e9
        return {"bound": "hbm", "achieved": a, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": a / PEAK_HBM_GBS}

    r_up = roof("expert_up", flops_up, up_bytes)
    r_down = roof("expert_down", flops_down, down_bytes)
    dominant = "expert_up" if stage_ms["expert_up"] >= stage_ms["expert_down"] else "expert_down"
    roofline = dict(r_up if dominant == "expert_up" else r_down)
    roofline["kernel"] = "k_grouped_gemm (" + ("SwiGLU up" if dominant == "expert_up" and cfg.act == "swiglu"
                                              else "ReLU up" if dominant == "expert_up" else "down") + ")"
    roofline["per_launch"] = {"flops": flops_up if dominant == "expert_up" else flops_down,
                              "bytes": up_bytes if dominant == "expert_up" else down_bytes,
                              "avg_ms": stage_ms[dominant]}
    roofline["traffic"] = measured_traffic(args.traffic_file, cfg.name, dominant)

    gemm_ms = stage_ms["expert_up"] + stage_ms["expert_down"]
    disp_bytes = T * d * es + kept * d * es                            # read x once, write k copies
    comb_bytes = kept * d * es + T * d * es + (T * d * es if cfg.residual else 0) + (T * d * es if shared is not None else 0)
    value = T * args.steps / wall
    res = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.act_dtype,
        "data": "synthetic (seeded N(0,1) activations, N(0,1/fan_in) weights)",
        "config": {"workload": workload_desc(cfg), "T": T, "d_model": d, "d_ff": F, "n_experts": E, "top_k": c.top_k,
                   "parallelism": "single GPU, all experts resident"},
        "grouped_gemm_pct_mfma_peak": 100.0 * (flops_up + flops_down) / (gemm_ms * 1e-3) / (peak_f * 1e12),
        "dispatch_pct_hbm_peak": 100.0 * disp_bytes / (stage_ms["dispatch"] * 1e-3) / (PEAK_HBM_GBS * 1e9),
        "combine_pct_hbm_peak": 100.0 * comb_bytes / (stage_ms["combine"] * 1e-3) / (PEAK_HBM_GBS * 1e9),
        "stages_ms": stage_ms,
        "expert_up_roofline": r_up,
        "expert_down_roofline": r_down,
        "roofline": roofline,
        "rows_kept": kept,
        "gemm_source_sha256": kernel_source_hash(),
        "experts_with_rows": active,
    }
    if shared is not None:
        res["shared_expert_roofline"] = roof("shared_expert", flops_sh, sh_bytes)
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(cfg, dinp, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res))


BACKWARD_METRIC = "MoE layer backward tokens/s (all gradients), Mixtral-shaped layer, 1 GPU"


def bench_backward(args, cfg, c, dinp, w, ws, st, moe, torch):
    """Time moe_layer_backward: one training forward (untimed; its up
    projection keeps the pre-activations) makes the saved tensors, then W
    warmup and K timed backward calls, each computing dx, the router
    gradients and every expert weight gradient."""
    import workloads
    T, E, k, d, F = c.T, c.n_experts, moe.route_slots(c), c.d_model, c.d_ff
    R = moe.max_rows(c)
    dev = dinp["x"].device
    dt = dinp["x"].dtype
    i32 = dict(dtype=torch.int32, device=dev)
    sv = dict(topk_idx=torch.empty((T, k), **i32), topk_gate=torch.empty((T, k), dtype=torch.float32, device=dev),
              expert_offsets=torch.empty((E + 1,), **i32), perm_src=torch.empty((R,), **i32),
              slot_pos=torch.empty((T, k), **i32), x_perm=torch.empty((R, d), dtype=dt, device=dev),
              y_perm=torch.empty((R, d), dtype=dt, device=dev))
    x = dinp["x"]
    moe.moe_route(c, x, w, sv["topk_idx"], sv["topk_gate"], None, st, ws)
    moe.moe_dispatch(c, x, sv["topk_idx"], sv["x_perm"], sv["expert_offsets"], sv["perm_src"], sv["slot_pos"], st,
                     ws)
    H = torch.empty((R, F), dtype=dt, device=dev)
    sv["pre_act"] = torch.empty((R, (2 if cfg.act == "swiglu" else 1) * F), dtype=dt, device=dev)
    moe.moe_expert_up_train(c, sv["x_perm"], sv["expert_offsets"], w, H, sv["pre_act"], ws)
    moe.moe_expert_down(c, H, sv["expert_offsets"], w, sv["y_perm"], ws)
    del H
    dy = workloads.make_output_grad(cfg, device=dev)
    g = dict(dx=torch.empty((T, d), dtype=dt, device=dev),
             dw_router=torch.empty((E, d), dtype=torch.float32, device=dev),
             dlogit_bias=torch.empty((E,), dtype=torch.float32, device=dev),
             dw_gate=torch.empty((E, F, d), dtype=dt, device=dev),
             dw_down=torch.empty((E, d, F), dtype=dt, device=dev))
    if cfg.act == "swiglu":
        g["dw_up"] = torch.empty((E, F, d), dtype=dt, device=dev)
    if cfg.n_shared:
        fs = cfg.F_shared
        g.update(dws_gate=torch.empty((fs, d), dtype=dt, device=dev), dws_up=torch.empty((fs, d), dtype=dt, device=dev),
                 dws_down=torch.empty((d, fs), dtype=dt, device=dev))
    bws = moe.backward_workspace(c)
    for _ in range(args.warmup):
        moe.moe_layer_backward(c, w, x, dy, sv, g, bws)
    torch.cuda.synchronize()
    log(f"bench: {args.warmup} warmup backward calls done, timing {args.steps}")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        moe.moe_layer_backward(c, w, x, dy, sv, g, bws)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    kept = int(sv["expert_offsets"][E].item())
    mult = 2 if cfg.act == "swiglu" else 1
    # matrix products of the backward: dh (1), dx (mult), dW2 (1), dW1 / dW3
    # (mult) -- twice the forward's; the routed a / u come saved from the
    # forward, the shared expert's are recomputed
    useful = 2.0 * kept * d * F * (2 + 2 * mult)
    recompute = 0.0
    if cfg.n_shared:
        useful += 2.0 * T * d * cfg.F_shared * 6
        recompute += 2.0 * T * d * cfg.F_shared * 2
    peak_f = PEAK_MFMA_TFLOPS[cfg.act_dtype]
    achieved = (useful + recompute) / (ms * 1e-3) / 1e12
    res = {
        "metric": BACKWARD_METRIC,
        "value": T * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.act_dtype,
        "data": "synthetic (seeded N(0,1) activations and output gradient, N(0,1/fan_in) weights)",
        "config": {"workload": workload_desc(cfg) + " backward", "T": T, "d_model": d, "d_ff": F, "n_experts": E,
                   "top_k": c.top_k, "parallelism": "single GPU, all experts resident"},
        "event_ms_per_call": ms,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak_f, "unit": "TFLOP/s",
                     "frac": achieved / peak_f, "traffic": None,
                     "kernel": "whole backward call (all matrix products; pre-activations saved by the forward)",
                     "per_launch": {"flops": useful + recompute, "useful_flops": useful, "avg_ms": ms}},
        "rows_kept": kept,
        "cpu_baseline": None,
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
