"""Measured ceilings of one MI355X, quoted beside the published peaks.

Binding of libmoe_peak.so (csrc/peak.hip), a measurement aid that is not part
of the layer's ABI: a register-only bf16 MFMA rate probe for the two MFMA
shapes, a device copy probe, and a cache flush (a read pass over a buffer
larger than the 256 MB last-level cache) for stage timings that must not find
their inputs in the cache.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict

import torch

from .build import PEAK_LIB_PATH

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(PEAK_LIB_PATH):
            raise RuntimeError(f"{PEAK_LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(PEAK_LIB_PATH)
        P = ctypes.c_void_p
        L.moe_peak_mfma.restype = ctypes.c_int
        L.moe_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P]
        L.moe_peak_copy.restype = ctypes.c_int
        L.moe_peak_copy.argtypes = [P, P, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, P]
        L.moe_cache_flush.restype = ctypes.c_int
        L.moe_cache_flush.argtypes = [P, ctypes.c_int64, ctypes.c_uint32, P, P]
        _lib = L
    return _lib


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _timed(fn, reps: int) -> float:
    """Best of `reps` event-timed calls, in seconds."""
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e-3)
    return best


def mfma_tflops(shape: int, blocks_per_cu: int = 1, iters: int = 10000, reps: int = 3) -> float:
    """bf16 MFMA rate (TFLOP/s) of waves each accumulating a 128 x 128 tile
    from register operands with MFMAs of one shape (16: 16x16x32, 32:
    32x32x16), 4 waves per block, blocks_per_cu blocks per compute unit (the
    256 accumulator registers per wave allow one block per CU; a second
    block only queues behind the first)."""
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = n_cu * blocks_per_cu
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")

    def run():
        rc = lib().moe_peak_mfma(shape, iters, blocks, ctypes.c_void_p(out.data_ptr()), _stream())
        if rc != 0:
            raise RuntimeError(f"moe_peak_mfma failed ({rc})")

    run()
    torch.cuda.synchronize()
    t = _timed(run, reps)
    flops = blocks * 4 * iters * (1048576.0 if shape == 16 else 524288.0)
    return flops / t / 1e12


def copy_gbs(mib: int = 2048, reps: int = 5, blocks_per_cu: int = 8, unroll: int = 8, nt: bool = False) -> float:
    """Device copy rate (GB/s counting bytes read + bytes written) over two
    buffers of mib MiB each (far beyond the 256 MB last-level cache)."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    flush(src)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count

    def run():
        rc = lib().moe_peak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), n,
                                 n_cu * blocks_per_cu, unroll, int(nt), _stream())
        if rc != 0:
            raise RuntimeError(f"moe_peak_copy failed ({rc})")

    run()
    torch.cuda.synchronize()
    t = _timed(run, reps)
    return 2.0 * n / t / 1e9


def best_copy_gbs() -> Dict[str, float]:
    """The copy probe over a small sweep of launch shapes; the best is the
    measured copy ceiling."""
    res = {}
    for bpc in (4, 8, 16):
        for unroll in (4, 8):
            for nt in (False, True):
                res[f"copy_b{bpc}_u{unroll}{'_nt' if nt else ''}"] = copy_gbs(blocks_per_cu=bpc, unroll=unroll, nt=nt,
                                                                             reps=3)
    return res


_sink = None


def flush(buf: torch.Tensor, salt: int = 0):
    """A read pass over the whole (contiguous, device) buffer, which should be
    larger than the last-level cache (256 MB): afterwards the caches hold
    clean lines of `buf` only."""
    global _sink
    if _sink is None or _sink.device != buf.device:
        _sink = torch.empty(4096 * 256, dtype=torch.int32, device=buf.device)
    nbytes = buf.numel() * buf.element_size() // 16 * 16
    never = (0x9E3779B9 * (salt + 1)) & 0xFFFFFFFF
    rc = lib().moe_cache_flush(ctypes.c_void_p(buf.data_ptr()), nbytes, never, ctypes.c_void_p(_sink.data_ptr()),
                               _stream())
    if rc != 0:
        raise RuntimeError(f"moe_cache_flush failed ({rc})")


def measure_all() -> Dict[str, float]:
    res = {
        "mfma_bf16_16x16x32_tflops": mfma_tflops(16),
        "mfma_bf16_32x32x16_tflops": mfma_tflops(32),
        **best_copy_gbs(),
    }
    res["copy_gbs"] = max(v for k, v in res.items() if k.startswith("copy_"))
    return res
