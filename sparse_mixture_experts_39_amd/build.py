"""Build libmoe.so (the gfx950 kernels and the C ABI of include/moe.h) in-tree.

Every HIP source is compiled with hipcc for gfx950 only, with packed-fp32
instructions disabled; route.hip and backward.hip are compiled without fp
contraction because the router's integer decisions (and the backward's
recomputed logits) rest on a fixed sequence of fp32 operations.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(os.path.dirname(HERE), "_build")
LIB_PATH = os.path.join(HERE, "libmoe.so")
# measurement aid (peak probes, cache flush): its own library, not the ABI
PEAK_SOURCE = "peak.hip"
PEAK_LIB_PATH = os.path.join(HERE, "libmoe_peak.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = {
    "moe_api.cpp": [],
    "route.hip": ["-ffp-contract=off"],
    "dispatch.hip": [],
    "combine.hip": [],
    "ffn.hip": [],
    "backward.hip": ["-ffp-contract=off"],
}
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, src + ".o")
    cmd = [HIPCC] + COMMON + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass of hipcc does not know the packed-fp32 feature and says so: harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _link(objs, path):
    tmp = path + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950"] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, path)


def build(jobs: int = 8) -> str:
    """Compile every source, link libmoe.so and libmoe_peak.so; always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    todo = list(SOURCES.items()) + [(PEAK_SOURCE, [])]
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda kv: _compile(*kv), todo))
    _link(objs[:-1], LIB_PATH)
    _link(objs[-1:], PEAK_LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
