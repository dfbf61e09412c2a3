"""Full-size parity: the Mixtral-8x7B-shaped and the DeepSeek-V3-shaped layers
through the C ABI against the CPU oracle on every token.

Inputs are drawn on the GPU with the workloads' seeds and copied to the host;
the oracle then runs the whole layer (about a minute of fp64 work on 16
cores for each).  Routing and dispatch must match bit for bit over all
tokens (top-k indices, selection scores, counts, offsets, permutation, drop
masks, x_perm bytes); every row of y_perm, the shared expert and every
output token within the bf16 tolerance of tests/gpu_helpers.py; the
whole-layer call's output equals the stage calls' byte for byte.  The sampled
full-size tests in test_gpu_parity.py stay as fast pre-checks.
"""
from __future__ import annotations

import time

import pytest
import torch

import oracle
import workloads
import tests.gpu_helpers as H
from tests.test_gpu_parity import check_all

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["mixtral", "dsv3"])
def test_full_size_layer_every_row(name):
    cfg = workloads.get(name)
    H.log(f"[full-size] {name}: drawing inputs on the GPU")
    dinp = workloads.make_inputs(cfg, device="cuda", with_noise=False)
    g = H.run_stages(cfg, dinp, noise_input=False)
    # the whole-layer call (its up projection gathers the rows of x) writes
    # the same bytes as the stage calls checked against the oracle below
    out_layer, _ = H.run_layer(cfg, dinp, noise_input=False, stats=False)
    assert torch.equal(out_layer.view(torch.int16), g["out"].view(torch.int16)), "layer differs from stages"
    H.log(f"[full-size] {name}: GPU layer done; copying inputs to the host")
    host = {k: v.cpu() for k, v in dinp.items()}
    del dinp
    torch.cuda.empty_cache()
    t0 = time.perf_counter()
    o = oracle.forward(cfg, host, noise="philox")
    H.log(f"[full-size] {name}: oracle layer in {time.perf_counter() - t0:.0f} s; comparing every row")
    err = check_all(cfg, g, o)
    H.log(f"[full-size] {name}: routing and dispatch bit-exact, out rel err {err:.2e}")
