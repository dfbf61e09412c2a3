"""Pins of the oracle's canonical fp32 scalar functions and its noise stream.

Each canonical function is checked against the mathematical function it
stands for (numpy's fp64 libm, i.e. the exact value to ~1e-16) within a few
fp32 ulps, plus exact special values.  A wrong series coefficient, a
dropped reduction term or a wrong quadrant rotation fails these bounds.
The Gaussian stream is checked against N(0,1) (mean, variance, KS distance,
lag correlation).  The Philox4x32-10 generator underneath it is pinned to the
generator's published known-answer vectors in tests/test_oracle_hash.py
(fixture tests/golden/philox4x32_10_kat.json, with its citation).
"""
import math

import numpy as np
import pytest

import oracle


def _ulp_err(y32, ref64):
    ref32 = ref64.astype(np.float32)
    sp = np.spacing(np.abs(ref32)).astype(np.float64)
    return np.abs(y32.astype(np.float64) - ref64) / sp


def test_exp_within_2ulp():
    rng = np.random.default_rng(11)
    x = rng.uniform(-87.0, 88.0, 1_000_000).astype(np.float32)
    y = oracle.map_f32("exp", x)
    assert _ulp_err(y, np.exp(x.astype(np.float64))).max() <= 2.0


def test_exp_special_values():
    y = oracle.map_f32("exp", np.array([0.0, -0.0, -100.0, 100.0, np.nan, 1.0], np.float32))
    assert y[0] == 1.0 and y[1] == 1.0
    assert y[2] == 0.0 and np.isinf(y[3]) and np.isnan(y[4])
    assert abs(float(y[5]) - math.e) <= 2 * np.spacing(np.float32(math.e))


def test_log_within_3ulp():
    rng = np.random.default_rng(12)
    x = np.exp(rng.uniform(-87, 88, 1_000_000)).astype(np.float32)
    x = x[(x > 0) & np.isfinite(x)]
    ref = np.log(x.astype(np.float64))
    y = oracle.map_f32("log", x)
    far = np.abs(ref) > 1e-3          # relative ulps are meaningless at the zero of log
    assert _ulp_err(y[far], ref[far]).max() <= 3.0
    assert np.abs(y[~far] - ref[~far]).max() <= 2e-10 + 4 * np.spacing(np.float32(1e-3))


def test_log_special_and_subnormal():
    y = oracle.map_f32("log", np.array([1.0, 0.0, -1.0, 2.0 ** -149, 2.0 ** -130, 2.0], np.float32))
    assert y[0] == 0.0 and np.isneginf(y[1]) and np.isnan(y[2])
    assert abs(y[3] - (-149 * math.log(2))) < 1e-4
    assert abs(y[4] - (-130 * math.log(2))) < 1e-4
    assert abs(y[5] - math.log(2)) <= np.spacing(np.float32(math.log(2)))


def test_softplus_and_sigmoid_relative_error():
    rng = np.random.default_rng(13)
    x = rng.uniform(-40, 40, 1_000_000).astype(np.float32)
    xd = x.astype(np.float64)
    sp = oracle.map_f32("softplus", x)
    ref = np.logaddexp(0.0, xd)
    assert (np.abs(sp - ref) / ref).max() < 6e-7
    sg = oracle.map_f32("sigmoid", x)
    ref = 1.0 / (1.0 + np.exp(-xd))
    ok = ref > 1e-37
    assert (np.abs(sg[ok] - ref[ok]) / ref[ok]).max() < 4e-7
    assert oracle.map_f32("softplus", np.array([0.0], np.float32))[0] == np.float32(math.log(2)) or \
        abs(oracle.map_f32("softplus", np.array([0.0], np.float32))[0] - math.log(2)) < 1.2e-7
    assert oracle.map_f32("sigmoid", np.array([0.0], np.float32))[0] == 0.5


def test_sincos_on_full_turn():
    rng = np.random.default_rng(14)
    th = rng.uniform(0, 2 * math.pi, 1_000_000).astype(np.float32)
    s = oracle.map_f32("sin", th)
    c = oracle.map_f32("cos", th)
    assert np.abs(s - np.sin(th.astype(np.float64))).max() < 2.5e-7
    assert np.abs(c - np.cos(th.astype(np.float64))).max() < 2.5e-7
    q = oracle.map_f32("sin", np.array([0.0, math.pi / 2, math.pi, 3 * math.pi / 2], np.float32))
    assert q[0] == 0.0 and abs(q[1] - 1) < 1e-7 and abs(q[2]) < 1e-7 and abs(q[3] + 1) < 1e-7


def test_gaussian_stream_is_standard_normal():
    n = oracle.normal(1003, 0, 0, 2_000_000).astype(np.float64)
    assert abs(n.mean()) < 5 * (1 / math.sqrt(n.size))
    assert abs(n.var() - 1.0) < 5 * math.sqrt(2.0 / n.size)
    xs = np.sort(n[:200_000])
    cdf = 0.5 * (1 + np.vectorize(math.erf)(xs / math.sqrt(2)))
    ks = np.max(np.abs(cdf - (np.arange(1, xs.size + 1) / xs.size)))
    assert ks < 1.63 / math.sqrt(xs.size)        # 1% critical value
    for lag in (1, 2, 3, 4, 8):                   # words of one Philox block and neighbours
        r = np.corrcoef(n[:-lag], n[lag:])[0, 1]
        assert abs(r) < 5 / math.sqrt(n.size)


def test_gaussian_stream_counter_mapping():
    """Element i depends on (seed, offset, i) only: a window drawn from a
    different start reproduces the same values; other seeds or offsets do not."""
    a = oracle.normal(7, 3, 0, 64)
    b = oracle.normal(7, 3, 16, 48)
    np.testing.assert_array_equal(a[16:], b)
    assert not np.array_equal(a, oracle.normal(8, 3, 0, 64))
    assert not np.array_equal(a, oracle.normal(7, 4, 0, 64))
    assert np.isfinite(a).all()
