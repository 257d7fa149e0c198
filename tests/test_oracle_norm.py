"""Pins of the oracle's gated group RMSNorm by closed forms."""
import math

import numpy as np

from oracle import bf16_to_f64, gated_group_rmsnorm
from workloads import bf16_bits


def _silu(z):
    return z / (1.0 + math.exp(-z))


def test_constant_group():
    G, W = 2, 8
    y = bf16_bits(np.array([[0.5] * W + [3.0] * W], np.float32))
    z = bf16_bits(np.array([[2.0] * (2 * W)], np.float32))
    w = bf16_bits(np.array([1.5] * (2 * W), np.float32))
    eps = 1e-5
    o, _ = gated_group_rmsnorm(y, z, w, G, eps)
    for gi, yv in enumerate([0.5, 3.0]):
        v = yv * _silu(2.0)
        want = 1.5 * v / math.sqrt(v * v + eps)
        assert np.max(np.abs(o[0, gi * W:(gi + 1) * W] - want)) < 1e-14


def test_single_nonzero_per_group_pins_group_size_and_eps():
    G, W = 4, 512
    yv = np.zeros((1, G * W), np.float32)
    yv[0, ::W] = 0.01                      # one non-zero per group
    y = bf16_bits(yv)
    z = bf16_bits(np.full((1, G * W), 30.0, np.float32))
    w = bf16_bits(np.ones(G * W, np.float32))
    eps = 1e-5
    o, _ = gated_group_rmsnorm(y, z, w, G, eps)
    a = bf16_to_f64(y[0, 0]) * _silu(30.0)
    want = a / math.sqrt(a * a / W + eps)
    assert abs(o[0, 0] - want) < 1e-12 and np.count_nonzero(o) == G


def test_gate_is_applied_before_the_mean_square():
    # y constant, gate varies inside the group: o = s_i / rms(s)
    W = 4
    y = bf16_bits(np.ones((1, W), np.float32))
    zs = [0.0, 1.0, -1.0, 2.0]
    z = bf16_bits(np.array([zs], np.float32))
    w = bf16_bits(np.ones(W, np.float32))
    o, _ = gated_group_rmsnorm(y, z, w, 1, 1e-5)
    s = [_silu(float(bf16_to_f64(z[0, i]))) for i in range(W)]
    rms = math.sqrt(sum(v * v for v in s) / W + 1e-5)
    assert np.max(np.abs(o[0] - np.array(s) / rms)) < 1e-14


def test_scale_invariance_with_scaled_eps():
    r = np.random.default_rng(0)
    y = bf16_bits(r.standard_normal((3, 64)).astype(np.float32))
    z = bf16_bits(r.standard_normal((3, 64)).astype(np.float32))
    w = bf16_bits((1 + 0.1 * r.standard_normal(64)).astype(np.float32))
    o1, _ = gated_group_rmsnorm(y, z, w, 4, 1e-5)
    y4 = bf16_bits(bf16_to_f64(y).astype(np.float32) * 4.0)   # exact in bf16
    o2, _ = gated_group_rmsnorm(y4, z, w, 4, 16e-5)
    assert np.max(np.abs(o1 - o2)) < 1e-13
