"""Pins of the SwiGLU oracle against closed forms, identities and finite differences."""

import math

import numpy as np

from oracle.swiglu import silu, swiglu_bwd_ref, swiglu_ref


def test_silu_closed_forms_and_limits():
    assert silu(0.0) == 0.0
    # sigmoid(ln 3) = 1 / (1 + 1/3) = 3/4
    assert abs(silu(math.log(3.0)) - 0.75 * math.log(3.0)) < 1e-15
    # sigmoid(-ln 3) = 1/4
    assert abs(silu(-math.log(3.0)) + 0.25 * math.log(3.0)) < 1e-15
    assert silu(60.0) == 60.0 * (1.0 / (1.0 + math.exp(-60.0)))
    assert abs(silu(60.0) - 60.0) < 1e-20
    assert 0.0 > silu(-60.0) > -1e-24
    assert silu(-1000.0) == 0.0  # exp overflows to inf: -1000 / inf


def test_silu_odd_part_identity():
    # silu(v) - silu(-v) = v (sigmoid(v) + sigmoid(-v) = 1)
    v = np.random.default_rng(1).normal(0.0, 4.0, 10000)
    assert np.max(np.abs(silu(v) - silu(-v) - v) / np.maximum(np.abs(v), 1e-300)) < 1e-14


def test_swiglu_at_closed_form_points():
    g = np.array([[0.0, math.log(3.0), -math.log(3.0), 50.0]])
    u = np.array([[7.0, 2.0, 4.0, -0.5]])
    h = swiglu_ref(np.concatenate([g, u], axis=1), 4)
    want = np.array([[0.0, 1.5 * math.log(3.0), -math.log(3.0), -25.0]], np.float32)
    assert np.array_equal(h, want)


def test_backward_is_the_derivative_of_the_forward():
    # central differences of h = silu(g) u in float64, against dL/dg and dL/du with dh
    rng = np.random.default_rng(2)
    M, I = 64, 32
    g = rng.normal(0.0, 3.0, (M, I))
    u = rng.normal(0.0, 1.0, (M, I))
    dh = rng.normal(0.0, 1.0, (M, I))
    eps = 1e-6
    num_dg = dh * (silu(g + eps) * u - silu(g - eps) * u) / (2 * eps)
    num_du = dh * (silu(g) * (u + eps) - silu(g) * (u - eps)) / (2 * eps)
    d = swiglu_bwd_ref(dh, np.concatenate([g, u], axis=1), I).astype(np.float64)
    scale = np.max(np.abs(num_dg))
    assert np.max(np.abs(d[:, :I] - num_dg)) < 1e-6 * scale
    assert np.max(np.abs(d[:, I:] - num_du)) < 1e-6 * np.max(np.abs(num_du))


def test_backward_at_a_closed_form_point():
    # g = ln 3: sigmoid = 3/4, d silu/dg = 3/4 (1 + ln3 / 4)
    l3 = math.log(3.0)
    d = swiglu_bwd_ref(np.array([[2.0]]), np.array([[l3, 5.0]]), 1)
    assert abs(d[0, 0] - np.float32(2.0 * 5.0 * 0.75 * (1 + l3 / 4))) <= 1e-6 * abs(d[0, 0])
    assert abs(d[0, 1] - np.float32(2.0 * 0.75 * l3)) <= 1e-6 * abs(d[0, 1])
