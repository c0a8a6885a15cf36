"""Pins of the oracle's Adam step (textbook Adam with bias correction; the per-splat layout of 59 elements and the
28 B per element accounting come from the rasterize forward + adam kernel audit page, section 2 "(f)")."""
import numpy as np
import pytest

from differentiable_gaussian_splatting_amd import scenes
from golden.load import load

B1, B2, EPS, LR = 0.9, 0.999, 1e-15, 1.6e-4


def bc(t):
    return scenes.adam_bias_corrections(B1, B2, t)


def test_first_step_from_zero_state_moves_by_lr_sign(orc):
    """At t = 1 from m = v = 0: m_hat = g, v_hat = g^2, so p' = p - lr g / (|g| + eps) ~ p - lr sign(g)."""
    rng = np.random.default_rng(0)
    g = rng.normal(0, 1e-3, 4096).astype(np.float32)
    p = rng.normal(0, 1, 4096).astype(np.float32)
    z = np.zeros_like(p)
    p1, m1, v1 = orc.adam_step(p, g, z, z, LR, B1, B2, EPS, *bc(1))
    want = p.astype(np.float64) - LR * g / (np.abs(g) + EPS)
    assert np.all(np.abs(p1 - want) <= 2 * np.spacing(np.abs(p)) + LR * 1e-6)
    # the (1 - beta) factors are the fp32 values 1 - 0.9f and 1 - 0.999f
    c1, c2 = float(1 - np.float32(B1)), float(1 - np.float32(B2))
    assert np.allclose(m1, c1 * g.astype(np.float64), rtol=1e-6, atol=0)
    assert np.allclose(v1, c2 * g.astype(np.float64) ** 2, rtol=1e-6, atol=0)


def test_constant_gradient_keeps_a_unit_step(orc):
    """With m = v = 0 and a constant gradient, bias correction makes m_hat = g and v_hat = g^2 at every step t, so
    each of ten steps moves p by lr sign(g)."""
    g = np.array([3e-3, -2e-4, 5e-2, -1.0], np.float32)
    p = np.zeros(4, np.float32)
    m = np.zeros(4, np.float32)
    v = np.zeros(4, np.float32)
    for t in range(1, 11):
        p, m, v = orc.adam_step(p, g, m, v, LR, B1, B2, EPS, *bc(t))
    assert np.allclose(p, -10 * LR * np.sign(g), rtol=1e-4, atol=0)


def test_zero_gradient_decays_moments(orc):
    m0 = np.array([1e-3, -2e-3], np.float32)
    v0 = np.array([4e-6, 1e-6], np.float32)
    p, m, v = orc.adam_step(np.zeros(2, np.float32), np.zeros(2, np.float32), m0, v0, LR, B1, B2, EPS, *bc(1000))
    assert np.allclose(m, 0.9 * m0, rtol=1e-6) and np.allclose(v, 0.999 * v0, rtol=1e-6)
    # the update still follows m_hat / sqrt(v_hat), with bc1 ~ 1 and bc2 ~ 1 - e^-1 at t = 1000
    b1, b2 = bc(1000)
    want = -LR * (0.9 * m0 / b1) / (np.sqrt(0.999 * v0 / b2) + EPS)
    assert np.allclose(p, want, rtol=1e-5)


def test_elements_are_independent(orc):
    rng = np.random.default_rng(1)
    p, g, m = (rng.normal(0, 1e-2, 100).astype(np.float32) for _ in range(3))
    v = (rng.normal(0, 1e-2, 100) ** 2).astype(np.float32)
    full = orc.adam_step(p, g, m, v, LR, B1, B2, EPS, *bc(7))
    for i in (0, 37, 99):
        one = orc.adam_step(p[i:i + 1], g[i:i + 1], m[i:i + 1], v[i:i + 1], LR, B1, B2, EPS, *bc(7))
        assert all(a[i] == b[0] for a, b in zip(full, one))


def test_group_layout_matches_the_pages():
    g = load("layout_sizes.txt")
    widths = dict(scenes.ADAM_GROUP_WIDTHS)
    n = g["splats"]
    assert n * widths["means"] == g["means_grad"] and n * widths["log_scales"] == g["log_scales_grad"]
    assert n * widths["rot_quats"] == g["rot_quats_grad"] and n * widths["raw_opacities"] == g["raw_opacities_grad"]
    assert n * widths["sh_coeffs"] == g["sh_coeffs_grad"]
    assert sum(widths.values()) * g["adam_bytes_per_element"] == g["adam_bytes_per_splat"]
    assert 4 * 4 + 3 * 4 == g["adam_bytes_per_element"]  # read grad, m, v, param; write m, v, param


def test_bias_corrections_at_step_1000():
    b1, b2 = bc(1000)
    # beta2 enters as the fp32 value 0.999f = 0.99900001287, so 1 - beta2^1000 sits 4.7e-6 below 1 - 0.999^1000
    assert b1 == np.float32(1.0) and abs(b2 - (1 - 0.999 ** 1000)) < 1e-5
