"""Pins of the L1 + SSIM loss oracle (oracle/loss.py): the window's closed form, a brute-force windowed sum with
explicit zero padding, closed forms on constant images, the identity case, the L1 term alone, and central finite
differences of the gradient."""
import math

import numpy as np

from oracle import loss as ol


def test_window_taps_closed_form():
    g = ol.gaussian_taps(11, 1.5)
    assert abs(g.sum() - 1) < 1e-15 and np.allclose(g, g[::-1], rtol=0, atol=0)
    assert np.argmax(g) == 5
    for i in range(5, 10):
        assert math.isclose(g[i + 1] / g[i], math.exp(-(2 * (i - 5) + 1) / (2 * 1.5 ** 2)), rel_tol=1e-13)


def brute_ssim(x, y, k, sigma):
    """SSIM map by explicit windowed sums over the zero-padded image, pixel by pixel."""
    g = ol.gaussian_taps(k, sigma)
    w = np.outer(g, g)
    H, W = x.shape
    r = k // 2
    S = np.zeros((H, W))
    for i in range(H):
        for j in range(W):
            m = [0.0] * 5
            for di in range(-r, r + 1):
                for dj in range(-r, r + 1):
                    ii, jj = i + di, j + dj
                    if 0 <= ii < H and 0 <= jj < W:
                        a, b, ww = x[ii, jj], y[ii, jj], w[di + r, dj + r]
                        m[0] += ww * a
                        m[1] += ww * b
                        m[2] += ww * a * a
                        m[3] += ww * b * b
                        m[4] += ww * a * b
            mx, my = m[0], m[1]
            sx, sy, sxy = m[2] - mx * mx, m[3] - my * my, m[4] - mx * my
            S[i, j] = ((2 * mx * my + ol.C1) * (2 * sxy + ol.C2)) / ((mx * mx + my * my + ol.C1) * (sx + sy + ol.C2))
    return S


def test_ssim_map_against_brute_force():
    rng = np.random.default_rng(1)
    H, W = 9, 13
    x = rng.uniform(0, 1, (H, W, 4))
    y = rng.uniform(0, 1, (H, W, 3))
    for k, sigma in ((11, 1.5), (7, 1.5)):
        S = ol.ssim_map(x, y, k, sigma)
        for c in range(3):
            assert np.allclose(S[c], brute_ssim(x[..., c], y[..., c], k, sigma), rtol=1e-12, atol=1e-14)
    L, l1, s = ol.l1_ssim(x, y)
    assert math.isclose(l1, np.abs(x[..., :3] - y).mean(), rel_tol=1e-13)
    assert math.isclose(s, ol.ssim_map(x, y).mean(), rel_tol=1e-13)
    assert math.isclose(L, 0.8 * l1 + 0.2 * (1 - s), rel_tol=1e-13)


def test_constant_images_interior_closed_form():
    H, W = 24, 25
    a, b = 0.3, 0.7
    x = np.full((H, W, 3), a)
    y = np.full((H, W, 3), b)
    S = ol.ssim_map(x, y)
    want = (2 * a * b + ol.C1) / (a * a + b * b + ol.C1)
    assert np.allclose(S[:, 5:-5, 5:-5], want, rtol=1e-10)
    # at a corner only the window's quarter (6 x 6 taps) lies inside the image: the means shrink by that weight
    g = ol.gaussian_taps()
    q = g[5:].sum() ** 2
    mx, my = q * a, q * b
    sx, sy, sxy = q * a * a - mx * mx, q * b * b - my * my, q * a * b - mx * my
    corner = ((2 * mx * my + ol.C1) * (2 * sxy + ol.C2)) / ((mx * mx + my * my + ol.C1) * (sx + sy + ol.C2))
    assert math.isclose(S[0, 0, 0], corner, rel_tol=1e-10)


def test_identical_images_give_zero_loss_and_gradient():
    rng = np.random.default_rng(2)
    x = rng.uniform(0, 1, (12, 10, 4))
    g, L = ol.l1_ssim_backward(x, x[..., :3])
    assert abs(L) < 1e-14
    assert np.abs(g).max() < 1e-15


def test_l1_term_alone():
    rng = np.random.default_rng(3)
    x = rng.uniform(0, 1, (6, 7, 4))
    y = rng.uniform(0, 1, (6, 7, 3))
    g, L = ol.l1_ssim_backward(x, y, lam=0.0)
    assert math.isclose(L, np.abs(x[..., :3] - y).mean(), rel_tol=1e-13)
    assert np.allclose(g[..., :3], np.sign(x[..., :3] - y) / (3 * 6 * 7), rtol=1e-13)
    assert (g[..., 3] == 0).all()


def test_gradient_matches_central_differences():
    rng = np.random.default_rng(4)
    H, W = 8, 9
    x = rng.uniform(0.1, 0.9, (H, W, 4))
    y = rng.uniform(0.1, 0.9, (H, W, 3))
    g, _ = ol.l1_ssim_backward(x, y)
    h = 1e-7
    for (i, j, c) in [(0, 0, 0), (3, 4, 1), (7, 8, 2), (4, 0, 2), (2, 6, 0), (5, 5, 1)]:
        xp, xm = x.copy(), x.copy()
        xp[i, j, c] += h
        xm[i, j, c] -= h
        fd = (ol.l1_ssim(xp, y)[0] - ol.l1_ssim(xm, y)[0]) / (2 * h)
        assert math.isclose(fd, g[i, j, c], rel_tol=1e-6, abs_tol=1e-12), ((i, j, c), fd, g[i, j, c])


def test_gpu_bar_fails_planted_mistakes():
    """The GPU test's gradient bar (gpuhelp.loss_grad_bar) is tight enough to catch a wrong reading: the oracle's
    gradient under a 13- or 9-tap window, a window width of 1.4, a loss weight of 0.19 or C2 10 % too large
    differs from the correct one by more than the bar, on the 64 x 64 image of the GPU test."""
    import sys, os
    sys.path.insert(0, os.path.dirname(__file__))
    from gpuhelp import loss_grad_bar
    rng = np.random.default_rng(64 * 1000 + 64)
    h = w = 64
    x = np.zeros((h, w, 4), np.float32)
    x[..., :3] = rng.uniform(0, 1, (h, w, 3))
    x[..., 3] = rng.uniform(0, 1, (h, w))
    y = rng.uniform(0, 1, (h, w, 3)).astype(np.float32)
    ref, _ = ol.l1_ssim_backward(x, y)
    bar = loss_grad_bar(ref)
    for kw in (dict(k=13), dict(k=9), dict(sigma=1.4), dict(lam=0.19)):
        g, _ = ol.l1_ssim_backward(x, y, **kw)
        assert (np.abs(g[..., :3] - ref[..., :3]) / bar).max() > 5.0, kw
    c2 = ol.C2
    try:
        ol.C2 = c2 * 1.1
        g, _ = ol.l1_ssim_backward(x, y)
    finally:
        ol.C2 = c2
    assert (np.abs(g[..., :3] - ref[..., :3]) / bar).max() > 5.0
