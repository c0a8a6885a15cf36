"""Pins of the oracle's backward pass: central finite differences, closed forms and the f32/f64 agreement.

The 9 per-splat gradients (mean xy, conic 3, rgb 3, opacity) and the forward-order form after = C_final - acc - mine
follow the M3 per-splat backward page (section 1, "brush's actual structure" and "differences" rows); the
"raw_alpha < 0.999" branch is the clamp condition named there.
"""
import math

import numpy as np
import pytest

from differentiable_gaussian_splatting_amd import scenes

RGB = (1.0, 0.5, 0.25)


def iso_splat(x, y, s, o, rgb=RGB):
    return np.array([x, y, 1.0 / (s * s), 0.0, 1.0 / (s * s), *rgb, o], np.float64)


def loss_and_fp(orc, sp64, bins, w, h, g):
    out, ft, lc, st = orc.render_forward(sp64, bins, w, h, "f64")
    return float(np.sum(out[..., :3] * g[..., :3])), st["fingerprint"]


def analytic(orc, sp64, bins, w, h, g, precision="f64"):
    out, ft, lc, _ = orc.render_forward(sp64, bins, w, h, precision)
    return orc.render_backward(sp64, bins, w, h, out, ft, lc, g, precision)


# ----------------------------------------------------------------------------------------------- closed forms
def single_bins(orc, n):
    return orc.Bins(np.zeros(n, np.uint64), np.arange(n, dtype=np.uint32), np.array([[0, n]], np.uint32), 1, 1)


def one_pixel_grad(h, w, px, py, ch):
    g = np.zeros((h, w, 4))
    g[py, px, ch] = 1.0
    return g


def test_single_splat_at_sigma_zero(orc):
    sp = iso_splat(8.5, 8.5, 2.0, 0.5)[None]
    b = single_bins(orc, 1)
    for ch in range(3):
        gr = analytic(orc, sp, b, 16, 16, one_pixel_grad(16, 16, 8, 8, ch))[0]
        # dC_ch/d rgb_ch = alpha = 0.5; dC_ch/do = rgb_ch * G = rgb_ch; at sigma = 0 the mean and conic gradients vanish
        assert gr[5 + ch] == 0.5 and sum(abs(gr[5 + k]) for k in range(3) if k != ch) == 0
        assert gr[8] == pytest.approx(RGB[ch], abs=1e-15)
        assert np.all(gr[:5] == 0)


def test_clamped_splat_has_no_opacity_or_geometry_gradient(orc):
    sp = iso_splat(8.5, 8.5, 2.0, 1.0)[None]
    g = np.random.default_rng(0).normal(size=(16, 16, 4))
    gr = analytic(orc, sp, single_bins(orc, 1), 16, 16, g)[0]
    # o * G >= 0.999 only near the centre; take one pixel there only
    g1 = one_pixel_grad(16, 16, 8, 8, 0)
    gr = analytic(orc, sp, single_bins(orc, 1), 16, 16, g1)[0]
    assert gr[5] == pytest.approx(float(np.float32(0.999)), abs=1e-12)
    assert np.all(gr[[0, 1, 2, 3, 4, 8]] == 0)


def test_two_splat_opacity_gradient(orc):
    # dC/d alpha_1 = c1 - c2 alpha_2 for C = c1 a1 + c2 a2 (1 - a1); at sigma = 0, d alpha_1 / d o_1 = 1
    c1, c2 = (1.0, 0.0, 0.5), (0.25, 1.0, 0.5)
    sp = np.stack([iso_splat(8.5, 8.5, 2.0, 0.5, c1), iso_splat(8.5, 8.5, 2.0, 0.25, c2)])
    b = single_bins(orc, 2)
    for ch in range(3):
        gr = analytic(orc, sp, b, 16, 16, one_pixel_grad(16, 16, 8, 8, ch))
        assert gr[0, 8] == pytest.approx(c1[ch] - c2[ch] * 0.25, abs=1e-15)
        assert gr[1, 8] == pytest.approx(c2[ch] * (1 - 0.5), abs=1e-15)
        assert gr[1, 5 + ch] == pytest.approx(0.25 * 0.5, abs=1e-15)


def test_mean_gradient_of_one_isotropic_splat(orc):
    # C = rgb o exp(-|d|^2 / (2 s^2)) at one pixel; dC/dx = C * (px + 0.5 - x) / s^2
    s, o, x, y = 2.0, 0.6, 8.2, 8.9
    sp = iso_splat(x, y, s, o)[None]
    px, py = 9, 8
    dx, dy = px + 0.5 - x, py + 0.5 - y
    C = o * math.exp(-(dx * dx + dy * dy) / (2 * s * s))
    gr = analytic(orc, sp, single_bins(orc, 1), 16, 16, one_pixel_grad(16, 16, px, py, 0))[0]
    assert gr[0] == pytest.approx(C * dx / (s * s), rel=1e-12)
    assert gr[1] == pytest.approx(C * dy / (s * s), rel=1e-12)
    # dC/da = -C dx^2 / 2, dC/db = -C dx dy, dC/dc = -C dy^2 / 2 for sigma = (a dx^2 + 2 b dx dy + c dy^2) / 2
    assert gr[2] == pytest.approx(-C * dx * dx / 2, rel=1e-12)
    assert gr[3] == pytest.approx(-C * dx * dy, rel=1e-12)
    assert gr[4] == pytest.approx(-C * dy * dy / 2, rel=1e-12)


# ----------------------------------------------------------------------------------------------- finite differences
def _fd_check(orc, sc, bins, g, idx_list, rel=1e-4, abs_tol=1e-6):
    w, h = sc.width, sc.height
    sp = sc.splats.astype(np.float64)
    an = analytic(orc, sp, bins, w, h, g)
    _, fp0 = loss_and_fp(orc, sp, bins, w, h, g)
    checked = skipped = 0
    worst = 0.0
    for i in idx_list:
        for j in range(9):
            th = sp[i, j]
            hstep = 1e-6 * max(1.0, abs(th))
            spp, spm = sp.copy(), sp.copy()
            spp[i, j] = th + hstep
            spm[i, j] = th - hstep
            lp, fpp = loss_and_fp(orc, spp, bins, w, h, g)
            lm, fpm = loss_and_fp(orc, spm, bins, w, h, g)
            if fpp != fp0 or fpm != fp0:  # a branch decision changed inside the stencil
                skipped += 1
                continue
            fd = (lp - lm) / (2 * hstep)
            err = abs(fd - an[i, j])
            worst = max(worst, err / (abs_tol + rel * abs(an[i, j])))
            assert err <= abs_tol + rel * abs(an[i, j]), (i, j, fd, an[i, j])
            checked += 1
    return checked, skipped, worst


def test_finite_differences_tiny_scene(orc):
    """Central differences of L = sum_px g . C over all 9 parameters of every splat of the tiny scene, in float64 with
    the bins frozen; stencils that flip a decision are skipped and counted."""
    sc = scenes.make_scene("tiny")
    bins = orc.bin(sc.splats, sc.depths, 64, 64)
    g = sc.v_out.astype(np.float64)
    checked, skipped, worst = _fd_check(orc, sc, bins, g, range(sc.spec.n))
    assert checked > 0.97 * 9 * sc.spec.n, (checked, skipped)


def test_finite_differences_dense_scene_with_stops(orc):
    sc = scenes.make_scene(scenes.SceneSpec("fd-dense", 40, 36, 400, seed=31,
                                            size_classes=((0.7, 0.3, 4.0), (0.3, 4.0, 16.0)),
                                            opacity_mu=1.0, opacity_sd=1.5, margin=6.0))
    bins = orc.bin(sc.splats, sc.depths, 40, 36)
    out, ft, lc, st = orc.render_forward(sc.splats.astype(np.float64), bins, 40, 36, "f64")
    assert st["stopped"] > 50  # the stop rule is exercised
    g = sc.v_out.astype(np.float64)
    rng = np.random.default_rng(1)
    checked, skipped, _ = _fd_check(orc, sc, bins, g, rng.choice(400, 120, replace=False))
    assert checked > 0.9 * 9 * 120, (checked, skipped)


@pytest.mark.parametrize("seed,vout_sd,smax", [(1, 0.01, 40.0), (2, 0.01, 40.0)])
def test_f32_backward_matches_f64(orc, seed, vout_sd, smax):
    """The fp32 oracle against the fp64 one at the workloads' upstream scales: N(0, 0.01) with splats up to 40 px
    and N(0, 1) with splats up to 8 px. (With N(0, 1) upstream gradients and 40 px splats the fp32 forward-order
    form itself loses about 2e-4 relative accuracy in conic gradients, from the cancellation in
    after = C_final - acc - mine.)"""
    sc = scenes.make_scene(scenes.SceneSpec("mix", 96, 80, 2000, seed=seed,
                                            size_classes=((0.7, 0.3, min(4.0, smax)), (0.3, min(4.0, smax), smax)),
                                            opacity_mu=-0.5, opacity_sd=1.5, vout_sd=vout_sd, margin=8.0))
    bins = orc.bin(sc.splats, sc.depths, 96, 80)
    # the comparison is about arithmetic, so both precisions must take the same decisions on this scene
    assert orc.render_forward(sc.splats, bins, 96, 80, "f32")[3]["fingerprint"] == \
        orc.render_forward(sc.splats.astype(np.float64), bins, 96, 80, "f64")[3]["fingerprint"]
    g32 = analytic(orc, sc.splats, bins, 96, 80, sc.v_out, "f32")
    g64 = analytic(orc, sc.splats.astype(np.float64), bins, 96, 80, sc.v_out.astype(np.float64))
    assert np.allclose(g32, g64, rtol=1e-4, atol=1e-4)


def test_f32_backward_matches_f64_tiny_scene(orc):
    sc = scenes.make_scene("tiny")
    bins = orc.bin(sc.splats, sc.depths, 64, 64)
    g32 = analytic(orc, sc.splats, bins, 64, 64, sc.v_out, "f32")
    g64 = analytic(orc, sc.splats.astype(np.float64), bins, 64, 64, sc.v_out.astype(np.float64))
    assert np.allclose(g32, g64, rtol=1e-4, atol=1e-4)


def test_threaded_oracle_matches_single_threaded(orc):
    """The all-cores timing wrapper runs the same per-pixel code by bands of tile rows: identical forward outputs,
    backward sums equal up to the order of double additions."""
    from differentiable_gaussian_splatting_amd import scenes
    sc = scenes.make_scene(scenes.SceneSpec(name="mt", width=120, height=88, n=2000, seed=41,
                                            size_classes=((1.0, 0.5, 12.0),)))
    b = orc.bin(sc.splats, sc.depths, 120, 88)
    out, ft, lc, _ = orc.render_forward(sc.splats, b, 120, 88)
    g = orc.render_backward(sc.splats, b, 120, 88, out, ft, lc, sc.v_out)
    for threads in (1, 3, 8):
        o2, f2, l2 = orc.render_forward_mt(sc.splats, b, 120, 88, threads)
        assert np.array_equal(o2, out) and np.array_equal(f2, ft) and np.array_equal(l2, lc)
        g2 = orc.render_backward_mt(sc.splats, b, 120, 88, out, ft, lc, sc.v_out, threads)
        assert np.allclose(g2, g, rtol=1e-6, atol=1e-9)


# ------------------------------------------------------------------ exact values on the fp32 method's decisions
@pytest.mark.parametrize("seed,vout_sd,smax", [(1, 0.01, 40.0), (2, 1.0, 8.0), (3, 1.0, 40.0)])
def test_exact_backward_is_the_fp64_chain_where_decisions_agree(orc, seed, vout_sd, smax):
    """render_backward_exact takes its decisions in fp32 and its values in fp64; on scenes where the fp32 and fp64
    forwards take every decision alike (same fingerprint), given the fp64 forward's output it must equal the fp64
    backward on it up to the order of double additions - the f64 path that the finite-difference pins above check."""
    sc = scenes.make_scene(scenes.SceneSpec("ex", 96, 80, 2000, seed=seed,
                                            size_classes=((0.7, 0.3, min(4.0, smax)), (0.3, min(4.0, smax), smax)),
                                            opacity_mu=-0.5, opacity_sd=1.5, vout_sd=vout_sd, margin=8.0))
    bins = orc.bin(sc.splats, sc.depths, 96, 80)
    out32, ft32, lc32, st32 = orc.render_forward(sc.splats, bins, 96, 80, "f32")
    sp64 = sc.splats.astype(np.float64)
    out64, ft64, lc64, st64 = orc.render_forward(sp64, bins, 96, 80, "f64")
    assert st32["fingerprint"] == st64["fingerprint"]
    g64 = orc.render_backward(sp64, bins, 96, 80, out64, ft64, lc64, sc.v_out.astype(np.float64), "f64")
    gx = orc.render_backward_exact(sc.splats, bins, 96, 80, out64, lc32, sc.v_out)
    scale = np.abs(g64).max()
    assert np.allclose(gx, g64, rtol=1e-9, atol=1e-12 * scale)
    # and on the fp32 forward's output the fp32 oracle is within its own rounding of it (loose: the last case is
    # where the fp32 form loses 2e-4)
    g32 = orc.render_backward(sc.splats, bins, 96, 80, out32, ft32, lc32, sc.v_out)
    gx32 = orc.render_backward_exact(sc.splats, bins, 96, 80, out32, lc32, sc.v_out)
    assert np.allclose(g32, gx32, rtol=1e-3, atol=1e-3 * scale)


def test_exact_backward_follows_the_fp32_decisions(orc):
    """A pixel whose fp32 o G reaches the 0.999 clamp while the fp64 product stays below it: the fp32 evaluation
    clamps (no opacity or geometry gradient from the pixel), fp64 would not; the exact-value backward follows fp32,
    with alpha = 0.999 exactly."""
    f = np.float32
    a = f(0.25)
    found = None
    for k in range(1, 400):  # splat offsets dx = -k / 1000 px: sigma about 1.25e-7 k^2, each a different G
        x = f(8.5 + k / 1000.0)
        dx = f(8.5) - x
        G32 = f(math.exp(-float(f(0.5) * (a * dx * dx))))
        G64 = math.exp(-(0.5 * (float(a) * float(dx) * float(dx))))
        o0 = f(float(f(0.999)) / G64)
        for step in range(-8, 9):  # o within a few ulps of the clamp
            o = o0
            for _ in range(abs(step)):
                o = np.nextafter(o, f(2) if step > 0 else f(0))
            if o <= 1 and f(o * G32) >= f(0.999) and float(o) * G64 < float(f(0.999)):
                found = o
                break
        if found is not None:
            break
    assert found is not None
    sp = np.array([x, 8.5, a, 0.0, a, 1.0, 0.5, 0.25, found], np.float32)
    g = np.zeros((16, 16, 4), np.float32)
    g[8, 8, 0] = 1.0
    lc = np.zeros((16, 16), np.uint32)
    lc[8, 8] = 1
    gx = orc.render_backward_exact(sp[None], single_bins(orc, 1), 16, 16, np.zeros((16, 16, 4)), lc, g)[0]
    assert gx[8] == 0 and np.all(gx[:5] == 0)            # clamped: no opacity or geometry term
    assert gx[5] == float(f(0.999))                       # alpha = 0.999 exactly, T = 1
