"""GPU L1 + SSIM loss (gsr_loss_l1_ssim) against the fp64 oracle (oracle/loss.py).

Bars, from the fp32 arithmetic: the variances sx = G * x^2 - mx^2 (and sy, sxy) lose up to 2u |G * x^2| to
cancellation, u = 2^-24, which relative to their floor C2 = 9e-4 is up to 1.4e-4 of D for values near 1 in the worst
case; the errors of a map value carry both signs and the gradient, a 121-term sum of products of them, averages them
down: measured, its error is at most about 6e-6 of the terms' scale on these images. So, element by element,
  |dL/dx_gpu - ref| <= 2e-5 |ref| + 2e-5 max|ref|      (the second term: the terms' scale, for elements that cancel)
(gpuhelp.loss_grad_bar), tight enough that the oracle's own gradient with a 9- or 13-tap window, a window width of
1.4, a loss weight of 0.19 or C2 10 % off fails it (tests/test_oracle_loss.py); and the three loss values within
2e-5 relative (per-pixel errors with both signs, averaged over the image in fp64). .w of v_out must be 0.
"""
import numpy as np
import pytest

from gpuhelp import banner, dev, host, loss_grad_bar

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    from differentiable_gaussian_splatting_amd import gsr
    c = gsr.Context(0)
    yield c
    c.close()


def smooth_target(rng, H, W):
    """A target with structure at several scales: random values blurred by a box, plus noise, in [0, 1]."""
    base = rng.uniform(0, 1, (H + 8, W + 8, 3))
    k = np.ones(5) / 5
    for ax in (0, 1):
        base = np.apply_along_axis(lambda v: np.convolve(v, k, mode="same"), ax, base)
    t = 0.8 * base[4:H + 4, 4:W + 4] + 0.2 * rng.uniform(0, 1, (H, W, 3))
    return np.clip(t, 0, 1).astype(np.float32)


def check(ctx, out_rgba, target):
    from differentiable_gaussian_splatting_amd import gsr
    from oracle import loss as ol
    v, loss = gsr.gsr_loss_l1_ssim(ctx, dev(out_rgba), dev(target))
    v, loss = host(v), host(loss)
    ref_g, ref_L = ol.l1_ssim_backward(out_rgba, target)
    L, l1, s = ol.l1_ssim(out_rgba, target)
    for got, want in zip(loss, (L, l1, s)):
        assert abs(got - want) <= 2e-5 * abs(want), (loss, (L, l1, s))
    assert (v[..., 3] == 0).all()
    err = np.abs(v[..., :3].astype(np.float64) - ref_g[..., :3])
    ratio = err / loss_grad_bar(ref_g)
    print(f"  loss {loss.tolist()} vs {(L, l1, s)}; gradient worst error / bound {ratio.max():.3g}")
    assert ratio.max() <= 1.0, np.unravel_index(np.argmax(ratio), ratio.shape)


@pytest.mark.parametrize("w,h", [(16, 16), (37, 23), (64, 64), (100, 37), (1, 40), (200, 145)])
def test_loss_on_random_images(ctx, w, h):
    banner(f"loss random {w}x{h}")
    rng = np.random.default_rng(w * 1000 + h)
    x = np.zeros((h, w, 4), np.float32)
    x[..., :3] = rng.uniform(0, 1, (h, w, 3))
    x[..., 3] = rng.uniform(0, 1, (h, w))
    check(ctx, x, smooth_target(rng, h, w))


def test_loss_on_a_rendered_image(ctx):
    """The forward's output at 800 x 800 (the path's image) against a structured target."""
    from differentiable_gaussian_splatting_amd import gsr, scenes
    banner("loss rendered raster410k")
    sc = scenes.make_scene("raster410k")
    sp = dev(sc.splats)
    bins = gsr.gsr_bin(ctx, sp, dev(sc.depths), sc.width, sc.height)
    out, _, _ = gsr.gsr_render_forward(ctx, sp, bins, sc.width, sc.height)
    check(ctx, host(out), smooth_target(np.random.default_rng(3), sc.height, sc.width))


def test_identical_images_give_zero_loss_and_gradient(ctx):
    from differentiable_gaussian_splatting_amd import gsr
    banner("loss identical images")
    rng = np.random.default_rng(6)
    x = rng.uniform(0, 1, (48, 40, 4)).astype(np.float32)
    v, loss = gsr.gsr_loss_l1_ssim(ctx, dev(x), dev(np.ascontiguousarray(x[..., :3])))
    v, loss = host(v), host(loss)
    assert abs(loss[0]) < 1e-6 and loss[1] == 0 and abs(loss[2] - 1) < 1e-6
    # the SSIM terms cancel exactly in exact arithmetic; fp32 leaves a residue far below one gradient unit 1 / (3 H W)
    assert np.abs(v).max() < 1e-3 / (3 * 48 * 40)


def test_loss_is_the_same_on_every_run(ctx):
    from differentiable_gaussian_splatting_amd import gsr
    banner("loss repeatability")
    rng = np.random.default_rng(7)
    x = rng.uniform(0, 1, (160, 130, 4)).astype(np.float32)
    y = smooth_target(rng, 160, 130)
    runs = [tuple(host(t).tobytes() for t in gsr.gsr_loss_l1_ssim(ctx, dev(x), dev(y))) for _ in range(3)]
    assert runs[0] == runs[1] == runs[2]
