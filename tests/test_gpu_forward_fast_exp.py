"""The forward with the hardware exponential (GSR_OPT_FORWARD_EXP = GSR_EXP_FAST) against the oracle.

In this mode exp(-sigma) is the hardware's (relative error below 1e-6) except within 2^-18 of the 1/255 threshold,
where the kernel takes the correctly rounded value: the reject decisions stay exact, so a pixel's compositing
candidates are the oracle's, but alpha (the 0.999 clamp included, which picks between o G and 0.999) and the
transmittance carry the fast values' error. The parity bar:
  * pixels whose last_contrib equals the oracle's: image and final_T within 1e-5 absolute (as the exact mode);
  * any other pixel must have stopped on a decision that rounding can flip: from the oracle's stop-free candidate
    trace, every candidate the GPU composited has exact T' >= 1e-4 (1 - e), and the one it stopped at (if the list
    went on) has exact T' < 1e-4 (1 + e), where e bounds the relative error of the GPU's T' there:
    e_j = sum over candidates i <= j of (alpha_i / (1 - alpha_i)) d + 3 u, with d = 2e-6 the bound on the fast
    alpha's relative error (argument rounding 6.6e-7, the hardware exp 1 ulp, the product 1 ulp: 8.4e-7, doubled)
    and u = 2^-24 for the rounding of 1 - alpha and of the product; its image and T must equal, within 1e-5, the
    oracle's colour and T composited up to the GPU's last contributor;
  * such pixels are rare: at most 1e-3 of the image.
The backward does not depend on the forward's exponential; its parity is tested on the oracle forward's outputs
(test_gpu_raster.py).
[A.9 f16 forward page, implementation listing; W1 warp sparse skip + exp-skip page, summary]
"""
import numpy as np
import pytest

from gpuhelp import banner, custom_scene, dev, host, oracle_bins, oracle_forward, scene

pytestmark = pytest.mark.gpu

IMG_TOL = 1e-5
ALPHA_REL = 2e-6
U = 2.0 ** -24


@pytest.fixture(scope="module")
def ctx():
    from differentiable_gaussian_splatting_amd import gsr
    c = gsr.Context(0)
    gsr.gsr_set_option(c, gsr.GSR_OPT_FORWARD_EXP, gsr.GSR_EXP_FAST)
    yield c
    c.close()


def stop_bound(alpha):
    """e_j for each candidate j of a trace (see the module docstring)."""
    a = alpha.astype(np.float64)
    return np.cumsum(a / (1.0 - a) * ALPHA_REL + 3 * U)


def check_fast_forward(gpu, ref, splats, ob, w, h):
    """Applies the module's bar; returns the number of pixels that stopped apart from the oracle."""
    import oracle
    out, ft, lc = host(gpu[0]), host(gpu[1]), host(gpu[2], np.uint32)
    r_out, r_ft, r_lc = ref[:3]
    same = lc == r_lc
    if same.any():
        d_img = np.abs(out - r_out)[same].max()
        d_T = np.abs(ft - r_ft)[same].max()
        assert d_img <= IMG_TOL and d_T <= IMG_TOL, (d_img, d_T)
    apart = np.argwhere(~same)
    assert len(apart) <= max(3, 1e-3 * lc.size), f"{len(apart)} pixels stop apart from the oracle"
    for py, px in apart:
        tr = oracle.trace_candidates(splats, ob, w, h, int(px), int(py))
        pos, tn, e = tr["pos"], tr["T_next"].astype(np.float64), stop_bound(tr["alpha"])
        if lc[py, px] == 0:
            i_g = -1
        else:
            hit = np.flatnonzero(pos == lc[py, px])
            assert len(hit) == 1, f"({px}, {py}): last_contrib {lc[py, px]} is not a compositing candidate"
            i_g = int(hit[0])
        # every candidate the GPU composited: exact T' at or above the threshold, up to the bound
        for j in range(i_g + 1):
            assert tn[j] >= 1e-4 * (1 - e[j]), (px, py, j, tn[j], e[j])
        # the candidate it stopped at, when the list went on
        if i_g + 1 < len(pos):
            j = i_g + 1
            assert tn[j] < 1e-4 * (1 + e[j]), (px, py, j, tn[j], e[j])
        want_rgb = tr["rgb"][i_g] if i_g >= 0 else np.zeros(3, np.float32)
        want_T = tn[i_g] if i_g >= 0 else 1.0
        assert np.abs(out[py, px, :3] - want_rgb).max() <= IMG_TOL and abs(ft[py, px] - want_T) <= IMG_TOL
        assert abs(out[py, px, 3] - (1 - want_T)) <= IMG_TOL
    return len(apart)


@pytest.mark.parametrize("name", ["tiny", "raster84k", "raster410k"])
def test_fast_forward_matches_oracle(ctx, name):
    from differentiable_gaussian_splatting_amd import gsr
    banner(f"forward fast exp {name}")
    sc = scene(name)
    sp = dev(sc.splats)
    bins = gsr.gsr_bin(ctx, sp, dev(sc.depths), sc.width, sc.height)
    gpu = gsr.gsr_render_forward(ctx, sp, bins, sc.width, sc.height)
    apart = check_fast_forward(gpu, oracle_forward(name), sc.splats, oracle_bins(name), sc.width, sc.height)
    print(f"  pixels stopped apart from the oracle: {apart}")


@pytest.mark.parametrize("w,h", [(24, 24), (100, 37), (17, 1), (200, 145)])
def test_fast_forward_ragged_images(ctx, w, h):
    import oracle
    from differentiable_gaussian_splatting_amd import gsr
    banner(f"forward fast exp ragged {w}x{h}")
    sc = custom_scene(name="rag", width=w, height=h, n=1500, seed=w + 31 * h,
                      size_classes=((0.7, 0.3, 4.0), (0.3, 4.0, 30.0)), opacity_mu=0.5, margin=30.0)
    ob = oracle.bin(sc.splats, sc.depths, w, h)
    sp = dev(sc.splats)
    bins = gsr.gsr_bin(ctx, sp, dev(sc.depths), w, h)
    check_fast_forward(gsr.gsr_render_forward(ctx, sp, bins, w, h), oracle.render_forward(sc.splats, ob, w, h),
                       sc.splats, ob, w, h)


def test_fast_forward_closed_form_stop_rule(ctx):
    """14 centred o = 0.5 splats: at sigma = 0 the hardware exponential is exact (2^0), so the chain is exact too:
    T = 2^-13 after 13 composites and the 14th stops."""
    from differentiable_gaussian_splatting_amd import gsr
    banner("forward fast exp stop rule")
    sp = np.tile(np.array([8.5, 8.5, 0.25, 0.0, 0.25, 1.0, 0.5, 0.25, 0.5], np.float32), (14, 1))
    bins = gsr.gsr_bin(ctx, dev(sp), dev(np.arange(1, 15, dtype=np.float32)), 16, 16)
    out, ft, lc = gsr.gsr_render_forward(ctx, dev(sp), bins, 16, 16)
    assert host(ft)[8, 8] == 2.0 ** -13 and host(lc)[8, 8] == 13


def test_fast_forward_bar_rejects_a_wrong_stop(ctx):
    """The bar is not vacuous: the exact forward's outputs with one pixel's last contributor moved two candidates
    back (a stop far from the threshold) fail it."""
    import oracle
    banner("forward fast exp bar check")
    name = "raster84k"
    sc = scene(name)
    ob = oracle_bins(name)
    ref = oracle_forward(name)
    lc = ref[2].copy()
    for py, px in np.argwhere(lc > 0)[::97]:  # a pixel whose candidate before its last is far above 1e-4
        tr = oracle.trace_candidates(sc.splats, ob, sc.width, sc.height, int(px), int(py))
        i = int(np.flatnonzero(tr["pos"] == lc[py, px])[0])
        if i >= 2 and tr["T_next"][i - 1] > 2e-4:
            break
    else:
        pytest.fail("no pixel to plant the wrong stop in")
    lc[py, px] = tr["pos"][i - 2]
    out, ft = ref[0].copy(), ref[1].copy()
    out[py, px, :3], ft[py, px] = tr["rgb"][i - 2], tr["T_next"][i - 2]
    out[py, px, 3] = 1 - ft[py, px]
    fake = tuple(dev(a) for a in (out, ft, lc))
    with pytest.raises(AssertionError):
        check_fast_forward(fake, ref, sc.splats, ob, sc.width, sc.height)
