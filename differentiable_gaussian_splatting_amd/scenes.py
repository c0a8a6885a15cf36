"""Seeded synthetic inputs for the splat rasterizer: 2D splats, depths, upstream image gradients, Adam state.

This module only draws inputs. It holds none of the rasterizer's arithmetic, so the HIP path and the CPU oracle can
both be fed from it without sharing any of the method's code.

A splat record is 9 float32 values {x, y, a, b, c, r, g, b, o}: the mean in pixels, the conic [[a, b], [b, c]] (the
inverse of the 2D covariance), the colour and the opacity color_a. The covariance is R diag(s1^2, s2^2) R^T with a
rotation angle theta, built in float64 and inverted before rounding to float32.

Draw order for every scene (numpy default_rng(seed)): x, y, (size class), s1, s2, theta, opacity, rgb, depth, then
the upstream image gradient. The workloads below stand in for the trained 410k-splat Lego checkpoint at 800x800 that
the pages measure on, which is not available; they keep its image size and splat count.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass
class SceneSpec:
    name: str
    width: int
    height: int
    n: int
    seed: int
    # (fraction, s_min, s_max) size classes, each log-uniform in [s_min, s_max] pixels
    size_classes: tuple = ((1.0, 0.5, 8.0),)
    opacity_mu: float = 0.0      # color_a = sigmoid(N(opacity_mu, opacity_sd))
    opacity_sd: float = 1.0
    depth_lo: float = 0.1
    depth_hi: float = 10.0
    vout_sd: float = 1.0         # upstream dL/dpixel ~ N(0, vout_sd) per channel
    depth_levels: int = 0        # > 0: depths quantised to this many levels (forces ties)
    margin: float = 0.0          # means drawn over [-margin, W + margin) x [-margin, H + margin)


# The five workloads: a tiny scene, two 800x800 raster scenes, a binning stress case and the full iteration shape.
SPECS = {
    "tiny": SceneSpec("tiny", 64, 64, 256, seed=1, size_classes=((1.0, 0.5, 8.0),), vout_sd=1.0),
    "raster84k": SceneSpec("raster84k", 800, 800, 84_000, seed=2, size_classes=((1.0, 0.3, 20.0),),
                           vout_sd=0.01),
    "raster410k": SceneSpec("raster410k", 800, 800, 410_000, seed=3,
                            size_classes=((0.7, 0.3, 4.0), (0.3, 4.0, 40.0)),
                            opacity_mu=-2.0, opacity_sd=1.5, vout_sd=0.01),
    "bin1m": SceneSpec("bin1m", 800, 800, 1_000_000, seed=4, size_classes=((1.0, 0.5, 40.0),)),
    "iter410k": SceneSpec("iter410k", 800, 800, 410_000, seed=5,
                          size_classes=((0.7, 0.3, 4.0), (0.3, 4.0, 40.0)),
                          opacity_mu=-2.0, opacity_sd=1.5, vout_sd=0.01),
}

# Adam parameter groups per splat: means 3, log_scales 3, rot_quats 4, raw_opacities 1, SH coefficients 16 x 3.
ADAM_GROUP_WIDTHS = (("means", 3), ("log_scales", 3), ("rot_quats", 4), ("raw_opacities", 1), ("sh_coeffs", 48))


@dataclass
class Scene:
    spec: SceneSpec
    splats: np.ndarray   # float32 [N, 9]
    depths: np.ndarray   # float32 [N]
    v_out: np.ndarray    # float32 [H, W, 4] (.w is drawn but ignored by the method)
    extra: dict = field(default_factory=dict)

    @property
    def width(self):
        return self.spec.width

    @property
    def height(self):
        return self.spec.height


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def make_scene(spec: SceneSpec | str, **overrides) -> Scene:
    if isinstance(spec, str):
        spec = SPECS[spec]
    if overrides:
        spec = SceneSpec(**{**spec.__dict__, **overrides})
    rng = np.random.default_rng(spec.seed)
    n, W, H = spec.n, spec.width, spec.height
    m = spec.margin
    x = rng.uniform(-m, W + m, n)
    y = rng.uniform(-m, H + m, n)
    # size class per splat: exact class counts, assigned by a random permutation
    fracs = np.array([c[0] for c in spec.size_classes], np.float64)
    counts = np.floor(fracs / fracs.sum() * n).astype(np.int64)
    counts[0] += n - counts.sum()
    cls = np.repeat(np.arange(len(counts)), counts)[rng.permutation(n)]
    lo = np.log(np.array([c[1] for c in spec.size_classes]))[cls]
    hi = np.log(np.array([c[2] for c in spec.size_classes]))[cls]
    s1 = np.exp(rng.uniform(lo, hi))
    s2 = np.exp(rng.uniform(lo, hi))
    theta = rng.uniform(0.0, np.pi, n)
    opac = _sigmoid(rng.normal(spec.opacity_mu, spec.opacity_sd, n))
    rgb = rng.uniform(0.0, 1.0, (n, 3))
    depth = rng.uniform(spec.depth_lo, spec.depth_hi, n)
    if spec.depth_levels > 0:
        depth = spec.depth_lo + np.floor((depth - spec.depth_lo) / (spec.depth_hi - spec.depth_lo)
                                         * spec.depth_levels) / spec.depth_levels * (spec.depth_hi - spec.depth_lo)
        depth = np.maximum(depth, spec.depth_lo)
    # covariance R diag(s1^2, s2^2) R^T and its inverse, in float64
    c, s = np.cos(theta), np.sin(theta)
    v1, v2 = s1 * s1, s2 * s2
    sxx = c * c * v1 + s * s * v2
    syy = s * s * v1 + c * c * v2
    sxy = c * s * (v1 - v2)
    det = sxx * syy - sxy * sxy
    splats = np.stack([x, y, syy / det, -sxy / det, sxx / det, rgb[:, 0], rgb[:, 1], rgb[:, 2], opac], axis=1)
    v_out = rng.normal(0.0, spec.vout_sd, (H, W, 4))
    return Scene(spec, splats.astype(np.float32), depth.astype(np.float32), v_out.astype(np.float32),
                 extra={"s1": s1, "s2": s2, "theta": theta})


def make_adam_groups(n: int, seed: int = 5):
    """Per group (name, param, grad, m, v) float32 arrays of n * width elements.

    params ~ N(0, 1), grads ~ N(0, 1e-3), m ~ N(0, 1e-3), v = N(0, 1e-3)^2 (so that v >= 0).
    """
    rng = np.random.default_rng(seed + 1000)
    groups = []
    for name, w in ADAM_GROUP_WIDTHS:
        k = n * w
        p = rng.normal(0.0, 1.0, k).astype(np.float32)
        g = rng.normal(0.0, 1e-3, k).astype(np.float32)
        mm = rng.normal(0.0, 1e-3, k).astype(np.float32)
        vv = (rng.normal(0.0, 1e-3, k) ** 2).astype(np.float32)
        groups.append((name, p, g, mm, vv))
    return groups


# Adam hyper-parameters of the full-iteration workload; step t = 1000.
ADAM_HPARAMS = {"lr": 1.6e-4, "beta1": 0.9, "beta2": 0.999, "eps": 1e-15, "step": 1000}


def adam_bias_corrections(beta1: float, beta2: float, step: int) -> tuple[float, float]:
    """bc1 = 1 - beta1^t and bc2 = 1 - beta2^t in float64, rounded to float32 (host-side scalars of the step)."""
    return float(np.float32(1.0 - np.float64(np.float32(beta1)) ** step)), \
        float(np.float32(1.0 - np.float64(np.float32(beta2)) ** step))


# ---------------------------------------------------------------------------------------------- 3D Gaussians
@dataclass
class GaussianSpec:
    """3D Gaussians in front of a pinhole camera, drawn so that their projected sizes follow `size_classes`
    (log-uniform, pixels) like the 2D workloads. Draw order (default_rng(seed)): depth z, pixel position, size class,
    per-axis log-scale jitter, quaternion, raw opacity, SH coefficients, then the upstream record gradient."""
    name: str
    width: int
    height: int
    n: int
    seed: int
    size_classes: tuple = ((1.0, 0.5, 8.0),)
    aniso_sd: float = 0.3        # log-scale jitter per axis around the class size
    opacity_mu: float = 0.0      # raw opacity ~ N(opacity_mu, opacity_sd)
    opacity_sd: float = 1.0
    depth_lo: float = 2.0
    depth_hi: float = 10.0
    margin: float = 0.0          # pixel positions drawn over [-margin, W + margin) x [-margin, H + margin)
    focal: float = 800.0
    cam_axis: tuple = (0.0, 0.0, 1.0)
    cam_angle: float = 0.0       # camera rotation about cam_axis, radians
    cam_t: tuple = (0.0, 0.0, 0.0)
    dc_sd: float = 1.0           # SH degree-0 coefficients ~ N(0, dc_sd)
    sh_sd: float = 0.1           # higher SH coefficients ~ N(0, sh_sd)
    grad_sd: float = 1e-2        # upstream dL/d(record) ~ N(0, grad_sd)
    near_frac: float = 0.0       # fraction placed behind the near plane (culled)


GAUSS_SPECS = {
    "gauss_tiny": GaussianSpec("gauss_tiny", 64, 48, 300, seed=11, size_classes=((1.0, 0.5, 8.0),), margin=8.0,
                               cam_axis=(0.3, -0.5, 0.8), cam_angle=0.4, cam_t=(0.2, -0.1, 0.5), near_frac=0.05),
    "gauss_ragged": GaussianSpec("gauss_ragged", 100, 37, 1_000, seed=12, size_classes=((0.7, 0.3, 4.0),
                                                                                         (0.3, 4.0, 40.0)),
                                 margin=20.0, cam_axis=(1.0, 0.2, 0.0), cam_angle=-0.3, near_frac=0.02),
    "gauss410k": GaussianSpec("gauss410k", 800, 800, 410_000, seed=13,
                              size_classes=((0.7, 0.3, 4.0), (0.3, 4.0, 40.0)), opacity_mu=-2.0, opacity_sd=1.5),
}


@dataclass
class GaussianScene:
    spec: GaussianSpec
    camera: dict            # R [3, 3], tv [3], fx, fy, cx, cy, near (float64 / float)
    means: np.ndarray       # float32 [N, 3]
    log_scales: np.ndarray  # float32 [N, 3]
    quats: np.ndarray       # float32 [N, 4] (w, x, y, z), not normalised
    raw_opacities: np.ndarray  # float32 [N]
    sh: np.ndarray          # float32 [N, 16, 3]
    splats_grad: np.ndarray  # float32 [N, 9] upstream gradient of the records

    @property
    def width(self):
        return self.spec.width

    @property
    def height(self):
        return self.spec.height


def _axis_angle(axis, angle):
    k = np.asarray(axis, np.float64)
    k = k / np.linalg.norm(k)
    K = np.array([[0, -k[2], k[1]], [k[2], 0, -k[0]], [-k[1], k[0], 0]])
    return np.eye(3) + np.sin(angle) * K + (1 - np.cos(angle)) * (K @ K)


def make_gaussians(spec: GaussianSpec | str, **overrides) -> GaussianScene:
    if isinstance(spec, str):
        spec = GAUSS_SPECS[spec]
    if overrides:
        spec = GaussianSpec(**{**spec.__dict__, **overrides})
    rng = np.random.default_rng(spec.seed)
    n, W, H, f = spec.n, spec.width, spec.height, spec.focal
    R = _axis_angle(spec.cam_axis, spec.cam_angle).astype(np.float32).astype(np.float64)
    tv = np.asarray(spec.cam_t, np.float32).astype(np.float64)
    cam = {"R": R, "tv": tv, "fx": f, "fy": f, "cx": W / 2.0, "cy": H / 2.0, "near": 0.01}
    z = rng.uniform(spec.depth_lo, spec.depth_hi, n)
    m = spec.margin
    px = rng.uniform(-m, W + m, n)
    py = rng.uniform(-m, H + m, n)
    fracs = np.array([c[0] for c in spec.size_classes], np.float64)
    counts = np.floor(fracs / fracs.sum() * n).astype(np.int64)
    counts[0] += n - counts.sum()
    cls = np.repeat(np.arange(len(counts)), counts)[rng.permutation(n)]
    lo = np.log(np.array([c[1] for c in spec.size_classes]))[cls]
    hi = np.log(np.array([c[2] for c in spec.size_classes]))[cls]
    s_px = np.exp(rng.uniform(lo, hi))
    log_scales = np.log(s_px * z / f)[:, None] + rng.normal(0.0, spec.aniso_sd, (n, 3))
    quats = rng.normal(size=(n, 4))
    raw_op = rng.normal(spec.opacity_mu, spec.opacity_sd, n)
    sh = rng.normal(0.0, spec.sh_sd, (n, 16, 3))
    sh[:, 0, :] = rng.normal(0.0, spec.dc_sd, (n, 3))
    grad = rng.normal(0.0, spec.grad_sd, (n, 9))
    # camera coordinates from the pixel position and depth, then world coordinates p = R^T (t - tv)
    t = np.stack([(px - cam["cx"]) * z / f, (py - cam["cy"]) * z / f, z], axis=1)
    k_near = int(round(spec.near_frac * n))
    if k_near:
        behind = rng.choice(n, k_near, replace=False)
        t[behind, 2] = rng.uniform(-1.0, cam["near"], k_near)
    means = (t - tv) @ R
    return GaussianScene(spec, cam, means.astype(np.float32), log_scales.astype(np.float32),
                         quats.astype(np.float32), raw_op.astype(np.float32), sh.astype(np.float32),
                         grad.astype(np.float32))


def make_target(width: int, height: int, seed: int = 21) -> np.ndarray:
    """A target image [H, W, 3] float32 in [0, 1] for the loss: uniform values averaged over a 5 x 5 box (structure at
    a few pixels' scale) mixed 4:1 with fresh uniform noise."""
    rng = np.random.default_rng(seed)
    base = rng.uniform(0.0, 1.0, (height + 4, width + 4, 3))
    c = np.cumsum(np.cumsum(np.pad(base, ((1, 0), (1, 0), (0, 0))), axis=0), axis=1)
    box = (c[5:, 5:] - c[:-5, 5:] - c[5:, :-5] + c[:-5, :-5]) / 25.0
    t = 0.8 * box + 0.2 * rng.uniform(0.0, 1.0, (height, width, 3))
    return np.clip(t, 0.0, 1.0).astype(np.float32)
