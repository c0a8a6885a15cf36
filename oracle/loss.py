"""Plain CPU oracle of the training loss that produces the rasterizer's upstream gradient: L1 + SSIM.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline leg may import this module.
The product path (the HIP library and its binding) never imports, links or calls it.

The pages name the loss of the trainer they profile (a fused L1 + SSIM loss and its backward, the SSIM kernel's
share of the iteration, its window sizes K = 7 and K = 11 in the SSIM float4 finding) but print no formula. The
reading taken here is the usual one for Gaussian splatting:

  L = (1 - lam) mean|x - y| + lam (1 - mean S),   lam = 0.2, means over all pixels and the 3 channels
  S = ((2 mx my + C1)(2 sxy + C2)) / ((mx^2 + my^2 + C1)(sx + sy + C2)),  C1 = 0.01^2, C2 = 0.03^2
  mx = G * x, sx = G * x^2 - mx^2, sxy = G * (x y) - mx my (and likewise for y), per channel, where G * is the
  correlation with the normalised 2D Gaussian window of size K = 11 and standard deviation 1.5 (the outer product of
  its normalised 1D taps), over the image padded with zeros ("same" size).

x is the rendered image (the rgb of out_rgba), y the target. The gradient of L with respect to x is the exact
derivative of this definition (fp64 automatic differentiation; the L1 term's derivative is sign(x - y), 0 where
x = y).
"""
from __future__ import annotations

import math

import numpy as np
import torch

LAMBDA = 0.2
C1 = 0.01 ** 2
C2 = 0.03 ** 2
WINDOW = 11
SIGMA = 1.5


def gaussian_taps(k: int = WINDOW, sigma: float = SIGMA) -> np.ndarray:
    """Normalised 1D Gaussian taps, centred, length k."""
    c = k // 2
    g = np.array([math.exp(-((i - c) ** 2) / (2.0 * sigma * sigma)) for i in range(k)])
    return g / g.sum()


def _window2d(k, sigma):
    g = torch.as_tensor(gaussian_taps(k, sigma))
    return torch.outer(g, g)


def _filter(img, w2):
    """Per-channel 2D correlation with zero padding: img [C, H, W] -> [C, H, W]."""
    C = img.shape[0]
    k = w2.shape[0]
    weight = w2.expand(C, 1, k, k).contiguous()
    return torch.nn.functional.conv2d(img[None], weight, padding=k // 2, groups=C)[0]


def _ssim(x, y, k, sigma):
    """SSIM map [C, H, W] of images [C, H, W]."""
    w2 = _window2d(k, sigma).to(x.dtype)
    mx, my = _filter(x, w2), _filter(y, w2)
    sx = _filter(x * x, w2) - mx * mx
    sy = _filter(y * y, w2) - my * my
    sxy = _filter(x * y, w2) - mx * my
    return ((2 * mx * my + C1) * (2 * sxy + C2)) / ((mx * mx + my * my + C1) * (sx + sy + C2))


def _loss(x, y, k, sigma, lam):
    S = _ssim(x, y, k, sigma)
    l1 = (x - y).abs().mean()
    return (1 - lam) * l1 + lam * (1 - S.mean()), l1, S.mean()


def ssim_map(out_rgba, target, k: int = WINDOW, sigma: float = SIGMA) -> np.ndarray:
    """The SSIM map S [3, H, W] (float64)."""
    with torch.no_grad():
        return _ssim(_chw(out_rgba), _chw(target), k, sigma).numpy()


def _chw(img):
    a = np.asarray(img, np.float64)
    return torch.as_tensor(np.ascontiguousarray(a[..., :3].transpose(2, 0, 1)))


def l1_ssim(out_rgba, target, k: int = WINDOW, sigma: float = SIGMA, lam: float = LAMBDA):
    """(loss, l1, mean ssim) in float64 for out_rgba [H, W, >= 3] (its first three channels) and target [H, W, 3]."""
    with torch.no_grad():
        L, l1, s = _loss(_chw(out_rgba), _chw(target), k, sigma, lam)
    return float(L), float(l1), float(s)


def l1_ssim_backward(out_rgba, target, k: int = WINDOW, sigma: float = SIGMA, lam: float = LAMBDA):
    """dL/d(out_rgba) as [H, W, 4] float64 (the 4th channel 0) and the loss."""
    x = _chw(out_rgba).requires_grad_(True)
    L, _, _ = _loss(x, _chw(target), k, sigma, lam)
    (g,) = torch.autograd.grad(L, x)
    H, W = g.shape[1], g.shape[2]
    out = np.zeros((H, W, 4))
    out[..., :3] = g.numpy().transpose(1, 2, 0)
    return out, float(L.detach())
