"""Plain CPU oracle of the projection of 3D Gaussians to the rasterizer's 2D splats, and of its backward pass.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline leg may import this module.
The product path (the HIP library and its binding) never imports, links or calls it.

What the pages fix (Gaussian-splatting trainer pages, the M3 per-splat backward page's full-scale parity table and
the forward/Adam audit's Adam byte accounting): five parameter groups per Gaussian - means 3, log_scales 3,
rot_quats 4, raw_opacities 1, sh_coeffs 16 x 3 (sh_degree 3, (d + 1)^2 coefficients per channel), 59 floats - and
that the rasterizer's opacity is the sigmoid of the raw opacity. They print no projection formula; the readings
taken here are the plainest ones of EWA splatting with a pinhole camera:

  t      = R p + tv                          camera coordinates (R, tv: world to camera); culled when t_z <= near
  s      = exp(log_scales), q = quat / |quat| (w, x, y, z), Rq its rotation matrix
  Sigma  = Rq diag(s)^2 Rq^T                 3D covariance
  J      = [[fx / tz, 0, -fx tx / tz^2], [0, fy / tz, -fy ty / tz^2]]   the projection's Jacobian at t
  Sigma' = J R Sigma R^T J^T + 0.3 I        2D covariance in pixels^2, with a 0.3 px^2 low-pass on the diagonal
  conic  = Sigma'^-1 = [[a, b], [b, c]]     so that sigma = 0.5 (a dx^2 + c dy^2) + b dx dy
  mean   = (fx tx / tz + cx, fy ty / tz + cy)
  rgb    = max(sum_k sh[k] Y_k(d) + 0.5, 0) with d = (p - camera centre) / |p - camera centre| and Y_k the real
           spherical harmonics of degrees 0..3 (orthonormal on the sphere, Condon-Shortley signs, in the order
           l = 0; l = 1: m = -1, 0, 1; ...), evaluated on the unit vector
  o      = 1 / (1 + exp(-raw_opacity)),  depth = tz

A culled Gaussian gives the record 0 and depth 0 (the binning then skips it) and zero gradients. The backward pass is
the exact derivative of this forward (fp64 automatic differentiation through the operations below), taking the
gradient of the 9 record values (with b counted once) to the gradients of the 5 parameter groups.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

LOWPASS = 0.3


@dataclass
class Camera:
    """Pinhole camera. R, tv: world to camera (t = R p + tv). (cx, cy) are in the frame of the pixel centres
    (pixel px has its centre at px + 0.5)."""
    R: np.ndarray   # [3, 3]
    tv: np.ndarray  # [3]
    fx: float
    fy: float
    cx: float
    cy: float
    near: float = 0.01

    def centre(self) -> np.ndarray:
        return -np.asarray(self.R, np.float64).T @ np.asarray(self.tv, np.float64)


def sh_constants():
    """Normalisation constants of the real spherical harmonics up to degree 3, from their closed forms."""
    pi = math.pi
    c0 = 1.0 / (2.0 * math.sqrt(pi))
    c1 = math.sqrt(3.0 / (4.0 * pi))
    c2 = (math.sqrt(15.0 / (4.0 * pi)), math.sqrt(15.0 / (4.0 * pi)), math.sqrt(5.0 / (16.0 * pi)),
          math.sqrt(15.0 / (4.0 * pi)), math.sqrt(15.0 / (16.0 * pi)))
    c3 = (math.sqrt(35.0 / (32.0 * pi)), math.sqrt(105.0 / (4.0 * pi)), math.sqrt(21.0 / (32.0 * pi)),
          math.sqrt(7.0 / (16.0 * pi)), math.sqrt(21.0 / (32.0 * pi)), math.sqrt(105.0 / (16.0 * pi)),
          math.sqrt(35.0 / (32.0 * pi)))
    return c0, c1, c2, c3


def sh_basis(d: torch.Tensor) -> torch.Tensor:
    """Y_k(d) for k = 0..15 at unit vectors d [N, 3] -> [N, 16]. Signs: (-1)^m for m > 0 folded into the
    constants (Condon-Shortley), as the real harmonics are usually tabulated."""
    c0, c1, c2, c3 = sh_constants()
    x, y, z = d[:, 0], d[:, 1], d[:, 2]
    xx, yy, zz = x * x, y * y, z * z
    one = torch.ones_like(x)
    cols = [
        c0 * one,
        -c1 * y, c1 * z, -c1 * x,
        c2[0] * x * y, -c2[1] * y * z, c2[2] * (2.0 * zz - xx - yy), -c2[3] * x * z, c2[4] * (xx - yy),
        -c3[0] * y * (3.0 * xx - yy), c3[1] * x * y * z, -c3[2] * y * (4.0 * zz - xx - yy),
        c3[3] * z * (2.0 * zz - 3.0 * xx - 3.0 * yy), -c3[4] * x * (4.0 * zz - xx - yy), c3[5] * z * (xx - yy),
        -c3[6] * x * (xx - 3.0 * yy),
    ]
    return torch.stack(cols, dim=1)


def quat_to_rotmat(q: torch.Tensor) -> torch.Tensor:
    """Rotation matrices [N, 3, 3] of unit quaternions q [N, 4] = (w, x, y, z)."""
    w, x, y, z = q[:, 0], q[:, 1], q[:, 2], q[:, 3]
    r = torch.stack([
        1 - 2 * (y * y + z * z), 2 * (x * y - w * z), 2 * (x * z + w * y),
        2 * (x * y + w * z), 1 - 2 * (x * x + z * z), 2 * (y * z - w * x),
        2 * (x * z - w * y), 2 * (y * z + w * x), 1 - 2 * (x * x + y * y),
    ], dim=1)
    return r.reshape(-1, 3, 3)


def _forward(cam: Camera, means, log_scales, quats, raw_op, sh, clamp_flip=None):
    """Torch fp64 forward; returns (splats [N, 9], depths [N]). clamp_flip: optional bool [N, 3]; where set, the
    colour channel takes the other side of its clamp decision (kept when the unclamped value is <= 0, clamped to 0
    when it is > 0), the reading a floating-point evaluation may take when that value lies within its rounding of 0."""
    R = torch.as_tensor(np.asarray(cam.R, np.float64))
    tv = torch.as_tensor(np.asarray(cam.tv, np.float64))
    t = means @ R.T + tv
    valid = t[:, 2] > cam.near
    one = torch.ones_like(t[:, 2])
    tz = torch.where(valid, t[:, 2], one)  # culled rows take a harmless stand-in; their outputs are zeroed below
    tx, ty = t[:, 0], t[:, 1]
    s = torch.exp(log_scales)
    qn = quats / torch.linalg.norm(quats, dim=1, keepdim=True)
    M = quat_to_rotmat(qn) * s[:, None, :]  # Rq diag(s)
    zero = torch.zeros_like(tz)
    J = torch.stack([torch.stack([cam.fx / tz, zero, -cam.fx * tx / (tz * tz)], 1),
                     torch.stack([zero, cam.fy / tz, -cam.fy * ty / (tz * tz)], 1)], 1)  # [N, 2, 3]
    T = J @ R @ M  # [N, 2, 3]
    S2 = T @ T.transpose(1, 2)
    sxx = S2[:, 0, 0] + LOWPASS
    sxy = S2[:, 0, 1]
    syy = S2[:, 1, 1] + LOWPASS
    det = sxx * syy - sxy * sxy
    a, b, c = syy / det, -sxy / det, sxx / det
    mx = cam.fx * tx / tz + cam.cx
    my = cam.fy * ty / tz + cam.cy
    centre = torch.as_tensor(cam.centre())
    v = means - centre
    d = v / torch.linalg.norm(v, dim=1, keepdim=True)
    Y = sh_basis(d)  # [N, 16]
    raw_rgb = torch.einsum("nk,nkc->nc", Y, sh.reshape(-1, 16, 3)) + 0.5
    lit = raw_rgb > 0
    if clamp_flip is not None:
        lit = lit ^ torch.as_tensor(np.asarray(clamp_flip, bool).reshape(-1, 3))
    rgb = torch.where(lit, raw_rgb, torch.zeros_like(raw_rgb))
    o = 1.0 / (1.0 + torch.exp(-raw_op))
    rec = torch.stack([mx, my, a, b, c, rgb[:, 0], rgb[:, 1], rgb[:, 2], o], 1)
    rec = torch.where(valid[:, None], rec, torch.zeros_like(rec))
    depth = torch.where(valid, t[:, 2], zero)
    return rec, depth


def _params64(means, log_scales, quats, raw_opacities, sh, grad=False):
    ts = [torch.as_tensor(np.asarray(a, np.float64)).clone() for a in (means, log_scales, quats, raw_opacities, sh)]
    ts[0] = ts[0].reshape(-1, 3)
    ts[1] = ts[1].reshape(-1, 3)
    ts[2] = ts[2].reshape(-1, 4)
    ts[3] = ts[3].reshape(-1)
    ts[4] = ts[4].reshape(-1, 48)
    if grad:
        for x in ts:
            x.requires_grad_(True)
    return ts


def project_forward(cam: Camera, means, log_scales, quats, raw_opacities, sh):
    """Splats [N, 9] and depths [N] (float64) of the Gaussians (any float arrays; means [N, 3], log_scales [N, 3],
    quats [N, 4], raw_opacities [N], sh [N, 48] as [N, 16, 3] coefficient-major)."""
    with torch.no_grad():
        rec, depth = _forward(cam, *_params64(means, log_scales, quats, raw_opacities, sh))
    return rec.numpy(), depth.numpy()


def unclamped_colour(cam: Camera, means, sh) -> np.ndarray:
    """sum_k sh[k] Y_k(d) + 0.5 per channel [N, 3] (float64): the colour before its clamp at 0."""
    with torch.no_grad():
        m = torch.as_tensor(np.asarray(means, np.float64).reshape(-1, 3))
        v = m - torch.as_tensor(cam.centre())
        d = v / torch.linalg.norm(v, dim=1, keepdim=True)
        shc = torch.as_tensor(np.asarray(sh, np.float64).reshape(-1, 16, 3))
        return (torch.einsum("nk,nkc->nc", sh_basis(d), shc) + 0.5).numpy()


def project_backward(cam: Camera, means, log_scales, quats, raw_opacities, sh, splats_grad, clamp_flip=None):
    """Gradients (float64) of the five parameter groups given dL/d(record) [N, 9]: the derivative of
    sum(splats_grad * record) through project_forward. clamp_flip as in _forward: the derivative with those colour
    channels' clamp decisions taken the other way."""
    ps = _params64(means, log_scales, quats, raw_opacities, sh, grad=True)
    rec, _ = _forward(cam, *ps, clamp_flip=clamp_flip)
    g = torch.as_tensor(np.asarray(splats_grad, np.float64).reshape(-1, 9))
    grads = torch.autograd.grad((rec * g).sum(), ps, allow_unused=True)
    out = []
    for p, gr in zip(ps, grads):
        out.append(np.zeros(tuple(p.shape)) if gr is None else gr.numpy())
    return tuple(out)
