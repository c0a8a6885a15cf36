"""Pins of the projection oracle (oracle/project.py) against facts that do not depend on it: orthonormality of the
spherical-harmonic basis by quadrature, closed forms of the pinhole projection of axis-aligned and rotated Gaussians,
invariance under a rigid motion of the scene together with the camera, and central finite differences of the
backward pass."""
import math

import numpy as np

from oracle import project as op


def cam_identity(fx=500.0, fy=450.0, cx=400.0, cy=300.0):
    return op.Camera(R=np.eye(3), tv=np.zeros(3), fx=fx, fy=fy, cx=cx, cy=cy)


def one(means, log_scales, quats, raw_op, sh):
    return (np.asarray(means, float).reshape(-1, 3), np.asarray(log_scales, float).reshape(-1, 3),
            np.asarray(quats, float).reshape(-1, 4), np.asarray(raw_op, float).reshape(-1),
            np.asarray(sh, float).reshape(-1, 48))


def test_sh_basis_is_orthonormal_on_the_sphere():
    """Gauss-Legendre in cos(theta) times a uniform grid in phi integrates products of degree <= 6 exactly."""
    import torch
    ct, wt = np.polynomial.legendre.leggauss(12)
    nphi = 16
    phi = 2 * math.pi * np.arange(nphi) / nphi
    C, P = np.meshgrid(ct, phi, indexing="ij")
    S = np.sqrt(1 - C * C)
    d = np.stack([S * np.cos(P), S * np.sin(P), C], -1).reshape(-1, 3)
    w = (wt[:, None] * np.full(nphi, 2 * math.pi / nphi)[None, :]).reshape(-1)
    Y = op.sh_basis(torch.as_tensor(d)).numpy()
    gram = (Y * w[:, None]).T @ Y
    assert np.abs(gram - np.eye(16)).max() < 1e-12


def test_sh_basis_bands_by_degree():
    """Each band l spans the harmonic polynomials of degree l: Y_k(-d) = (-1)^l Y_k(d)."""
    import torch
    rng = np.random.default_rng(1)
    d = rng.normal(size=(50, 3))
    d /= np.linalg.norm(d, axis=1, keepdims=True)
    Yp = op.sh_basis(torch.as_tensor(d)).numpy()
    Ym = op.sh_basis(torch.as_tensor(-d)).numpy()
    parity = np.array([1] + [-1] * 3 + [1] * 5 + [-1] * 7, float)
    assert np.allclose(Ym, Yp * parity, atol=1e-14)


def test_degree0_colour_is_view_independent():
    c0 = 1.0 / (2.0 * math.sqrt(math.pi))
    cam = cam_identity()
    n = 5
    rng = np.random.default_rng(2)
    means = np.column_stack([rng.uniform(-1, 1, n), rng.uniform(-1, 1, n), rng.uniform(3, 6, n)])
    sh = np.zeros((n, 16, 3))
    sh[:, 0, :] = rng.normal(size=(n, 3))
    rec, _ = op.project_forward(cam, *one(means, np.zeros((n, 3)), np.tile([1, 0, 0, 0], (n, 1)), np.zeros(n), sh))
    assert np.allclose(rec[:, 5:8], np.maximum(c0 * sh[:, 0, :] + 0.5, 0.0), atol=1e-15)


def test_axis_aligned_gaussian_closed_form():
    cam = cam_identity()
    z, sx, sy, sz, rho = 4.0, 0.05, 0.02, 0.3, -0.7
    rec, depth = op.project_forward(cam, *one([0, 0, z], np.log([sx, sy, sz]), [1, 0, 0, 0], [rho], np.zeros(48)))
    vx = (cam.fx * sx / z) ** 2 + 0.3
    vy = (cam.fy * sy / z) ** 2 + 0.3
    want = [cam.cx, cam.cy, 1 / vx, 0.0, 1 / vy, 0.5, 0.5, 0.5, 1 / (1 + math.exp(-rho))]
    assert np.allclose(rec[0], want, rtol=1e-13, atol=1e-15)
    assert depth[0] == z


def test_rotation_about_the_view_axis_swaps_the_axes():
    cam = cam_identity()
    z, sx, sy = 5.0, 0.07, 0.01
    h = math.sqrt(0.5)
    rec, _ = op.project_forward(cam, *one([0, 0, z], np.log([sx, sy, 0.2]), [h, 0, 0, h], [0.0], np.zeros(48)))
    vx = (cam.fx * sy / z) ** 2 + 0.3
    vy = (cam.fy * sx / z) ** 2 + 0.3
    assert np.allclose(rec[0, 2:5], [1 / vx, 0.0, 1 / vy], rtol=1e-12, atol=1e-15)


def test_off_axis_mean_and_camera_translation():
    cam = op.Camera(R=np.eye(3), tv=np.array([0.5, -0.25, 1.0]), fx=300.0, fy=320.0, cx=10.0, cy=20.0)
    p = np.array([0.3, 0.4, 2.0])
    rec, depth = op.project_forward(cam, *one(p, np.log([0.1] * 3), [1, 0, 0, 0], [0.0], np.zeros(48)))
    t = p + cam.tv
    assert np.allclose(rec[0, :2], [cam.fx * t[0] / t[2] + cam.cx, cam.fy * t[1] / t[2] + cam.cy], rtol=1e-14)
    assert depth[0] == t[2]


def test_quaternion_scale_does_not_matter():
    rng = np.random.default_rng(3)
    n = 6
    means = np.column_stack([rng.uniform(-1, 1, n), rng.uniform(-1, 1, n), rng.uniform(2, 5, n)])
    ls, q, rho, sh = rng.normal(-2, 0.5, (n, 3)), rng.normal(size=(n, 4)), rng.normal(size=n), rng.normal(0, .3, (n, 48))
    cam = cam_identity()
    a, _ = op.project_forward(cam, *one(means, ls, q, rho, sh))
    b, _ = op.project_forward(cam, *one(means, ls, 3.7 * q, rho, sh))
    assert np.allclose(a, b, rtol=1e-12, atol=1e-14)


def rot_from_quat(q):
    w, x, y, z = q / np.linalg.norm(q)
    return np.array([[1 - 2 * (y * y + z * z), 2 * (x * y - w * z), 2 * (x * z + w * y)],
                     [2 * (x * y + w * z), 1 - 2 * (x * x + z * z), 2 * (y * z - w * x)],
                     [2 * (x * z - w * y), 2 * (y * z + w * x), 1 - 2 * (x * x + y * y)]])


def quat_mul(a, b):
    w1, x1, y1, z1 = a
    w2, x2, y2, z2 = b
    return np.array([w1 * w2 - x1 * x2 - y1 * y2 - z1 * z2, w1 * x2 + x1 * w2 + y1 * z2 - z1 * y2,
                     w1 * y2 - x1 * z2 + y1 * w2 + z1 * x2, w1 * z2 + x1 * y2 - y1 * x2 + z1 * w2])


def test_rigid_motion_of_scene_and_camera_changes_nothing():
    """Moving every Gaussian by p -> Q p + u, turning each by Q (quaternion product), and moving the camera with them
    (R' = R Q^T, tv' = tv - R Q^T u) leaves the geometry of every record unchanged. The colours change unless the SH
    coefficients rotate too, so they are set to degree 0 here."""
    rng = np.random.default_rng(4)
    n = 8
    cam = op.Camera(R=rot_from_quat(np.array([0.9, 0.1, -0.2, 0.3])), tv=np.array([0.1, 0.2, 4.0]), fx=400.0,
                    fy=420.0, cx=300.0, cy=200.0)
    means = rng.normal(0, 0.6, (n, 3))
    ls, q, rho = rng.normal(-2, 0.4, (n, 3)), rng.normal(size=(n, 4)), rng.normal(size=n)
    sh = np.zeros((n, 48))
    sh[:, :3] = rng.normal(size=(n, 3))
    qq = np.array([0.7, -0.3, 0.5, 0.2])
    qq /= np.linalg.norm(qq)
    Q, u = rot_from_quat(qq), np.array([1.0, -2.0, 0.5])
    cam2 = op.Camera(R=cam.R @ Q.T, tv=cam.tv - cam.R @ Q.T @ u, fx=cam.fx, fy=cam.fy, cx=cam.cx, cy=cam.cy)
    q2 = np.array([quat_mul(qq, qi) for qi in q])
    a, da = op.project_forward(cam, *one(means, ls, q, rho, sh))
    b, db = op.project_forward(cam2, *one(means @ Q.T + u, ls, q2, rho, sh))
    assert (da > cam.near).all()
    assert np.allclose(a, b, rtol=1e-10, atol=1e-12)
    assert np.allclose(da, db, rtol=1e-12)


def test_culled_gaussians_give_zero_records_and_gradients():
    cam = cam_identity()
    means = np.array([[0, 0, 0.005], [0, 0, -1.0], [0.1, 0, 3.0]])
    n = 3
    args = one(means, np.full((n, 3), -2.0), np.tile([1, 0, 0, 0], (n, 1)), np.zeros(n), np.full((n, 48), 0.1))
    rec, depth = op.project_forward(cam, *args)
    assert (rec[:2] == 0).all() and (depth[:2] == 0).all() and depth[2] == 3.0 and rec[2, 8] == 0.5
    grads = op.project_backward(cam, *args, np.ones((n, 9)))
    for g in grads:
        assert (g.reshape(n, -1)[:2] == 0).all()
        assert np.isfinite(g).all()


def test_backward_matches_central_differences():
    rng = np.random.default_rng(5)
    n = 4
    cam = op.Camera(R=rot_from_quat(np.array([0.95, 0.05, 0.2, -0.1])), tv=np.array([0.2, -0.1, 3.0]), fx=350.0,
                    fy=330.0, cx=200.0, cy=180.0)
    params = [rng.normal(0, 0.5, (n, 3)), rng.normal(-2, 0.3, (n, 3)), rng.normal(size=(n, 4)), rng.normal(size=n),
              rng.normal(0, 0.3, (n, 48))]
    w = rng.normal(size=(n, 9))
    grads = op.project_backward(cam, *params, w)

    def loss(ps):
        rec, _ = op.project_forward(cam, *ps)
        return float((rec * w).sum())

    h = 1e-6
    for gi, p in enumerate(params):
        flat = p.reshape(-1)
        for j in range(flat.size):
            up = [x.copy() for x in params]
            dn = [x.copy() for x in params]
            up[gi].reshape(-1)[j] += h
            dn[gi].reshape(-1)[j] -= h
            fd = (loss(up) - loss(dn)) / (2 * h)
            an = grads[gi].reshape(-1)[j]
            assert abs(fd - an) <= 1e-5 * (1 + abs(an)), (gi, j, fd, an)


def test_backward_closed_forms():
    """dL/draw_opacity = g_o o (1 - o); dL/dsh[0][c] = g_c / (2 sqrt(pi)) where the colour is not clamped, else 0."""
    rng = np.random.default_rng(6)
    n = 10
    cam = cam_identity()
    means = np.column_stack([rng.uniform(-1, 1, n), rng.uniform(-1, 1, n), rng.uniform(2, 5, n)])
    sh = rng.normal(0, 1.0, (n, 48))
    rho = rng.normal(size=n)
    args = one(means, rng.normal(-2, 0.3, (n, 3)), rng.normal(size=(n, 4)), rho, sh)
    g = rng.normal(size=(n, 9))
    grads = op.project_backward(cam, *args, g)
    o = 1 / (1 + np.exp(-rho))
    assert np.allclose(grads[3], g[:, 8] * o * (1 - o), rtol=1e-13)
    rec, _ = op.project_forward(cam, *args)
    lit = rec[:, 5:8] > 0
    assert (~lit).any() and lit.any()
    want = np.where(lit, g[:, 5:8] / (2 * math.sqrt(math.pi)), 0.0)
    assert np.allclose(grads[4].reshape(n, 16, 3)[:, 0, :], want, rtol=1e-13, atol=1e-15)


def test_flipped_clamp_decisions():
    """clamp_flip takes a channel's clamp decision the other way: a lit channel becomes 0 with no SH gradient, a
    clamped one takes its unclamped value, and its DC gradient is then g_c / (2 sqrt(pi)); unflagged channels and
    the other groups' gradients from the colour are unchanged. The unclamped colour equals the record where lit."""
    rng = np.random.default_rng(16)
    n = 12
    cam = cam_identity()
    means = np.column_stack([rng.uniform(-1, 1, n), rng.uniform(-1, 1, n), rng.uniform(2, 5, n)])
    sh = rng.normal(0, 1.0, (n, 48))
    args = one(means, rng.normal(-2, 0.3, (n, 3)), rng.normal(size=(n, 4)), rng.normal(size=n), sh)
    g = rng.normal(size=(n, 9))
    rec, _ = op.project_forward(cam, *args)
    raw = op.unclamped_colour(cam, means, sh)
    lit = raw > 0
    assert lit.any() and (~lit).any()
    assert np.allclose(rec[:, 5:8], np.where(lit, raw, 0.0), rtol=1e-13, atol=1e-15)
    flip = np.zeros((n, 3), bool)
    flip[::2, 0] = True
    flip[1::3, 2] = True
    base = op.project_backward(cam, *args, g)
    fl = op.project_backward(cam, *args, g, clamp_flip=flip)
    lit_f = lit ^ flip
    dc = 1 / (2 * math.sqrt(math.pi))
    assert np.allclose(fl[4].reshape(n, 16, 3)[:, 0, :], np.where(lit_f, g[:, 5:8] * dc, 0.0), rtol=1e-13, atol=1e-15)
    same = ~flip.any(axis=1)
    for a, b in zip(base, fl):
        assert np.array_equal(a.reshape(n, -1)[same], b.reshape(n, -1)[same])
    for k in (1, 2, 3):  # log_scales, quats, raw opacity: the colour does not reach them
        assert np.array_equal(base[k], fl[k])


def test_covariance_uses_the_derivative_of_the_mean_projection():
    """EWA: Sigma' = J Sigma_cam J^T + 0.3 I with J the derivative of the pixel mean with respect to the camera-space
    position. J is taken here by central differences of the oracle's own projected means, so the closed form below
    shares nothing with the oracle's Jacobian."""
    rng = np.random.default_rng(7)
    cam = op.Camera(R=rot_from_quat(np.array([0.8, -0.2, 0.3, 0.1])), tv=np.array([-0.3, 0.4, 3.5]), fx=610.0,
                    fy=580.0, cx=320.0, cy=240.0)
    for _ in range(4):
        p = rng.normal(0, 0.8, 3)
        ls, q = rng.normal(-2.5, 0.5, 3), rng.normal(size=4)
        rec, _ = op.project_forward(cam, *one(p, ls, q, [0.0], np.zeros(48)))
        h = 1e-6
        Jw = np.zeros((2, 3))
        for k in range(3):
            e = np.zeros(3)
            e[k] = h
            up, _ = op.project_forward(cam, *one(p + e, ls, q, [0.0], np.zeros(48)))
            dn, _ = op.project_forward(cam, *one(p - e, ls, q, [0.0], np.zeros(48)))
            Jw[:, k] = (up[0, :2] - dn[0, :2]) / (2 * h)  # d(mean)/d(world position)
        Rq = rot_from_quat(q)
        Sigma = Rq @ np.diag(np.exp(2 * ls)) @ Rq.T
        S2 = Jw @ Sigma @ Jw.T + 0.3 * np.eye(2)
        conic = np.linalg.inv(S2)
        assert np.allclose(rec[0, 2:5], [conic[0, 0], conic[0, 1], conic[1, 1]], rtol=1e-6, atol=1e-9)


def test_colour_direction_is_from_the_camera_centre():
    """Degree-1 colour at a camera away from the origin: rgb = 0.5 + C1 (-y s1 + z s2 - x s3), (x, y, z) the unit
    vector from the camera centre to the mean, C1 = sqrt(3 / (4 pi))."""
    cam = op.Camera(R=np.eye(3), tv=np.array([0.5, -0.25, 1.0]), fx=300.0, fy=320.0, cx=10.0, cy=20.0)
    rng = np.random.default_rng(8)
    c1 = math.sqrt(3.0 / (4.0 * math.pi))
    for _ in range(3):
        p = np.array([rng.uniform(-1, 1), rng.uniform(-1, 1), rng.uniform(1, 3)])
        sh = np.zeros((16, 3))
        sh[1:4] = rng.normal(0, 0.2, (3, 3))
        rec, _ = op.project_forward(cam, *one(p, np.log([0.1] * 3), [1, 0, 0, 0], [0.0], sh))
        v = p - (-cam.tv)
        x, y, z = v / np.linalg.norm(v)
        want = 0.5 + c1 * (-y * sh[1] + z * sh[2] - x * sh[3])
        assert np.allclose(rec[0, 5:8], np.maximum(want, 0), rtol=1e-13, atol=1e-15)
