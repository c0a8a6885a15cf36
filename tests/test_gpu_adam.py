"""GPU fused Adam against the oracle: bit-exact (both sides evaluate the same IEEE fp32 operations in order)."""
import numpy as np
import pytest

from differentiable_gaussian_splatting_amd import scenes
from gpuhelp import banner, dev, host

pytestmark = pytest.mark.gpu

HP = scenes.ADAM_HPARAMS


@pytest.fixture(scope="module")
def ctx():
    from differentiable_gaussian_splatting_amd import gsr
    c = gsr.Context(0)
    yield c
    c.close()


def check_groups(ctx, groups, lrs, step):
    import oracle
    from differentiable_gaussian_splatting_amd import gsr
    bc1, bc2 = scenes.adam_bias_corrections(HP["beta1"], HP["beta2"], step)
    dev_groups = [(dev(p), dev(g), dev(m), dev(v), lr) for (_, p, g, m, v), lr in zip(groups, lrs)]
    gsr.gsr_adam_step(ctx, dev_groups, HP["beta1"], HP["beta2"], HP["eps"], bc1, bc2)
    for (name, p, g, m, v), (dp, _, dm, dv, _), lr in zip(groups, dev_groups, lrs):
        rp, rm, rv = oracle.adam_step(p, g, m, v, lr, HP["beta1"], HP["beta2"], HP["eps"], bc1, bc2)
        assert np.array_equal(host(dp), rp), f"{name}: param differs"
        assert np.array_equal(host(dm), rm), f"{name}: m differs"
        assert np.array_equal(host(dv), rv), f"{name}: v differs"


def test_adam_full_iteration_shape(ctx):
    banner("adam 410k x 59")
    groups = scenes.make_adam_groups(410_000, seed=5)
    check_groups(ctx, groups, [HP["lr"]] * 5, HP["step"])


@pytest.mark.parametrize("n", [1, 3, 257, 1023, 1025])
def test_adam_odd_sizes_and_per_group_lr(ctx, n):
    banner(f"adam n={n}")
    groups = scenes.make_adam_groups(n, seed=n)
    check_groups(ctx, groups, [1e-3, 2e-4, 5e-5, 1e-2, 1.6e-4], step=3)


def test_adam_unaligned_and_empty_groups(ctx):
    """Arrays that start one element past a 16-byte boundary take the scalar path; empty groups are skipped."""
    import oracle
    from differentiable_gaussian_splatting_amd import gsr
    banner("adam unaligned")
    rng = np.random.default_rng(0)
    base = [rng.normal(0, s, 5001).astype(np.float32) for s in (1.0, 1e-3, 1e-3)]
    base.append((rng.normal(0, 1e-3, 5001) ** 2).astype(np.float32))
    d = [dev(a) for a in base]
    views = [t[1:] for t in d]  # 4-byte offset
    empty = [dev(np.zeros(0, np.float32)) for _ in range(4)]
    bc1, bc2 = scenes.adam_bias_corrections(0.9, 0.999, 10)
    gsr.gsr_adam_step(ctx, [(*empty, 1e-3), (*views, 1e-3), (*empty, 1e-3)], 0.9, 0.999, 1e-15, bc1, bc2)
    rp, rm, rv = oracle.adam_step(base[0][1:], base[1][1:], base[2][1:], base[3][1:], 1e-3, 0.9, 0.999, 1e-15, bc1,
                                  bc2)
    assert np.array_equal(host(d[0])[1:], rp) and np.array_equal(host(d[2])[1:], rm)
    assert np.array_equal(host(d[3])[1:], rv) and host(d[0])[0] == base[0][0]


def test_adam_eight_groups(ctx):
    banner("adam 8 groups")
    groups = []
    for q in range(8):
        groups.extend(scenes.make_adam_groups(100 + 37 * q, seed=q)[:1])
    check_groups(ctx, groups, [1e-4 * (q + 1) for q in range(8)], step=50)


def test_adam_rejects_too_many_groups(ctx):
    from differentiable_gaussian_splatting_amd import gsr
    banner("adam argument errors")
    t = dev(np.zeros(4, np.float32))
    with pytest.raises(ValueError):
        gsr.gsr_adam_step(ctx, [(t, t, t, t, 1e-3)] * 9, 0.9, 0.999, 1e-15, 0.1, 0.001)
    with pytest.raises(gsr.GsrError):
        gsr.gsr_adam_step(ctx, [(t, t, t, t, 1e-3)], 0.9, 0.999, 1e-15, 0.0, 0.001)
