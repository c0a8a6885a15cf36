"""The timed step of bench.py on its own workload (iter410k: 800 x 800, 410,000 splats), in the launch
configuration bench.py times (default options, the arena reserved, the tile order taken from the previous
forward), against the oracle: bins bit-exact, the image and final T within 1e-5 and last_contrib exact, the
9 splat gradients within 1e-4 + 1e-4 |oracle|, and one fused Adam step over the 59 floats per splat bit-exact.
Every output element is compared."""
import numpy as np
import pytest

from gpuhelp import banner, grads_close, host

pytestmark = pytest.mark.gpu


def test_bench_step_matches_oracle():
    import torch

    import oracle
    from differentiable_gaussian_splatting_amd import gsr, scenes
    banner("bench step iter410k")
    sc = scenes.make_scene("iter410k")
    W, H, N = sc.width, sc.height, sc.spec.n
    hp = scenes.ADAM_HPARAMS
    bc = scenes.adam_bias_corrections(hp["beta1"], hp["beta2"], hp["step"])
    adam_host = scenes.make_adam_groups(N, seed=sc.spec.seed)
    ctx = gsr.Context(0)
    try:
        splats = torch.from_numpy(sc.splats).cuda()
        depths = torch.from_numpy(sc.depths).cuda()
        v_out = torch.from_numpy(sc.v_out).cuda()
        out = torch.empty((H, W, 4), dtype=torch.float32, device="cuda")
        ft = torch.empty((H, W), dtype=torch.float32, device="cuda")
        lc = torch.empty((H, W), dtype=torch.int32, device="cuda")
        grad = torch.empty((N, 9), dtype=torch.float32, device="cuda")
        b = gsr.gsr_bin(ctx, splats, depths, W, H)
        gsr.gsr_reserve(ctx, int(b.num_pairs * 1.05) + 1024, N)
        for _ in range(2):  # as the bench's warmup: the later launches take the tile order of a previous forward
            b = gsr.gsr_bin(ctx, splats, depths, W, H)
            gsr.gsr_render_forward(ctx, splats, b, W, H, out, ft, lc)
            gsr.gsr_render_backward(ctx, splats, b, W, H, out, ft, lc, v_out, grad)
        groups = [tuple(torch.from_numpy(a).cuda() for a in g[1:]) + (hp["lr"],) for g in adam_host]
        gsr.gsr_adam_step(ctx, groups, hp["beta1"], hp["beta2"], hp["eps"], *bc)
        keys, vals, ranges = (host(t) for t in gsr.gsr_bins_copy(ctx, b))
        out_h, ft_h, lc_h, grad_h = host(out), host(ft), host(lc, np.uint32), host(grad)
        groups_h = [tuple(host(t) for t in g[:4]) for g in groups]
    finally:
        ctx.close()

    ob = oracle.bin(sc.splats, sc.depths, W, H)
    assert np.array_equal(keys.view(np.uint64), ob.keys) and np.array_equal(vals.view(np.uint32), ob.vals)
    assert np.array_equal(ranges.view(np.uint32), ob.ranges)
    r_out, r_ft, r_lc, _ = oracle.render_forward(sc.splats, ob, W, H)
    assert np.array_equal(lc_h, r_lc)
    assert np.abs(out_h - r_out).max() <= 1e-5 and np.abs(ft_h - r_ft).max() <= 1e-5
    r_grad = oracle.render_backward(sc.splats, ob, W, H, r_out, r_ft, r_lc, sc.v_out)
    ok, worst, at = grads_close(grad_h, r_grad)
    print(f"  pairs {ob.num_pairs}; gradients worst |gpu-ref| / (1e-4 + 1e-4 |ref|) = {worst:.3g} at {at}")
    assert ok, (worst, at)
    for (name, p, g, m, v), (dp, _, dm, dv) in zip(adam_host, groups_h):
        rp, rm, rv = oracle.adam_step(p, g, m, v, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], *bc)
        assert np.array_equal(dp, rp) and np.array_equal(dm, rm) and np.array_equal(dv, rv), name
