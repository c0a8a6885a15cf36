"""A whole step recorded once as a HIP graph and replayed. With GSR_OPT_BIN_SYNC_FREE, gsr_bin queues its launches
without waiting for the pair count, and with the arena reserved no call allocates, so bin + forward + backward +
Adam can be captured on a stream. Between the replays, eager work overwrites the outputs and the arena's bins, and
the program synchronises. Every replay must reproduce the eager step: the bins' first count pairs and ranges, the
image, final T and last_contrib byte for byte, the gradients within the parity bar (their float atomics add in any
order), and the Adam state bit for bit."""
import numpy as np
import pytest

from gpuhelp import banner, grads_close, host, scene

pytestmark = pytest.mark.gpu


def test_step_replays_as_a_graph():
    import torch

    from differentiable_gaussian_splatting_amd import gsr, scenes
    banner("graph-captured step raster84k")
    sc = scene("raster84k")
    W, H, N = sc.width, sc.height, sc.spec.n
    hp = scenes.ADAM_HPARAMS
    bc = scenes.adam_bias_corrections(hp["beta1"], hp["beta2"], hp["step"])
    adam_host = scenes.make_adam_groups(N, seed=sc.spec.seed)
    ctx = gsr.Context(0)
    try:
        gsr.gsr_set_option(ctx, gsr.GSR_OPT_BIN_SYNC_FREE, 1)
        splats = torch.from_numpy(sc.splats).cuda()
        depths = torch.from_numpy(sc.depths).cuda()
        v_out = torch.from_numpy(sc.v_out).cuda()
        out = torch.empty((H, W, 4), dtype=torch.float32, device="cuda")
        ft = torch.empty((H, W), dtype=torch.float32, device="cuda")
        lc = torch.empty((H, W), dtype=torch.int32, device="cuda")
        grad = torch.empty((N, 9), dtype=torch.float32, device="cuda")
        init = [tuple(torch.from_numpy(a).cuda() for a in g[1:]) for g in adam_host]  # (param, grad, m, v)
        work = [tuple(t.clone() for t in g) for g in init]
        groups = [w + (hp["lr"],) for w in work]

        def reset():
            for w, i in zip(work, init):
                for a, b in zip(w, i):
                    a.copy_(b)

        def step():
            b = gsr.gsr_bin(ctx, splats, depths, W, H)
            gsr.gsr_render_forward(ctx, splats, b, W, H, out, ft, lc)
            gsr.gsr_render_backward(ctx, splats, b, W, H, out, ft, lc, v_out, grad)
            gsr.gsr_adam_step(ctx, groups, hp["beta1"], hp["beta2"], hp["eps"], *bc)
            return b

        def snapshot(b, P):
            keys, vals, ranges = gsr.gsr_bins_copy(ctx, b)
            return {"keys": host(keys, np.uint64)[:P], "vals": host(vals, np.uint32)[:P],
                    "ranges": host(ranges, np.uint32), "out": host(out), "ft": host(ft),
                    "lc": host(lc, np.uint32), "grad": host(grad),
                    "adam": [host(t) for w in work for t in (w[0], w[2], w[3])]}

        gsr.gsr_bin(ctx, splats, depths, W, H)  # no count seen yet: this call waits once
        P, over = gsr.gsr_bin_pair_count(ctx)
        assert not over
        gsr.gsr_reserve(ctx, 2 * P, N)  # the capacity comes from the reservation: nothing grows below
        for _ in range(2):  # eager steps grow every buffer the step uses
            reset()
            step()
        reset()
        b = step()
        torch.cuda.synchronize()
        assert gsr.gsr_bin_pair_count(ctx) == (P, False)
        ref = snapshot(b, P)

        reset()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, capture_error_mode="relaxed"):
            bg = step()
        torch.cuda.synchronize()
        assert bg.num_pairs == b.num_pairs  # the same capacity, so the same buffers
        small = scene("tiny")
        sp_small, d_small = torch.from_numpy(small.splats).cuda(), torch.from_numpy(small.depths).cuda()
        for r in range(3):
            # eager work between the replays that overwrites what the graph must rebuild: the outputs, and the
            # arena's ranges and values (a smaller scene: within the reserved sizes, so nothing moves)
            reset()
            for t in (out, ft, grad):
                t.fill_(float("nan"))
            lc.fill_(-1)
            gsr.gsr_bin(ctx, sp_small, d_small, small.width, small.height)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = snapshot(bg, P)
            for k in ("keys", "vals", "ranges", "out", "ft", "lc"):
                assert np.array_equal(got[k], ref[k]), (r, k)
            ok, worst, at = grads_close(got["grad"], ref["grad"])
            assert ok, (r, worst, at)
            for q, (x, y) in enumerate(zip(got["adam"], ref["adam"])):
                assert np.array_equal(x, y), (r, q)
        del graph
    finally:
        ctx.close()
