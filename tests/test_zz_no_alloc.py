"""gsr_render_forward_noalloc (the forward for callers that cannot allocate) against gsr_render_forward: the same
kernels on the same bins, so every output must be the same bits. Two calls in a row, the second on a smaller image
(fewer tiles), so the second runs on the scratch the first left behind; a call beyond the scratch's tile limit is
refused before anything is queued."""
import ctypes

import numpy as np
import pytest

from gpuhelp import banner, dev, host, scene

pytestmark = pytest.mark.gpu


def render_both(ctx, name):
    import torch
    from differentiable_gaussian_splatting_amd import gsr
    sc = scene(name)
    W, H = sc.width, sc.height
    sp = dev(sc.splats)
    bins = gsr.gsr_bin(ctx, sp, dev(sc.depths), W, H)
    ref = gsr.gsr_render_forward(ctx, sp, bins, W, H)
    out = (torch.full((H, W, 4), float("nan"), device="cuda"), torch.full((H, W), float("nan"), device="cuda"),
           torch.full((H, W), -1, dtype=torch.int32, device="cuda"))
    gsr.gsr_render_forward_noalloc(ctx, sp, bins, W, H, *out)
    torch.cuda.synchronize()
    for a, b in zip(ref, out):
        assert host(a).tobytes() == host(b).tobytes()
    return bins


def test_noalloc_forward_matches_the_allocating_one():
    from differentiable_gaussian_splatting_amd import gsr
    ctx = gsr.Context(0)
    try:
        banner("no-alloc forward raster84k (2500 tiles)")
        render_both(ctx, "raster84k")
        banner("no-alloc forward tiny (16 tiles), after the larger call")
        render_both(ctx, "tiny")
        banner("no-alloc forward raster84k again")
        render_both(ctx, "raster84k")
        # 4112 x 16 px = 257 x 1 tiles is fine; 4112 x 4112 = 66049 tiles exceeds the 65536-tile scratch
        lib = gsr.load()
        bins = gsr.gsr_bins(None, None, None, 0, 257, 257, None, 0)
        st = lib.gsr_render_forward_noalloc(ctx.handle, None, None, 0, ctypes.byref(bins), 4112, 4112, None, None,
                                            None)
        assert st == gsr.GSR_EINVAL and b"scratch" in lib.gsr_last_error(ctx.handle)
    finally:
        ctx.close()
