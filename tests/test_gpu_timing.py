"""GSR_OPT_KERNEL_TIMING and gsr_kernel_times: rings of HIP event pairs around each entry point's main kernels."""
import numpy as np
import pytest

from gpuhelp import banner, dev, scene

pytestmark = pytest.mark.gpu


@pytest.fixture()
def ctx():
    from differentiable_gaussian_splatting_amd import gsr
    c = gsr.Context(0)
    yield c
    c.close()


def test_kernel_times_record_each_stage_in_a_ring(ctx):
    from differentiable_gaussian_splatting_amd import gsr
    banner("kernel timing rings")
    sc = scene("raster84k")
    sp, dp, vo = dev(sc.splats), dev(sc.depths), dev(sc.v_out)
    gsr.gsr_set_option(ctx, gsr.GSR_OPT_BIN_SCHEME, gsr.GSR_BIN_PRESORT)
    gsr.gsr_set_option(ctx, gsr.GSR_OPT_KERNEL_TIMING, 3)
    for _ in range(5):
        b = gsr.gsr_bin(ctx, sp, dp, sc.width, sc.height)
        out, ft, lc = gsr.gsr_render_forward(ctx, sp, b, sc.width, sc.height)
        gsr.gsr_render_backward(ctx, sp, b, sc.width, sc.height, out, ft, lc, vo)
    for stage in (gsr.GSR_STAGE_BIN, gsr.GSR_STAGE_FORWARD, gsr.GSR_STAGE_BACKWARD, gsr.GSR_STAGE_DEPTH_SORT,
                  gsr.GSR_STAGE_TILE_SORT):
        t = gsr.gsr_kernel_times(ctx, stage)
        assert len(t) == 3 and all(0 < x < 1000 for x in t), (stage, t)  # the last 3 of 5 launches
        assert len(gsr.gsr_kernel_times(ctx, stage, max_count=2)) == 2
    # the two sorts lie inside the bin stage
    assert sum(gsr.gsr_kernel_times(ctx, gsr.GSR_STAGE_DEPTH_SORT)) + \
        sum(gsr.gsr_kernel_times(ctx, gsr.GSR_STAGE_TILE_SORT)) < sum(gsr.gsr_kernel_times(ctx, gsr.GSR_STAGE_BIN))
    assert gsr.gsr_kernel_times(ctx, gsr.GSR_STAGE_ADAM) == []  # nothing recorded yet
    z = dev(np.zeros(8, np.float32))
    gsr.gsr_adam_step(ctx, [(z, z, z, z, 1e-3)], 0.9, 0.999, 1e-15, 0.1, 0.001)
    assert len(gsr.gsr_kernel_times(ctx, gsr.GSR_STAGE_ADAM)) == 1
    # setting the option again clears the rings; 0 turns timing off
    gsr.gsr_set_option(ctx, gsr.GSR_OPT_KERNEL_TIMING, 4)
    assert gsr.gsr_kernel_times(ctx, gsr.GSR_STAGE_FORWARD) == []
    gsr.gsr_set_option(ctx, gsr.GSR_OPT_KERNEL_TIMING, 0)
    with pytest.raises(gsr.GsrError):
        gsr.gsr_kernel_times(ctx, gsr.GSR_STAGE_FORWARD)


def test_kernel_times_of_the_tile_first_binning(ctx):
    """The tile-first scheme (the default) records its counting sort's scans, its scatter and the per-tile order;
    no depth sort runs."""
    from differentiable_gaussian_splatting_amd import gsr
    banner("kernel timing tile-first")
    sc = scene("raster84k")
    sp, dp = dev(sc.splats), dev(sc.depths)
    gsr.gsr_set_option(ctx, gsr.GSR_OPT_KERNEL_TIMING, 3)
    for _ in range(4):
        gsr.gsr_bin(ctx, sp, dp, sc.width, sc.height)
    inner = 0.0
    for stage in (gsr.GSR_STAGE_TILE_SCAN, gsr.GSR_STAGE_TILE_SORT, gsr.GSR_STAGE_TILE_DEPTH):
        t = gsr.gsr_kernel_times(ctx, stage)
        assert len(t) == 3 and all(0 < x < 1000 for x in t), (stage, t)
        inner += sum(t)
    assert gsr.gsr_kernel_times(ctx, gsr.GSR_STAGE_DEPTH_SORT) == []
    assert inner < sum(gsr.gsr_kernel_times(ctx, gsr.GSR_STAGE_BIN))


def test_kernel_timing_rejects_bad_arguments(ctx):
    from differentiable_gaussian_splatting_amd import gsr
    banner("kernel timing argument errors")
    with pytest.raises(gsr.GsrError):
        gsr.gsr_set_option(ctx, gsr.GSR_OPT_KERNEL_TIMING, 4097)
    with pytest.raises(gsr.GsrError):
        gsr.gsr_set_option(ctx, gsr.GSR_OPT_KERNEL_TIMING, -1)
    gsr.gsr_set_option(ctx, gsr.GSR_OPT_KERNEL_TIMING, 2)
    for bad in (-1, gsr.GSR_STAGE_TILE_SCAN + 1):
        with pytest.raises(gsr.GsrError):
            gsr.gsr_kernel_times(ctx, bad)
