"""Failure handling through the C ABI: counts that do not fit their 32-bit fields (GSR_EOVERFLOW) and a device arena
that cannot grow (GSR_ENOMEM). Every failing call here is refused on the host before anything is queued, so no
kernel ever sees the bad sizes; the conditions are forced from the host (sizes, and the arena byte limit
GSR_OPT_ARENA_LIMIT). After each failure the same context must still give the oracle's bins bit for bit.
[C0 resident arena + C1 pass skip page, section 2 table, row "C0 resident arena": the arena keeps its buffers]
"""
import ctypes

import numpy as np
import pytest

from gpuhelp import banner, dev, host, oracle_bins, scene

pytestmark = pytest.mark.gpu


def check_bins(ctx, name):
    from differentiable_gaussian_splatting_amd import gsr
    sc = scene(name)
    b = gsr.gsr_bin(ctx, dev(sc.splats), dev(sc.depths), sc.width, sc.height)
    keys, vals, ranges = gsr.gsr_bins_copy(ctx, b)
    ob = oracle_bins(name)
    assert np.array_equal(host(keys, np.uint64), ob.keys)
    assert np.array_equal(host(vals, np.uint32), ob.vals)
    assert np.array_equal(host(ranges, np.uint32), ob.ranges)
    return b


def test_overflow_is_refused_before_any_launch():
    from differentiable_gaussian_splatting_amd import gsr
    banner("errors: EOVERFLOW")
    lib = gsr.load()
    ctx = gsr.Context(0)
    try:
        h = ctx.handle
        # backward: n * 9 >= 2^32 (checked before the pointers, which are null here)
        n_big = (1 << 32) // 9 + 1
        bins = gsr.gsr_bins(None, None, None, 0, 1, 1, None, 0)
        st = lib.gsr_render_backward(h, None, None, n_big, ctypes.byref(bins), 16, 16, None, None, None, None, None)
        assert st == gsr.GSR_EOVERFLOW, st
        assert b"n * 9" in lib.gsr_last_error(h)
        # radix sort: n >= 2^32
        st = lib.gsr_radix_sort(h, None, None, None, 1 << 32, 32, None, None)
        assert st == gsr.GSR_EOVERFLOW, st
        # reserve: 2^32 pairs
        st = lib.gsr_reserve(h, 1 << 32, 16)
        assert st == gsr.GSR_EOVERFLOW, st
        # projection: n * 48 >= 2^32
        cam = gsr.camera(np.eye(3), [0, 0, 0], 100.0, 100.0, 8.0, 8.0)
        st = lib.gsr_project_forward(h, None, ctypes.byref(cam), (1 << 32) // 48 + 1, None, None, None, None, None,
                                     None, None)
        assert st == gsr.GSR_EOVERFLOW, st
        check_bins(ctx, "tiny")
    finally:
        ctx.close()


def test_arena_limit_gives_enomem_and_leaves_the_arena_usable():
    from differentiable_gaussian_splatting_amd import gsr
    banner("errors: ENOMEM under an arena limit")
    lib = gsr.load()
    ctx = gsr.Context(0)
    try:
        h = ctx.handle
        gsr.gsr_set_option(ctx, gsr.GSR_OPT_ARENA_LIMIT, 64 << 20)
        check_bins(ctx, "raster84k")  # about 30 MB of arena
        # the 410k scene needs about 220 MB of pairs: refused, and the arena stays as it was
        sc = scene("raster410k")
        with pytest.raises(gsr.GsrError) as e:
            gsr.gsr_bin(ctx, dev(sc.splats), dev(sc.depths), sc.width, sc.height)
        assert e.value.status == gsr.GSR_ENOMEM and "arena limit" in str(e.value)
        check_bins(ctx, "raster84k")
        # an impossible reservation (32 GB of keys alone)
        st = lib.gsr_reserve(h, (1 << 32) - 1, (1 << 32) - 1)
        assert st == gsr.GSR_ENOMEM, st
        check_bins(ctx, "raster84k")
        check_bins(ctx, "tiny")
        # a negative limit is rejected; lifting the limit lets the large scene through
        assert lib.gsr_set_option(h, gsr.GSR_OPT_ARENA_LIMIT, -1) == gsr.GSR_EINVAL
        gsr.gsr_set_option(ctx, gsr.GSR_OPT_ARENA_LIMIT, 0)
        b = gsr.gsr_bin(ctx, dev(sc.splats), dev(sc.depths), sc.width, sc.height)
        assert b.num_pairs == oracle_bins("raster410k").num_pairs
    finally:
        ctx.close()
