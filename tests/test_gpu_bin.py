"""GPU binning and radix sort against the oracle: bit-exact keys, values and tile ranges."""
import numpy as np
import pytest

from gpuhelp import banner, custom_scene, dev, host, oracle_bins, scene

pytestmark = pytest.mark.gpu

SCHEMES = {"presort": 0, "key64": 1, "tile_depth": 2}


@pytest.fixture(scope="module")
def ctx():
    from differentiable_gaussian_splatting_amd import gsr
    c = gsr.Context(0)
    yield c
    c.close()


def gpu_bin(ctx, splats, depths, w, h, scheme):
    from differentiable_gaussian_splatting_amd import gsr
    gsr.gsr_set_option(ctx, gsr.GSR_OPT_BIN_SCHEME, SCHEMES[scheme])
    b = gsr.gsr_bin(ctx, dev(splats), dev(depths), w, h)
    keys, vals, ranges = gsr.gsr_bins_copy(ctx, b)
    return b, host(keys, np.uint64), host(vals, np.uint32), host(ranges, np.uint32)


def assert_bins_equal(ctx, splats, depths, w, h, scheme, ref=None):
    import oracle
    if ref is None:
        ref = oracle.bin(splats, depths, w, h)
    from differentiable_gaussian_splatting_amd import gsr
    b, k, v, r = gpu_bin(ctx, splats, depths, w, h, scheme)
    assert b.num_pairs == ref.num_pairs
    assert np.array_equal(k, ref.keys), "sorted keys differ"
    assert np.array_equal(v, ref.vals), "sorted values differ"
    assert np.array_equal(r, ref.ranges), "tile ranges differ"
    n = splats.shape[0]
    sp = host(gsr.gsr_bins_splat_pairs(ctx, b), np.uint32)
    assert sp.shape == (n,) and np.array_equal(sp, np.bincount(ref.vals, minlength=n)), "splat_pairs differ"
    return b


@pytest.mark.parametrize("scheme", list(SCHEMES))
@pytest.mark.parametrize("name", ["tiny", "raster84k", "raster410k", "bin1m"])
def test_bin_matches_oracle(ctx, name, scheme):
    banner(f"bin {name} scheme={scheme}")
    sc = scene(name)
    b = assert_bins_equal(ctx, sc.splats, sc.depths, sc.width, sc.height, scheme, oracle_bins(name))
    assert b.num_pairs > sc.spec.n  # several tiles per splat on every workload


@pytest.mark.parametrize("scheme", list(SCHEMES))
@pytest.mark.parametrize("w,h", [(24, 24), (100, 37), (17, 1), (16, 16), (1, 300), (1023, 769)])
def test_bin_ragged_images(ctx, w, h, scheme):
    banner(f"bin ragged {w}x{h} scheme={scheme}")
    sc = custom_scene(name="ragged", width=w, height=h, n=3000, seed=w * 7 + h, size_classes=((1.0, 0.3, 30.0),),
                      margin=40.0)
    assert_bins_equal(ctx, sc.splats, sc.depths, w, h, scheme)


@pytest.mark.parametrize("scheme", list(SCHEMES))
def test_bin_depth_ties_and_invalid_splats(ctx, scheme):
    banner(f"bin ties+invalid scheme={scheme}")
    sc = custom_scene(name="ties", width=160, height=120, n=20000, seed=9, size_classes=((1.0, 0.5, 12.0),),
                      depth_levels=5, margin=30.0)
    sp, d = sc.splats.copy(), sc.depths.copy()
    rng = np.random.default_rng(3)
    bad = rng.choice(len(d), 600, replace=False)
    sp[bad[:100], 0] = np.nan
    sp[bad[100:200], 8] = 1.5
    sp[bad[200:300], 2] = -1.0
    d[bad[300:400]] = 0.0
    d[bad[400:500]] = np.inf
    sp[bad[500:600], 3] = 100.0  # det < 0
    assert_bins_equal(ctx, sp, d, 160, 120, scheme)


@pytest.mark.parametrize("scheme", list(SCHEMES))
def test_bin_empty_and_all_culled(ctx, scheme):
    banner(f"bin empty scheme={scheme}")
    assert_bins_equal(ctx, np.zeros((0, 9), np.float32), np.zeros(0, np.float32), 800, 800, scheme)
    sc = custom_scene(name="off", width=64, height=64, n=500, seed=2, margin=0.0)
    sp = sc.splats.copy()
    sp[:, 0] += 10000.0  # everything off screen
    b = assert_bins_equal(ctx, sp, sc.depths, 64, 64, scheme)
    assert b.num_pairs == 0


@pytest.mark.parametrize("scheme", ["presort", "tile_depth"])
@pytest.mark.parametrize("w,h,n", [(16, 16, 700), (1024, 1024, 1 << 20), (65536, 32768, 3000)])
def test_bin_packed_and_unpacked_tile_sort(ctx, w, h, n, scheme):
    """The presort scheme packs (tile, splat) into one 32-bit key when bits(n - 1) + bits(tiles - 1) <= 32: a
    single tile (no tile pass: not packed), 2^20 splats on 4096 tiles (exactly 32 bits: packed), and 2^23 tiles
    with 3000 splats (36 bits: the two-array form). It also carries each splat's count in its depth-sort value when
    bits(n - 1) + bits(tiles) <= 32: the first case does, the other two (33 and 36 bits) gather the counts through
    the sorted indices instead. The tile-first scheme takes its counting sort in the first two cases and, past 8192
    tiles, emission and the radix sort of the tile ids (the two-array form at 36 bits). All bit-exact against the
    oracle."""
    banner(f"bin packing {w}x{h} n={n} scheme={scheme}")
    # round splats of s in 0.5-20 px over the image (drawn here: the scene generator's per-pixel upstream gradient
    # would not fit the largest image)
    rng = np.random.default_rng(n + w)
    s = np.exp(rng.uniform(np.log(0.5), np.log(20.0), n))
    sp = np.zeros((n, 9), np.float32)
    sp[:, 0], sp[:, 1] = rng.uniform(0, w, n), rng.uniform(0, h, n)
    sp[:, 2] = sp[:, 4] = 1.0 / s ** 2
    sp[:, 5:8] = rng.uniform(0, 1, (n, 3))
    sp[:, 8] = rng.uniform(0.05, 1.0, n)
    depths = rng.uniform(0.1, 10.0, n).astype(np.float32)
    assert_bins_equal(ctx, sp, depths, w, h, scheme)


def test_bin_arena_growth_and_reuse(ctx):
    """A fresh context grows its arena call by call; results stay bit-exact, and a smaller call after a larger
    one reuses the arena."""
    from differentiable_gaussian_splatting_amd import gsr
    banner("bin arena growth")
    fresh = gsr.Context(0)
    try:
        for name in ("tiny", "raster84k", "tiny"):
            sc = scene(name)
            assert_bins_equal(fresh, sc.splats, sc.depths, sc.width, sc.height, "presort", oracle_bins(name))
    finally:
        fresh.close()


@pytest.mark.parametrize("scheme", ["presort", "tile_depth"])
def test_bin_is_deterministic(ctx, scheme):
    """The tile-first scheme's counting sort places each block's pairs in LDS-atomic order; the per-tile order by
    (depth, splat) must still make every output identical from call to call."""
    banner(f"bin determinism raster84k scheme={scheme}")
    sc = scene("raster84k")
    runs = [gpu_bin(ctx, sc.splats, sc.depths, 800, 800, scheme)[1:] for _ in range(3)]
    for r in runs[1:]:
        assert all(np.array_equal(a, b) for a, b in zip(r, runs[0]))


@pytest.mark.parametrize("scheme", list(SCHEMES))
@pytest.mark.parametrize("name", ["tiny", "raster84k"])
def test_bin_without_keys(ctx, name, scheme):
    from differentiable_gaussian_splatting_amd import gsr
    banner(f"bin keys off {name} scheme={scheme}")
    sc = scene(name)
    gsr.gsr_set_option(ctx, gsr.GSR_OPT_BIN_SCHEME, SCHEMES[scheme])
    gsr.gsr_set_option(ctx, gsr.GSR_OPT_BIN_KEYS, 0)
    try:
        b = gsr.gsr_bin(ctx, dev(sc.splats), dev(sc.depths), sc.width, sc.height)
        assert b.raw.keys is None
        _, v, r = gsr.gsr_bins_copy(ctx, b)
        ref = oracle_bins(name)
        assert np.array_equal(host(v, np.uint32), ref.vals) and np.array_equal(host(r, np.uint32), ref.ranges)
    finally:
        gsr.gsr_set_option(ctx, gsr.GSR_OPT_BIN_KEYS, 1)


# ------------------------------------------------------------------------------------------------ the sort alone
@pytest.mark.parametrize("n", [0, 1, 255, 256, 257, 1234, 4095, 4096, 4097, 100000, 1000003, 2097151, 2097152,
                               3000017])
@pytest.mark.parametrize("key_bits", [64, 44, 13])
def test_radix_sort_matches_stable_sort(ctx, n, key_bits):
    import oracle
    from differentiable_gaussian_splatting_amd import gsr
    banner(f"radix sort n={n} key_bits={key_bits}")
    rng = np.random.default_rng(n + key_bits)
    keys = rng.integers(0, np.iinfo(np.uint64).max, n, dtype=np.uint64, endpoint=True)
    if key_bits < 64:
        keys &= np.uint64((1 << key_bits) - 1)
    vals = rng.permutation(n).astype(np.uint32) if n else np.zeros(0, np.uint32)
    ko, vo = gsr.gsr_radix_sort(ctx, dev(keys), dev(vals), key_bits)
    rk, rv = oracle.sort_pairs(keys, vals)
    assert np.array_equal(host(ko, np.uint64), rk) and np.array_equal(host(vo, np.uint32), rv)


def test_radix_sort_ties_heavy(ctx):
    import oracle
    from differentiable_gaussian_splatting_amd import gsr
    banner("radix sort ties n=5000")
    rng = np.random.default_rng(5000)
    keys = rng.integers(0, 7, 5000).astype(np.uint64) << np.uint64(32)
    vals = rng.permutation(5000).astype(np.uint32)
    ko, vo = gsr.gsr_radix_sort(ctx, dev(keys), dev(vals), 64)
    rk, rv = oracle.sort_pairs(keys, vals)
    assert np.array_equal(host(vo, np.uint32), rv) and np.array_equal(host(ko, np.uint64), rk)


def test_radix_sort_rejects_bad_arguments(ctx):
    from differentiable_gaussian_splatting_amd import gsr
    banner("radix sort argument errors")
    k = dev(np.zeros(10, np.uint64))
    v = dev(np.zeros(10, np.uint32))
    with pytest.raises(gsr.GsrError):
        gsr.gsr_radix_sort(ctx, k, v, 0)
    with pytest.raises(gsr.GsrError):
        gsr.gsr_radix_sort(ctx, k, v, 65)


# ------------------------------------------------------------------------------------- exact-ellipse overlap rule
def set_rule(ctx, rule):
    from differentiable_gaussian_splatting_amd import gsr
    gsr.gsr_set_option(ctx, gsr.GSR_OPT_BIN_RULE, gsr.GSR_BIN_ELLIPSE if rule == "ellipse" else gsr.GSR_BIN_BOX)


@pytest.mark.parametrize("scheme", list(SCHEMES))
@pytest.mark.parametrize("name", ["tiny", "raster84k", "bin1m"])
def test_bin_ellipse_rule_matches_oracle(ctx, name, scheme):
    import oracle
    banner(f"bin ellipse {name} scheme={scheme}")
    sc = scene(name)
    ref = oracle.bin(sc.splats, sc.depths, sc.width, sc.height, rule="ellipse")
    set_rule(ctx, "ellipse")
    try:
        assert_bins_equal(ctx, sc.splats, sc.depths, sc.width, sc.height, scheme, ref)
    finally:
        set_rule(ctx, "box")
    print(f"  {ref.num_pairs} pairs")


@pytest.mark.parametrize("w,h", [(24, 24), (100, 37), (1023, 769)])
def test_bin_ellipse_rule_ragged_images(ctx, w, h):
    import oracle
    banner(f"bin ellipse ragged {w}x{h}")
    sc = custom_scene(name="r", width=w, height=h, n=3000, seed=w + h, size_classes=((1.0, 0.5, 30.0),), margin=20.0)
    set_rule(ctx, "ellipse")
    try:
        for scheme in SCHEMES:
            assert_bins_equal(ctx, sc.splats, sc.depths, w, h, scheme,
                              oracle.bin(sc.splats, sc.depths, w, h, rule="ellipse"))
    finally:
        set_rule(ctx, "box")


@pytest.mark.parametrize("seed", range(16))
def test_tile_first_random_scenes(ctx, seed):
    """Seeded random scenes for the tile-first scheme's two-level counting sort: image sizes from 1 to 400 pixels a
    side (odd tile counts leave super-tiles partly off the grid), 1 to 20,000 splats of 0.2-60 px, means spread past
    the image, and in half of them depths quantised to a few levels (ties and crowded buckets). A fresh context per
    scene (its first call has no pair count to go by). Bit-exact against the oracle; then the same scene under the
    other schemes, and under the ellipse rule with every scheme."""
    import oracle
    from differentiable_gaussian_splatting_amd import gsr
    rng = np.random.default_rng(1000 + seed)
    w, h = int(rng.integers(1, 401)), int(rng.integers(1, 401))
    n = int(rng.choice([1, 2, 50, 500, 5000, 20000]))
    levels = int(rng.choice([0, 0, 2, 7])) if seed % 2 else 0
    sc = custom_scene(name="rand", width=w, height=h, n=n, seed=2000 + seed,
                      size_classes=((0.6, 0.2, 6.0), (0.4, 6.0, 60.0)), margin=float(rng.uniform(0, 80)),
                      depth_levels=levels)
    banner(f"bin tile-first random seed={seed} {w}x{h} n={n} levels={levels}")
    ref = oracle.bin(sc.splats, sc.depths, w, h)
    c = gsr.Context(0)
    try:
        assert_bins_equal(c, sc.splats, sc.depths, w, h, "tile_depth", ref)
        assert_bins_equal(c, sc.splats, sc.depths, w, h, "tile_depth", ref)
        # the same scene under the other schemes, and under the ellipse rule (per-tile lists) with every scheme
        for scheme in SCHEMES:
            if scheme != "tile_depth":
                assert_bins_equal(c, sc.splats, sc.depths, w, h, scheme, ref)
        ref_e = oracle.bin(sc.splats, sc.depths, w, h, rule="ellipse")
        set_rule(c, "ellipse")
        for scheme in SCHEMES:
            assert_bins_equal(c, sc.splats, sc.depths, w, h, scheme, ref_e)
    finally:
        c.close()


@pytest.mark.parametrize("rule", ["box", "ellipse"])
@pytest.mark.parametrize("w,h,n,cluster,levels", [(16, 16, 6000, 0.0, 0), (64, 48, 30000, 0.0, 0),
                                                   (800, 800, 200000, 0.3, 0), (16, 16, 6000, 0.0, 3),
                                                   (16, 16, 70000, 0.0, 0), (16, 16, 70000, 0.0, 3)])
def test_tile_depth_long_lists(ctx, w, h, n, cluster, levels, rule):
    """Lists longer than the tile-first scheme's on-chip capacities: one tile of 6000 pairs; twelve tiles of 5-11
    thousand; 16 tiles of up to 25 thousand (30% of the splats in a 48-pixel square) among 2,484 short ones, both
    forms in one launch; one tile of 6000 pairs at three depths (crowded buckets); and one tile of 70,000 pairs
    (positions past 16 bits), at spread depths and at three. Under the box rule the lists are the super-tiles' (the
    same splats), ordered in chunks of at most 4608 on chip, or by the radix sort through the arena when one chunk
    would be longer (70,000 at three depths); under the ellipse rule each tile's list is ordered on its own, past
    3456 pairs by buckets through the arena, or by the radix sort when a bucket is crowded. Bit-exact against the
    oracle on a fresh context and again with the count seen."""
    import oracle
    from differentiable_gaussian_splatting_amd import gsr
    banner(f"bin tile_depth long lists {w}x{h} n={n} cluster={cluster} levels={levels} rule={rule}")
    rng = np.random.default_rng(n)
    s = np.exp(rng.uniform(np.log(0.5), np.log(8.0), n))
    sp = np.zeros((n, 9), np.float32)
    sp[:, 0], sp[:, 1] = rng.uniform(0, w, n), rng.uniform(0, h, n)
    k = int(cluster * n)
    sp[:k, 0], sp[:k, 1] = rng.uniform(376, 424, k), rng.uniform(376, 424, k)
    sp[:, 2] = sp[:, 4] = 1.0 / s ** 2
    sp[:, 5:8] = rng.uniform(0, 1, (n, 3))
    sp[:, 8] = rng.uniform(0.05, 1.0, n)
    depths = rng.uniform(0.1, 10.0, n).astype(np.float32)
    depths[: n // 10] = depths[n // 10: 2 * (n // 10)]  # equal depths: ties keep splat order
    if levels:
        depths = rng.choice(np.array([0.5, 2.0, 7.5], np.float32)[:levels], n)
    ref = oracle.bin(sp, depths, w, h, rule=rule)
    lens = ref.ranges[:, 1].astype(np.int64) - ref.ranges[:, 0]
    assert lens.max() > 4608
    c = gsr.Context(0)
    try:
        set_rule(c, rule)
        assert_bins_equal(c, sp, depths, w, h, "tile_depth", ref)
        assert_bins_equal(c, sp, depths, w, h, "tile_depth", ref)
    finally:
        c.close()


@pytest.mark.parametrize("w,h", [(2048, 1024), (2064, 1024)])
def test_tile_first_fused_tile_limit(ctx, w, h):
    """The tile-first scheme's counting sort keeps a counter per tile in LDS, up to 8192 tiles: 2048 x 1024 (8192
    tiles) takes it, 2064 x 1024 (8256) emission and the radix sort of the tile ids. Both bit-exact."""
    banner(f"bin tile-first fused limit {w}x{h}")
    sc = custom_scene(name="limit", width=w, height=h, n=20000, seed=w + h, size_classes=((1.0, 0.3, 30.0),),
                      margin=40.0)
    assert_bins_equal(ctx, sc.splats, sc.depths, w, h, "tile_depth")


@pytest.mark.parametrize("rule,m", [("box", 1), ("box", 2), ("box", 4608), ("box", 4609), ("ellipse", 1),
                                    ("ellipse", 2), ("ellipse", 3456), ("ellipse", 3457)])
def test_tile_depth_list_length_edges(ctx, rule, m):
    """One tile holding exactly m pairs: a single entry, two, the on-chip capacity and one more (the arena path).
    Under the box rule the counting sort's super-tile (here the one tile, its three other tiles off the grid) orders
    up to 4608 entries on chip; under the ellipse rule each tile's list is ordered on its own, up to 3456 on chip.
    Splats of 0.3-1 px inside the tile's inner 8 x 8 pixels, so each covers that tile only; a third of them share
    depths, so ties are ordered by splat index."""
    banner(f"bin tile-depth list length rule={rule} m={m}")
    rng = np.random.default_rng(m)
    s = rng.uniform(0.3, 1.0, m)
    sp = np.zeros((m, 9), np.float32)
    sp[:, 0], sp[:, 1] = rng.uniform(4.5, 11.5, m), rng.uniform(4.5, 11.5, m)
    sp[:, 2] = sp[:, 4] = 1.0 / s ** 2
    sp[:, 5:8] = rng.uniform(0, 1, (m, 3))
    sp[:, 8] = rng.uniform(0.05, 1.0, m)
    depths = rng.uniform(0.1, 10.0, m).astype(np.float32)
    depths[: m // 3] = depths[m - m // 3:]
    import oracle
    ref = oracle.bin(sp, depths, 16, 16, rule=rule)
    assert ref.num_pairs == m
    from differentiable_gaussian_splatting_amd import gsr
    c = gsr.Context(0)  # a fresh context: the tile-first path on the first call
    try:
        set_rule(c, rule)
        assert_bins_equal(c, sp, depths, 16, 16, "tile_depth", ref)
    finally:
        c.close()
