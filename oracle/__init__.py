"""Plain CPU oracle of the tile-based differentiable 2D-splat rasterizer (ctypes front end of oracle.cpp).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline leg may import this module.
The product path (the HIP library and its binding) never imports, links or calls it.

Every function takes and returns numpy arrays on the host. Layouts:
  splats   [N, 9]  {x, y, a, b, c, r, g, b, o}  (float32, or float64 for the *_f64 variants)
  depths   [N]     float32
  keys     [P]     uint64  (tile_id << 32) | float-bits(depth)
  vals     [P]     uint32  splat index
  ranges   [T, 2]  uint32  per-tile [start, end) into keys/vals, T = ceil(W/16) * ceil(H/16)
  out_rgba [H, W, 4], final_T [H, W], last_contrib [H, W] uint32, v_out [H, W, 4], splats_grad [N, 9]
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# Plain IEEE arithmetic: no fused multiply-add contraction, no fast-math.
_CXXFLAGS = ["-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", "-ffp-contract=off", "-fno-fast-math"]

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.cpp into liboracle.so with g++ (host only)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["g++", *_CXXFLAGS, _SRC, "-o", tmp], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    u32, u64, f32 = ctypes.c_uint32, ctypes.c_uint64, ctypes.c_float
    lib.oracle_bin_count.argtypes = [P, P, u32, u32, u32, P]
    lib.oracle_tile_rect.argtypes = [P, f32, u32, u32, P]
    lib.oracle_bin.argtypes = [P, P, u32, u32, u32, P, P, P, u64]
    lib.oracle_bin_rule.argtypes = [P, P, u32, u32, u32, ctypes.c_int, P, P, P, u64]
    lib.oracle_bin_count_rule.argtypes = [P, P, u32, u32, u32, ctypes.c_int, P]
    lib.oracle_ellipse_meets_tile.argtypes = [P, u32, u32]
    lib.oracle_sort_pairs.argtypes = [P, P, u64, P, P]
    lib.oracle_render_forward_f32.argtypes = [P, P, P, u32, u32, P, P, P, P]
    lib.oracle_render_forward_f64.argtypes = [P, P, P, u32, u32, P, P, P, P]
    lib.oracle_render_backward_f32.argtypes = [P, u32, P, P, u32, u32, P, P, P, P, P, P]
    lib.oracle_render_backward_f64.argtypes = [P, u32, P, P, u32, u32, P, P, P, P, P]
    lib.oracle_adam_step.argtypes = [P, P, P, P, u64, f32, f32, f32, f32, f32, f32]
    lib.oracle_render_forward_f32_mt.argtypes = [P, P, P, u32, u32, P, P, P, u32]
    lib.oracle_render_backward_f32_mt.argtypes = [P, u32, P, P, u32, u32, P, P, P, P, P, u32]
    lib.oracle_trace_pixel_f32.argtypes = [P, P, P, u32, u32, u32, u32, u32, P, P, P, P, P]
    lib.oracle_trace_candidates_f32.argtypes = [P, P, P, u32, u32, u32, u32, u32, P, P, P, P]
    lib.oracle_render_backward_exact.argtypes = [P, u32, P, P, u32, u32, P, P, P, P, u32]
    for name in ("oracle_bin_count", "oracle_tile_rect", "oracle_bin", "oracle_sort_pairs",
                 "oracle_render_forward_f32", "oracle_render_forward_f64", "oracle_render_backward_f32",
                 "oracle_render_backward_f64", "oracle_adam_step", "oracle_trace_pixel_f32",
                 "oracle_trace_candidates_f32", "oracle_render_backward_exact"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def tiles_of(width: int, height: int) -> tuple[int, int]:
    return (width + 15) // 16, (height + 15) // 16


@dataclass
class Bins:
    keys: np.ndarray    # uint64 [P]
    vals: np.ndarray    # uint32 [P]
    ranges: np.ndarray  # uint32 [T, 2]
    tiles_x: int
    tiles_y: int

    @property
    def num_pairs(self) -> int:
        return int(self.keys.shape[0])


def tile_rect(splat, depth: float, width: int, height: int):
    """(tx0, tx1, ty0, ty1) of one splat's tile rectangle, or None when it is culled or off the grid."""
    lib = _load()
    s = _c(splat, np.float32).reshape(9)
    rect = np.zeros(4, np.uint32)
    empty = lib.oracle_tile_rect(_ptr(s), ctypes.c_float(depth), width, height, _ptr(rect))
    return None if empty else tuple(int(v) for v in rect)


RULES = {"box": 0, "ellipse": 1}


def ellipse_meets_tile(splat, tx: int, ty: int) -> bool:
    """The exact-ellipse rule's test of one splat against one tile."""
    s = _c(splat, np.float32).reshape(9)
    return bool(_load().oracle_ellipse_meets_tile(_ptr(s), tx, ty))


def bin_count(splats, depths, width: int, height: int, rule: str = "box") -> int:
    """Number of (splat, tile) pairs the binning emits under the rule."""
    s = _c(splats, np.float32).reshape(-1, 9)
    d = _c(depths, np.float32).reshape(-1)
    p = ctypes.c_uint64(0)
    _check(_load().oracle_bin_count_rule(_ptr(s), _ptr(d), s.shape[0], width, height, RULES[rule],
                                         ctypes.byref(p)), "bin_count")
    return int(p.value)


def bin(splats, depths, width: int, height: int, rule: str = "box") -> Bins:
    """Emit, stable-sort and range-extract the (tile | depth) keys; rule 'box' (the 3-sigma box) or 'ellipse'
    (the box's tiles that the 3-sigma ellipse meets)."""
    lib = _load()
    s = _c(splats, np.float32).reshape(-1, 9)
    d = _c(depths, np.float32).reshape(-1)
    n = s.shape[0]
    assert d.shape[0] == n
    r = RULES[rule]
    p = ctypes.c_uint64(0)
    _check(lib.oracle_bin_count_rule(_ptr(s), _ptr(d), n, width, height, r, ctypes.byref(p)), "bin_count")
    tx, ty = tiles_of(width, height)
    keys = np.zeros(p.value, np.uint64)
    vals = np.zeros(p.value, np.uint32)
    ranges = np.zeros((tx * ty, 2), np.uint32)
    _check(lib.oracle_bin_rule(_ptr(s), _ptr(d), n, width, height, r, _ptr(keys), _ptr(vals), _ptr(ranges),
                               p.value), "bin")
    return Bins(keys, vals, ranges, tx, ty)


def sort_pairs(keys, vals):
    lib = _load()
    k = _c(keys, np.uint64).reshape(-1)
    v = _c(vals, np.uint32).reshape(-1)
    ko = np.empty_like(k)
    vo = np.empty_like(v)
    _check(lib.oracle_sort_pairs(_ptr(k), _ptr(v), k.shape[0], _ptr(ko), _ptr(vo)), "sort_pairs")
    return ko, vo


STAT_NAMES = ("visited", "sigma_neg", "alpha_reject", "contrib", "stopped", "sigma_ge_skip", "clamped",
              "fingerprint")


def render_forward(splats, bins: Bins, width: int, height: int, precision: str = "f32"):
    """Returns (out_rgba [H,W,4], final_T [H,W], last_contrib [H,W], stats dict)."""
    lib = _load()
    dt = np.float32 if precision == "f32" else np.float64
    s = _c(splats, dt).reshape(-1, 9)
    out = np.zeros((height, width, 4), dt)
    ft = np.zeros((height, width), dt)
    lc = np.zeros((height, width), np.uint32)
    st = np.zeros(8, np.uint64)
    vals = _c(bins.vals, np.uint32)
    ranges = _c(bins.ranges, np.uint32)
    fn = lib.oracle_render_forward_f32 if precision == "f32" else lib.oracle_render_forward_f64
    _check(fn(_ptr(s), _ptr(vals), _ptr(ranges), width, height, _ptr(out), _ptr(ft), _ptr(lc), _ptr(st)),
           "render_forward")
    return out, ft, lc, {k: int(v) for k, v in zip(STAT_NAMES, st)}


BWD_STAT_NAMES = ("visited", "sigma_neg", "sigma_ge_skip", "alpha_reject", "contrib", "clamped")


def render_backward(splats, bins: Bins, width: int, height: int, out_rgba, final_T, last_contrib, v_out,
                    precision: str = "f32", stats: dict | None = None):
    """Returns splats_grad [N, 9] (float32, or float64 for precision='f64'). For precision='f32', a dict passed
    as `stats` receives the replay counters (BWD_STAT_NAMES)."""
    lib = _load()
    dt = np.float32 if precision == "f32" else np.float64
    s = _c(splats, dt).reshape(-1, 9)
    n = s.shape[0]
    grad = np.zeros((n, 9), dt)
    args = [_ptr(s), n, _ptr(_c(bins.vals, np.uint32)), _ptr(_c(bins.ranges, np.uint32)), width, height,
            _ptr(_c(out_rgba, dt)), _ptr(_c(final_T, dt)), _ptr(_c(last_contrib, np.uint32)), _ptr(_c(v_out, dt)),
            _ptr(grad)]
    if precision == "f32":
        st = np.zeros(6, np.uint64)
        _check(lib.oracle_render_backward_f32(*args, _ptr(st)), "render_backward")
        if stats is not None:
            stats.update({k: int(v) for k, v in zip(BWD_STAT_NAMES, st)})
    else:
        _check(lib.oracle_render_backward_f64(*args), "render_backward")
    return grad


def render_backward_exact(splats, bins: Bins, width: int, height: int, out_rgba, last_contrib, v_out,
                          threads: int = 0):
    """The backward's exact values on its given inputs (oracle_render_backward_exact): float64 [N, 9]. Decisions
    (composite, clamp) as the fp32 backward takes them for entries before last_contrib; sigma, G, alpha, T and the
    gradient terms in fp64, with C_final = out_rgba (the forward output the backward is given, taken in double).
    `threads` 0: up to 16 host threads."""
    lib = _load()
    s = _c(splats, np.float32).reshape(-1, 9)
    n = s.shape[0]
    grad = np.zeros((n, 9), np.float64)
    _check(lib.oracle_render_backward_exact(_ptr(s), n, _ptr(_c(bins.vals, np.uint32)),
                                            _ptr(_c(bins.ranges, np.uint32)), width, height,
                                            _ptr(_c(out_rgba, np.float64)), _ptr(_c(last_contrib, np.uint32)),
                                            _ptr(_c(v_out, np.float32)), _ptr(grad),
                                            threads or min(16, os.cpu_count() or 1)), "render_backward_exact")
    return grad


def render_forward_mt(splats, bins: Bins, width: int, height: int, threads: int):
    """render_forward (f32) spread over host threads by bands of tile rows (for timing on all cores); the same
    outputs as the single-threaded call."""
    lib = _load()
    s = _c(splats, np.float32).reshape(-1, 9)
    out = np.zeros((height, width, 4), np.float32)
    ft = np.zeros((height, width), np.float32)
    lc = np.zeros((height, width), np.uint32)
    _check(lib.oracle_render_forward_f32_mt(_ptr(s), _ptr(_c(bins.vals, np.uint32)), _ptr(_c(bins.ranges, np.uint32)),
                                            width, height, _ptr(out), _ptr(ft), _ptr(lc), threads), "forward_mt")
    return out, ft, lc


def render_backward_mt(splats, bins: Bins, width: int, height: int, out_rgba, final_T, last_contrib, v_out,
                       threads: int):
    """render_backward (f32) spread over host threads; per-thread sums in double added in thread order."""
    lib = _load()
    s = _c(splats, np.float32).reshape(-1, 9)
    n = s.shape[0]
    grad = np.zeros((n, 9), np.float32)
    _check(lib.oracle_render_backward_f32_mt(_ptr(s), n, _ptr(_c(bins.vals, np.uint32)),
                                             _ptr(_c(bins.ranges, np.uint32)), width, height,
                                             _ptr(_c(out_rgba, np.float32)), _ptr(_c(final_T, np.float32)),
                                             _ptr(_c(last_contrib, np.uint32)), _ptr(_c(v_out, np.float32)),
                                             _ptr(grad), threads), "backward_mt")
    return grad


def adam_step(param, grad, m, v, lr, beta1, beta2, eps, bc1, bc2):
    """One Adam step on float32 arrays; returns new (param, m, v) copies."""
    lib = _load()
    p = np.array(param, np.float32, copy=True).reshape(-1)
    mm = np.array(m, np.float32, copy=True).reshape(-1)
    vv = np.array(v, np.float32, copy=True).reshape(-1)
    g = _c(grad, np.float32).reshape(-1)
    _check(lib.oracle_adam_step(_ptr(p), _ptr(g), _ptr(mm), _ptr(vv), p.shape[0], lr, beta1, beta2, eps, bc1, bc2),
           "adam_step")
    return p, mm, vv


def adam_step_visible(param, grad, m, v, lr, beta1, beta2, eps, bc1, bc2, visible):
    """Visible-only Adam (rasterize forward + adam kernel audit page, section 2 "(h)"): the rows [n, k] of splats with
    visible[i] true take adam_step; the other rows of param, m and v are returned unchanged. Returns new copies."""
    vis = np.asarray(visible, bool).reshape(-1)
    n = vis.shape[0]
    p = np.array(param, np.float32, copy=True).reshape(n, -1)
    mm = np.array(m, np.float32, copy=True).reshape(n, -1)
    vv = np.array(v, np.float32, copy=True).reshape(n, -1)
    g = np.asarray(grad, np.float32).reshape(n, -1)
    if vis.any():
        rp, rm, rv = adam_step(p[vis], g[vis], mm[vis], vv[vis], lr, beta1, beta2, eps, bc1, bc2)
        k = p.shape[1]
        p[vis], mm[vis], vv[vis] = rp.reshape(-1, k), rm.reshape(-1, k), rv.reshape(-1, k)
    return p.reshape(-1), mm.reshape(-1), vv.reshape(-1)


TRACE_CODES = {1: "sigma_neg", 2: "alpha_reject", 3: "stop", 4: "composite", 5: "composite_clamped"}


def trace_pixel(splats, bins: Bins, width: int, height: int, px: int, py: int, max_len: int = 1 << 20):
    """Per-entry trace of one pixel's forward: dict of arrays code, sigma, alpha, T_before, T_after."""
    lib = _load()
    s = _c(splats, np.float32).reshape(-1, 9)
    t = (py // 16) * bins.tiles_x + (px // 16)
    n = min(max_len, int(bins.ranges[t, 1] - bins.ranges[t, 0]))
    code = np.zeros(n, np.uint32)
    sig, al, tb, ta = (np.zeros(n, np.float32) for _ in range(4))
    j = lib.oracle_trace_pixel_f32(_ptr(s), _ptr(_c(bins.vals, np.uint32)), _ptr(_c(bins.ranges, np.uint32)),
                                   width, height, px, py, n, _ptr(code), _ptr(sig), _ptr(al), _ptr(tb), _ptr(ta))
    if j < 0:
        raise ValueError("pixel outside the image")
    return {"code": code[:j], "sigma": sig[:j], "alpha": al[:j], "T_before": tb[:j], "T_after": ta[:j]}


def trace_candidates(splats, bins: Bins, width: int, height: int, px: int, py: int):
    """One pixel's compositing candidates with the stop test left out (oracle_trace_candidates_f32): dict of
    arrays pos (1-based list position), alpha, T_next (T (1 - alpha)) and rgb [m, 3] (the colour once composited).
    The forward stops at the first candidate whose T_next is below 1e-4."""
    lib = _load()
    s = _c(splats, np.float32).reshape(-1, 9)
    t = (py // 16) * bins.tiles_x + (px // 16)
    n = int(bins.ranges[t, 1] - bins.ranges[t, 0])
    pos = np.zeros(n, np.uint32)
    al, tn = np.zeros(n, np.float32), np.zeros(n, np.float32)
    rgb = np.zeros((n, 3), np.float32)
    j = lib.oracle_trace_candidates_f32(_ptr(s), _ptr(_c(bins.vals, np.uint32)), _ptr(_c(bins.ranges, np.uint32)),
                                        width, height, px, py, n, _ptr(pos), _ptr(al), _ptr(tn), _ptr(rgb))
    if j < 0:
        raise ValueError("pixel outside the image")
    return {"pos": pos[:j], "alpha": al[:j], "T_next": tn[:j], "rgb": rgb[:j]}
