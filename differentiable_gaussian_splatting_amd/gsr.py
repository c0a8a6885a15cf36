"""Thin Python binding of libgsr (include/gsr.h): argument marshalling only, every step runs in the HIP library.

Tensors are PyTorch device tensors; the work is queued on torch's current stream unless a stream is given. Unsigned
buffers (keys, values, ranges, last contributors) are carried in torch's signed integer dtypes of the same width
(int64 for uint64, int32 for uint32); the bits are what the library reads and writes.

torch is imported before libgsr.so is loaded, so the library binds to the HIP runtime torch already loaded and the
two share devices, allocations and streams. If the library is missing the import fails: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgsr.so")

GSR_OK, GSR_EINVAL, GSR_ENOMEM, GSR_EHIP, GSR_EOVERFLOW = 0, -1, -2, -3, -4
GSR_OPT_BIN_SCHEME, GSR_BIN_PRESORT, GSR_BIN_KEY64, GSR_OPT_BIN_KEYS, GSR_OPT_RASTER_SKIP = 1, 0, 1, 2, 3
GSR_OPT_BIN_RULE, GSR_BIN_BOX, GSR_BIN_ELLIPSE = 4, 0, 1
GSR_OPT_DETERMINISTIC = 5
GSR_OPT_KERNEL_TIMING = 6
GSR_OPT_BACKWARD_SCHEME, GSR_BACKWARD_PER_PIXEL, GSR_BACKWARD_PER_SPLAT = 7, 0, 1
GSR_OPT_ARENA_LIMIT = 8
GSR_OPT_TILE_ORDER, GSR_ORDER_COST, GSR_ORDER_LENGTH, GSR_ORDER_NONE = 9, 0, 1, 2
GSR_OPT_BIN_SYNC_FREE = 10
GSR_BIN_TILE_DEPTH = 2
GSR_OPT_FORWARD_EXP, GSR_EXP_EXACT, GSR_EXP_FAST = 11, 0, 1
(GSR_STAGE_BIN, GSR_STAGE_FORWARD, GSR_STAGE_BACKWARD, GSR_STAGE_ADAM, GSR_STAGE_PROJECT_FORWARD,
 GSR_STAGE_PROJECT_BACKWARD, GSR_STAGE_LOSS, GSR_STAGE_DEPTH_SORT, GSR_STAGE_TILE_SORT, GSR_STAGE_TILE_DEPTH,
 GSR_STAGE_TILE_SCAN) = range(11)
GSR_ADAM_MAX_GROUPS = 8
_STATUS = {GSR_EINVAL: "GSR_EINVAL", GSR_ENOMEM: "GSR_ENOMEM", GSR_EHIP: "GSR_EHIP", GSR_EOVERFLOW: "GSR_EOVERFLOW"}


class GsrError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class gsr_bins(ctypes.Structure):
    _fields_ = [("keys", ctypes.c_void_p), ("vals", ctypes.c_void_p), ("ranges", ctypes.c_void_p),
                ("num_pairs", ctypes.c_uint32), ("tiles_x", ctypes.c_uint32), ("tiles_y", ctypes.c_uint32),
                ("splat_pairs", ctypes.c_void_p), ("num_splats", ctypes.c_uint32)]


class gsr_adam_group(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("m", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("count", ctypes.c_uint64), ("lr", ctypes.c_float)]


class gsr_camera(ctypes.Structure):
    _fields_ = [("R", ctypes.c_float * 9), ("tv", ctypes.c_float * 3), ("fx", ctypes.c_float),
                ("fy", ctypes.c_float), ("cx", ctypes.c_float), ("cy", ctypes.c_float), ("near", ctypes.c_float)]


def camera(R, tv, fx: float, fy: float, cx: float, cy: float, near: float = 0.01) -> gsr_camera:
    """A gsr_camera from a 3x3 world-to-camera rotation R (any nested sequence or array), a translation tv and the
    pinhole intrinsics."""
    flat = [float(v) for row in R for v in row]
    return gsr_camera((ctypes.c_float * 9)(*flat), (ctypes.c_float * 3)(*[float(v) for v in tv]), fx, fy, cx, cy,
                      near)


# Every symbol include/gsr.h declares, with its ctypes signature.
_P, _U32, _U64, _I32, _I64, _F = (ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int32,
                                  ctypes.c_int64, ctypes.c_float)
SIGNATURES = {
    "gsr_create": (_I32, [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]),
    "gsr_destroy": (None, [_P]),
    "gsr_last_error": (ctypes.c_char_p, [_P]),
    "gsr_reserve": (_I32, [_P, _U64, _U32]),
    "gsr_set_option": (_I32, [_P, _I32, _I64]),
    "gsr_bin": (_I32, [_P, _P, _P, _P, _U32, _U32, _U32, ctypes.POINTER(gsr_bins)]),
    "gsr_bin_pair_count": (_I32, [_P, ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_int32)]),
    "gsr_bins_copy": (_I32, [_P, _P, ctypes.POINTER(gsr_bins), _P, _P, _P, _P]),
    "gsr_radix_sort": (_I32, [_P, _P, _P, _P, _U64, _U32, _P, _P]),
    "gsr_radix_pass_count": (_U32, [_U64, _U32]),
    "gsr_render_forward": (_I32, [_P, _P, _P, _U32, ctypes.POINTER(gsr_bins), _U32, _U32, _P, _P, _P]),
    "gsr_render_forward_noalloc": (_I32, [_P, _P, _P, _U32, ctypes.POINTER(gsr_bins), _U32, _U32, _P, _P, _P]),
    "gsr_render_backward": (_I32, [_P, _P, _P, _U32, ctypes.POINTER(gsr_bins), _U32, _U32, _P, _P, _P, _P, _P]),
    "gsr_adam_step": (_I32, [_P, _P, ctypes.POINTER(gsr_adam_group), _U32, _F, _F, _F, _F, _F]),
    "gsr_kernel_times": (_I32, [_P, _I32, _P, _U32, _P]),
    "gsr_adam_step_visible": (_I32, [_P, _P, ctypes.POINTER(gsr_adam_group), _U32, _F, _F, _F, _F, _F, _P, _U32]),
    "gsr_project_forward": (_I32, [_P, _P, ctypes.POINTER(gsr_camera), _U32, _P, _P, _P, _P, _P, _P, _P]),
    "gsr_project_backward": (_I32, [_P, _P, ctypes.POINTER(gsr_camera), _U32, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                    _P, _P]),
    "gsr_loss_l1_ssim": (_I32, [_P, _P, _U32, _U32, _P, _P, _P, _P]),
}

_lib = None


def load():
    """Loads libgsr.so (in-tree build) and declares its signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built: run python -m differentiable_gaussian_splatting_amd.build")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtypes, numel=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype {dtypes}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, has {t.numel()}")


class Context:
    """Owns a gsr_ctx (and its device arena) on one device."""

    def __init__(self, device: int | torch.device = 0):
        lib = load()
        self.device = torch.device("cuda", device if isinstance(device, int) else device.index or 0)
        h = ctypes.c_void_p()
        st = lib.gsr_create(ctypes.byref(h), self.device.index)
        if st != GSR_OK:
            raise GsrError(st, f"gsr_create(device {self.device.index}) failed")
        self.handle = h

    def check(self, st: int, what: str):
        if st != GSR_OK:
            msg = load().gsr_last_error(self.handle)
            raise GsrError(st, f"{what}: {msg.decode() if msg else ''}")

    def close(self):
        if getattr(self, "handle", None):
            load().gsr_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Bins:
    """A gsr_bins view plus references to whatever owns its memory."""

    def __init__(self, raw: gsr_bins, owners=()):
        self.raw = raw
        self._owners = owners

    num_pairs = property(lambda self: int(self.raw.num_pairs))
    tiles_x = property(lambda self: int(self.raw.tiles_x))
    tiles_y = property(lambda self: int(self.raw.tiles_y))


def gsr_create(device=0) -> Context:
    return Context(device)


def gsr_destroy(ctx: Context):
    ctx.close()


def gsr_reserve(ctx: Context, max_pairs: int, max_splats: int):
    ctx.check(load().gsr_reserve(ctx.handle, max_pairs, max_splats), "gsr_reserve")


def gsr_set_option(ctx: Context, option: int, value: int):
    ctx.check(load().gsr_set_option(ctx.handle, option, value), "gsr_set_option")


def gsr_kernel_times(ctx: Context, stage: int, max_count: int = 4096) -> list:
    """GPU milliseconds of the last recorded launches of `stage` (GSR_OPT_KERNEL_TIMING on), oldest first."""
    buf = (ctypes.c_float * max(1, max_count))()
    count = ctypes.c_uint32(0)
    ctx.check(load().gsr_kernel_times(ctx.handle, stage, buf, max_count, ctypes.byref(count)), "gsr_kernel_times")
    return [float(buf[i]) for i in range(count.value)]


def gsr_radix_pass_count(num_tiles: int, digit_bits: int) -> int:
    return int(load().gsr_radix_pass_count(num_tiles, digit_bits))


def gsr_bin(ctx: Context, splats: torch.Tensor, depths: torch.Tensor, width: int, height: int,
            stream=None) -> Bins:
    n = depths.numel()
    _need(splats, "splats", (torch.float32,), n * 9, ctx.device)
    _need(depths, "depths", (torch.float32,), n, ctx.device)
    raw = gsr_bins()
    ctx.check(load().gsr_bin(ctx.handle, _stream(stream), _ptr(splats), _ptr(depths), n, width, height,
                             ctypes.byref(raw)), "gsr_bin")
    return Bins(raw, (ctx,))


def gsr_bin_pair_count(ctx: Context) -> tuple[int, bool]:
    """(pairs, overflowed) of the context's last gsr_bin, waiting for the count if that call did not."""
    pairs, over = ctypes.c_uint64(0), ctypes.c_int32(0)
    ctx.check(load().gsr_bin_pair_count(ctx.handle, ctypes.byref(pairs), ctypes.byref(over)), "gsr_bin_pair_count")
    return int(pairs.value), bool(over.value)


def bins_from_tensors(keys: torch.Tensor | None, vals: torch.Tensor, ranges: torch.Tensor, width: int,
                      height: int) -> Bins:
    """A gsr_bins view over caller tensors: keys int64 [P] (may be None), vals int32 [P], ranges int32 [T, 2]."""
    tx, ty = (width + 15) // 16, (height + 15) // 16
    _need(vals, "vals", (torch.int32,))
    _need(ranges, "ranges", (torch.int32,), 2 * tx * ty)
    if keys is not None:
        _need(keys, "keys", (torch.int64,), vals.numel())
    raw = gsr_bins(_ptr(keys), _ptr(vals), _ptr(ranges), vals.numel(), tx, ty, None, 0)
    return Bins(raw, (keys, vals, ranges))


def gsr_bins_copy(ctx: Context, bins: Bins, stream=None):
    """Copies a bins view into new tensors: keys int64 [P] (None if the bins carry none; empty when P = 0, where the
    library may leave the pointers NULL), vals int32 [P], ranges int32 [T, 2]."""
    P, T = bins.num_pairs, bins.tiles_x * bins.tiles_y
    dev = ctx.device
    keys = torch.empty(P, dtype=torch.int64, device=dev) if (bins.raw.keys or P == 0) else None
    vals = torch.empty(P, dtype=torch.int32, device=dev)
    ranges = torch.empty((T, 2), dtype=torch.int32, device=dev)
    ctx.check(load().gsr_bins_copy(ctx.handle, _stream(stream), ctypes.byref(bins.raw),
                                   _ptr(keys) if P else None, _ptr(vals) if P else None, _ptr(ranges), None),
              "gsr_bins_copy")
    return keys, vals, ranges


def gsr_bins_splat_pairs(ctx: Context, bins: Bins, stream=None) -> torch.Tensor:
    """The number of pairs each splat emitted, copied into a new int32 tensor [num_splats]."""
    out = torch.empty(int(bins.raw.num_splats), dtype=torch.int32, device=ctx.device)
    ctx.check(load().gsr_bins_copy(ctx.handle, _stream(stream), ctypes.byref(bins.raw), None, None, None,
                                   _ptr(out)), "gsr_bins_copy")
    return out


def gsr_radix_sort(ctx: Context, keys: torch.Tensor, vals: torch.Tensor, key_bits: int = 64, stream=None):
    n = keys.numel()
    _need(keys, "keys", (torch.int64,), n, ctx.device)
    _need(vals, "vals", (torch.int32,), n, ctx.device)
    ko = torch.empty_like(keys)
    vo = torch.empty_like(vals)
    ctx.check(load().gsr_radix_sort(ctx.handle, _stream(stream), _ptr(keys), _ptr(vals), n, key_bits, _ptr(ko),
                                    _ptr(vo)), "gsr_radix_sort")
    return ko, vo


def gsr_render_forward(ctx: Context, splats: torch.Tensor, bins: Bins, width: int, height: int,
                       out_rgba: torch.Tensor | None = None, final_T: torch.Tensor | None = None,
                       last_contrib: torch.Tensor | None = None, stream=None):
    """Returns (out_rgba float32 [H, W, 4], final_T float32 [H, W], last_contrib int32 [H, W])."""
    dev = ctx.device
    n = splats.numel() // 9
    _need(splats, "splats", (torch.float32,), n * 9, dev)
    if out_rgba is None:
        out_rgba = torch.empty((height, width, 4), dtype=torch.float32, device=dev)
    if final_T is None:
        final_T = torch.empty((height, width), dtype=torch.float32, device=dev)
    if last_contrib is None:
        last_contrib = torch.empty((height, width), dtype=torch.int32, device=dev)
    _need(out_rgba, "out_rgba", (torch.float32,), height * width * 4, dev)
    _need(final_T, "final_T", (torch.float32,), height * width, dev)
    _need(last_contrib, "last_contrib", (torch.int32,), height * width, dev)
    ctx.check(load().gsr_render_forward(ctx.handle, _stream(stream), _ptr(splats), n, ctypes.byref(bins.raw), width,
                                        height, _ptr(out_rgba), _ptr(final_T), _ptr(last_contrib)),
              "gsr_render_forward")
    return out_rgba, final_T, last_contrib


def gsr_render_forward_noalloc(ctx: Context, splats: torch.Tensor, bins: Bins, width: int, height: int,
                               out_rgba: torch.Tensor, final_T: torch.Tensor, last_contrib: torch.Tensor,
                               stream=None):
    """gsr_render_forward into caller-given outputs, with no device allocation by the library (its scratch is a
    fixed per-device array; at most 65536 tiles)."""
    dev = ctx.device
    n = splats.numel() // 9
    _need(splats, "splats", (torch.float32,), n * 9, dev)
    _need(out_rgba, "out_rgba", (torch.float32,), height * width * 4, dev)
    _need(final_T, "final_T", (torch.float32,), height * width, dev)
    _need(last_contrib, "last_contrib", (torch.int32,), height * width, dev)
    ctx.check(load().gsr_render_forward_noalloc(ctx.handle, _stream(stream), _ptr(splats), n, ctypes.byref(bins.raw),
                                                width, height, _ptr(out_rgba), _ptr(final_T), _ptr(last_contrib)),
              "gsr_render_forward_noalloc")
    return out_rgba, final_T, last_contrib


def gsr_render_backward(ctx: Context, splats: torch.Tensor, bins: Bins, width: int, height: int,
                        out_rgba: torch.Tensor, final_T: torch.Tensor, last_contrib: torch.Tensor,
                        v_out: torch.Tensor, splats_grad: torch.Tensor | None = None, stream=None):
    """Returns splats_grad float32 [N, 9]."""
    dev = ctx.device
    n = splats.numel() // 9
    _need(splats, "splats", (torch.float32,), n * 9, dev)
    _need(out_rgba, "out_rgba", (torch.float32,), height * width * 4, dev)
    _need(final_T, "final_T", (torch.float32,), height * width, dev)
    _need(last_contrib, "last_contrib", (torch.int32,), height * width, dev)
    _need(v_out, "v_out", (torch.float32,), height * width * 4, dev)
    if splats_grad is None:
        splats_grad = torch.empty((n, 9), dtype=torch.float32, device=dev)
    _need(splats_grad, "splats_grad", (torch.float32,), n * 9, dev)
    ctx.check(load().gsr_render_backward(ctx.handle, _stream(stream), _ptr(splats), n, ctypes.byref(bins.raw), width,
                                         height, _ptr(out_rgba), _ptr(final_T), _ptr(last_contrib), _ptr(v_out),
                                         _ptr(splats_grad)), "gsr_render_backward")
    return splats_grad


def gsr_adam_step(ctx: Context, groups, beta1: float, beta2: float, eps: float, bc1: float, bc2: float,
                  stream=None):
    """groups: sequence of (param, grad, m, v, lr) float32 device tensors of equal sizes; updated in place."""
    arr = _adam_groups(ctx, groups)
    ctx.check(load().gsr_adam_step(ctx.handle, _stream(stream), arr, len(groups), beta1, beta2, eps, bc1, bc2),
              "gsr_adam_step")


def gsr_adam_step_visible(ctx: Context, groups, beta1: float, beta2: float, eps: float, bc1: float, bc2: float,
                          visible, n: int | None = None, stream=None):
    """gsr_adam_step for the splats with a non-zero entry in `visible` only: a Bins (its splat_pairs, with n given)
    or an int32 device tensor [n]. Each group holds n splats' elements, consecutive per splat."""
    if isinstance(visible, Bins):
        if n is None:
            raise ValueError("n is needed with a Bins")
        ptr = visible.raw.splat_pairs if n else None
        if n and not ptr:
            raise ValueError("these bins carry no splat_pairs")
    else:
        n = visible.numel() if n is None else n
        _need(visible, "visible", (torch.int32,), n, ctx.device)
        ptr = _ptr(visible)
    arr = _adam_groups(ctx, groups)
    ctx.check(load().gsr_adam_step_visible(ctx.handle, _stream(stream), arr, len(groups), beta1, beta2, eps, bc1,
                                           bc2, ptr, n), "gsr_adam_step_visible")


def _adam_groups(ctx: Context, groups):
    if len(groups) > GSR_ADAM_MAX_GROUPS:
        raise ValueError(f"at most {GSR_ADAM_MAX_GROUPS} groups")
    arr = (gsr_adam_group * max(1, len(groups)))()
    for q, (p, g, m, v, lr) in enumerate(groups):
        k = p.numel()
        for t, name in ((p, "param"), (g, "grad"), (m, "m"), (v, "v")):
            _need(t, f"group {q} {name}", (torch.float32,), k, ctx.device)
        arr[q] = gsr_adam_group(_ptr(p), _ptr(g), _ptr(m), _ptr(v), k, lr)
    return arr


_PARAM_WIDTHS = (("means", 3), ("log_scales", 3), ("quats", 4), ("raw_opacities", 1), ("sh", 48))


def _need_params(ctx: Context, params):
    n = params[0].numel() // 3
    for t, (name, k) in zip(params, _PARAM_WIDTHS):
        _need(t, name, (torch.float32,), n * k, ctx.device)
    return n


def gsr_project_forward(ctx: Context, cam: gsr_camera, means, log_scales, quats, raw_opacities, sh,
                        splats: torch.Tensor | None = None, depths: torch.Tensor | None = None, stream=None):
    """Returns (splats float32 [N, 9], depths float32 [N]) of the Gaussians (float32 device tensors: means [N, 3],
    log_scales [N, 3], quats [N, 4], raw_opacities [N], sh [N, 16, 3])."""
    params = (means, log_scales, quats, raw_opacities, sh)
    n = _need_params(ctx, params)
    dev = ctx.device
    if splats is None:
        splats = torch.empty((n, 9), dtype=torch.float32, device=dev)
    if depths is None:
        depths = torch.empty(n, dtype=torch.float32, device=dev)
    _need(splats, "splats", (torch.float32,), n * 9, dev)
    _need(depths, "depths", (torch.float32,), n, dev)
    ctx.check(load().gsr_project_forward(ctx.handle, _stream(stream), ctypes.byref(cam), n,
                                         *[_ptr(t) for t in params], _ptr(splats), _ptr(depths)),
              "gsr_project_forward")
    return splats, depths


def gsr_project_backward(ctx: Context, cam: gsr_camera, means, log_scales, quats, raw_opacities, sh,
                         splats_grad: torch.Tensor, grads=None, stream=None):
    """Returns the gradients (means, log_scales, quats, raw_opacities, sh), each shaped like its parameter."""
    params = (means, log_scales, quats, raw_opacities, sh)
    n = _need_params(ctx, params)
    _need(splats_grad, "splats_grad", (torch.float32,), n * 9, ctx.device)
    if grads is None:
        grads = tuple(torch.empty_like(t) for t in params)
    for t, g, (name, k) in zip(params, grads, _PARAM_WIDTHS):
        _need(g, name + "_grad", (torch.float32,), n * k, ctx.device)
    ctx.check(load().gsr_project_backward(ctx.handle, _stream(stream), ctypes.byref(cam), n,
                                          *[_ptr(t) for t in params], _ptr(splats_grad), *[_ptr(g) for g in grads]),
              "gsr_project_backward")
    return grads


def gsr_loss_l1_ssim(ctx: Context, out_rgba: torch.Tensor, target: torch.Tensor, v_out: torch.Tensor | None = None,
                     loss: torch.Tensor | None = None, stream=None):
    """L1 + SSIM of out_rgba [H, W, 4] (its rgb) against target [H, W, 3]. Returns (v_out float32 [H, W, 4],
    loss float32 [3] = (L, mean|x - y|, mean SSIM)), both on the device."""
    dev = ctx.device
    H, W = out_rgba.shape[0], out_rgba.shape[1]
    _need(out_rgba, "out_rgba", (torch.float32,), H * W * 4, dev)
    _need(target, "target", (torch.float32,), H * W * 3, dev)
    if v_out is None:
        v_out = torch.empty((H, W, 4), dtype=torch.float32, device=dev)
    if loss is None:
        loss = torch.empty(3, dtype=torch.float32, device=dev)
    _need(v_out, "v_out", (torch.float32,), H * W * 4, dev)
    _need(loss, "loss", (torch.float32,), 3, dev)
    ctx.check(load().gsr_loss_l1_ssim(ctx.handle, _stream(stream), W, H, _ptr(out_rgba), _ptr(target), _ptr(v_out),
                                      _ptr(loss)), "gsr_loss_l1_ssim")
    return v_out, loss
