"""Shared helpers of the GPU parity tests: device transfer, per-scene oracle results (cached), case banners."""
from __future__ import annotations

import functools
import sys

import numpy as np

from differentiable_gaussian_splatting_amd import scenes


def banner(msg: str):
    """Names the case on stdout before a GPU step, so a run that ends abruptly still says what it was doing."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    elif a.dtype == np.uint64:
        a = a.view(np.int64)
    return torch.from_numpy(a).cuda()


def host(t, dtype=None):
    a = t.cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


@functools.lru_cache(maxsize=8)
def scene(name: str):
    return scenes.make_scene(name)


def custom_scene(**kw):
    return scenes.make_scene(scenes.SceneSpec(**kw))


@functools.lru_cache(maxsize=8)
def oracle_bins(name: str):
    import oracle
    sc = scene(name)
    return oracle.bin(sc.splats, sc.depths, sc.width, sc.height)


@functools.lru_cache(maxsize=4)
def oracle_forward(name: str):
    import oracle
    sc = scene(name)
    return oracle.render_forward(sc.splats, oracle_bins(name), sc.width, sc.height)


@functools.lru_cache(maxsize=4)
def oracle_backward(name: str):
    import oracle
    sc = scene(name)
    out, ft, lc, _ = oracle_forward(name)
    return oracle.render_backward(sc.splats, oracle_bins(name), sc.width, sc.height, out, ft, lc, sc.v_out)


def grads_close(gpu: np.ndarray, ref: np.ndarray, atol=1e-4, rtol=1e-4):
    """Dual tolerance |gpu - ref| <= atol + rtol |ref| element by element; returns (ok, worst ratio, argmax)."""
    ratio = np.abs(gpu.astype(np.float64) - ref) / (atol + rtol * np.abs(ref.astype(np.float64)))
    i = int(np.argmax(ratio)) if ratio.size else 0
    worst = float(ratio.reshape(-1)[i]) if ratio.size else 0.0
    return worst <= 1.0, worst, np.unravel_index(i, ratio.shape) if ratio.size else None


# Bar of the loss gradient (gsr_loss_l1_ssim's v_out) against the fp64 oracle, element by element: 2e-5 of the
# element plus 2e-5 of the largest element (the scale of the 121-term sums, for elements that cancel). The fp32
# kernel's worst measured error is about 6e-6 on these terms; a CPU test checks that the bar fails the oracle's own
# gradient under a wrong window size, window width, loss weight or SSIM constant.
LOSS_GRAD_REL = 2e-5


def loss_grad_bar(ref: np.ndarray) -> np.ndarray:
    ref = np.asarray(ref, np.float64)
    return LOSS_GRAD_REL * np.abs(ref[..., :3]) + LOSS_GRAD_REL * np.abs(ref).max()
