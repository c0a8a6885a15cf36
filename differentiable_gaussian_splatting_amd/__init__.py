"""MI355X-native tile-based differentiable 2D-splat rasterizer: binning, forward, backward and fused Adam.

The compute lives in libgsr.so (hand-written HIP for gfx950 behind a C ABI, declared in include/gsr.h). The `gsr`
submodule is its thin ctypes binding; `scenes` draws seeded synthetic inputs. Importing this package loads neither.
"""
__all__ = ["gsr", "scenes"]
