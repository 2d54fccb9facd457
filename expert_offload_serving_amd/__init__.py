"""MI355X (gfx950) NVFP4 routed-MoE layer with an HBM expert cache.

The compute lives in libmoe_nvfp4.so (hand-written HIP kernels, C ABI in
include/moe_nvfp4.h); `_lib` binds it with ctypes and `layer` adds torch
allocation helpers.  `synth` makes seeded synthetic inputs.
"""
from ._lib import LIB_PATH, MoeError, lib  # noqa: F401

__all__ = ["LIB_PATH", "MoeError", "lib"]
