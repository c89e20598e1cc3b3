"""ctypes loader for libskinny.so (built in-tree by build.py)."""

import ctypes
import os

from . import build as _build

_LIB = None

c_int, c_size_t, c_float, c_void_p = ctypes.c_int, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p
P = c_void_p


class SkinnyLayer(ctypes.Structure):
    """struct skinny_layer of skinny.h."""
    _fields_ = [("kind", c_int), ("weights", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("K", c_int), ("N", c_int)]


def _declare(lib):
    sig = {
        "nvfp4_pack": (c_int, [P, P, c_float, c_int, c_int, P, ctypes.POINTER(c_size_t)]),
        "nvfp4_gemm": (c_int, [P, P, P, c_int, c_int, c_int, P, c_size_t, P]),
        "nvfp4_gemm_config": (c_int, [P, P, P, c_int, c_int, c_int, P, c_size_t, P, c_int, c_int, c_int, c_int]),
        "nvfp4_gemm_noalloc": (c_int, [P, P, P, c_int, c_int, c_int, P]),
        "nvfp4_pack_swiglu": (c_int, [P, P, c_float, P, P, c_float, c_int, c_int, P, ctypes.POINTER(c_size_t)]),
        "nvfp4_gemm_swiglu": (c_int, [P, P, P, c_int, c_int, c_int, P, c_size_t, P]),
        "nvfp4_gemm_swiglu_config": (c_int, [P, P, P, c_int, c_int, c_int, P, c_size_t, P,
                                             c_int, c_int, c_int, c_int]),
        "fp8_gemm": (c_int, [P, P, P, P, c_int, c_int, c_int, P, c_size_t, P]),
        "fp8_gemm_config": (c_int, [P, P, P, P, c_int, c_int, c_int, P, c_size_t, P, c_int, c_int, c_int, c_int]),
        "fp8_pack": (c_int, [P, c_int, c_int, P, ctypes.POINTER(c_size_t)]),
        "fp8_gemm_packed": (c_int, [P, P, P, P, c_int, c_int, c_int, P, c_size_t, P]),
        "fp8_gemm_packed_config": (c_int, [P, P, P, P, c_int, c_int, c_int, P, c_size_t, P,
                                           c_int, c_int, c_int, c_int]),
        "lm_head_gemm_argmax": (c_int, [P, P, P, P, c_int, c_int, c_int, P, c_size_t, P]),
        "lm_head_verify_greedy": (c_int, [P, P, P, P, P, c_int, c_int, c_int, P, c_size_t, P]),
        "lm_head_verify_greedy_config": (c_int, [P, P, P, P, P, c_int, c_int, c_int, P, c_size_t, P,
                                                 c_int, c_int, c_int, c_int]),
        "lm_head_gemm_argmax_config": (c_int, [P, P, P, P, c_int, c_int, c_int, P, c_size_t, P,
                                               c_int, c_int, c_int, c_int]),
        "skinny_workspace_bytes_config": (c_size_t, [c_int] * 8),
        "skinny_config_supported": (c_int, [c_int] * 8),
        "skinny_default_config": (c_int, [c_int] * 4 + [ctypes.POINTER(c_int)] * 4),
        "skinny_read_probe": (c_int, [P, c_size_t, P, P]),
        "skinny_read_probe_pattern": (c_int, [P, c_size_t, c_int, c_int, c_int, P, ctypes.POINTER(c_size_t), P]),
        "nvfp4_quantize": (c_int, [P, c_int, c_int, P, P, ctypes.POINTER(c_float)]),
        "fp8_quantize": (c_int, [P, c_int, c_int, P, P]),
        "skinny_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int]),
        "skinny_strerror": (ctypes.c_char_p, [c_int]),
        "skinny_layers_workspace_bytes": (c_size_t, [ctypes.POINTER(SkinnyLayer), c_int, c_int]),
        "skinny_layers_run": (c_int, [ctypes.POINTER(SkinnyLayer), c_int, ctypes.POINTER(P), ctypes.POINTER(P),
                                      c_int, P, c_size_t, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


def lib():
    """The loaded library; it is built first only if no built copy exists.

    torch is imported first: PyTorch for ROCm ships its own HIP runtime
    (libamdhip64), and the library must bind to that same runtime, whose
    streams and device buffers the binding passes in.  Loaded before torch,
    the library would pull in the system's runtime, and its launches on
    torch's streams fail."""
    global _LIB
    if _LIB is None:
        try:
            import torch  # noqa: F401
        except ImportError:       # host-only use (packing, quantizing) without torch
            pass
        if not os.path.exists(_build.LIB):
            _build.build()
        _LIB = _declare(ctypes.CDLL(_build.LIB))
    return _LIB


EXPORTED = ("nvfp4_pack", "nvfp4_gemm", "fp8_gemm", "lm_head_gemm_argmax", "nvfp4_quantize",
            "fp8_quantize", "skinny_workspace_bytes", "skinny_strerror", "nvfp4_gemm_config",
            "fp8_gemm_config", "lm_head_gemm_argmax_config", "skinny_workspace_bytes_config",
            "skinny_config_supported", "skinny_read_probe", "nvfp4_pack_swiglu", "nvfp4_gemm_swiglu",
            "nvfp4_gemm_swiglu_config", "lm_head_verify_greedy", "lm_head_verify_greedy_config",
            "skinny_layers_workspace_bytes", "skinny_layers_run", "fp8_pack", "fp8_gemm_packed",
            "fp8_gemm_packed_config", "skinny_default_config", "nvfp4_gemm_noalloc",
            "skinny_read_probe_pattern")
