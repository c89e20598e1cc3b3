"""Host-side preparation of the decode-shape workloads.

Draws the seeded synthetic weights and activations (synth.py), compresses the
weights with the library's host quantizer and, for NVFP4, packs them.  The
result is host arrays; callers move them to the device.
"""

import numpy as np

from . import nvfp4_quantize, fp8_quantize, nvfp4_pack, nvfp4_pack_swiglu, synth


def nvfp4_case(M, K, N, seed=0):
    """dict(codes, scales, g, blob, x) for an NVFP4 GEMM of shape (M, K, N)."""
    rng = np.random.default_rng(seed)
    w = synth.draw_weights(rng, K, N)
    x = synth.draw_activations(rng, M, K)
    codes, scales, g = nvfp4_quantize(w)
    del w
    blob = nvfp4_pack(codes, scales, g, K, N)
    return {"fmt": "nvfp4", "M": M, "K": K, "N": N, "codes": codes, "scales": scales, "g": g,
            "blob": blob, "x": x, "weight_bytes": codes.nbytes + scales.nbytes + 4}


def swiglu_case(M, K, F, seed=0):
    """dict for a SwiGLU pair: the fused gate+up weight [K, 2F] is drawn as for
    nvfp4_case(M, K, 2F, seed); its first F columns are the gate projection and
    the last F the up projection, each quantized with its own per-tensor scale."""
    rng = np.random.default_rng(seed)
    w = synth.draw_weights(rng, K, 2 * F)
    x = synth.draw_activations(rng, M, K)
    gate = nvfp4_quantize(np.ascontiguousarray(w[:, :F]))
    up = nvfp4_quantize(np.ascontiguousarray(w[:, F:]))
    del w
    blob = nvfp4_pack_swiglu(gate, up, K, F)
    nbytes = sum(a.nbytes for a in gate[:2] + up[:2]) + 8
    return {"fmt": "swiglu", "M": M, "K": K, "F": F, "gate": gate, "up": up, "blob": blob, "x": x,
            "weight_bytes": nbytes}


def fp8_case(M, K, N, seed=0):
    """dict(codes, scales, x) for an FP8 GEMM of shape (M, K, N)."""
    rng = np.random.default_rng(seed)
    w = synth.draw_weights(rng, K, N)
    x = synth.draw_activations(rng, M, K)
    codes, scales = fp8_quantize(w)
    del w
    return {"fmt": "fp8", "M": M, "K": K, "N": N, "codes": codes, "scales": scales, "x": x,
            "weight_bytes": codes.nbytes + scales.nbytes}


def named_case(name, M=None, seed=0):
    """One of synth.WORKLOADS at full size; M defaults to the largest M listed.

    Smaller M of the same workload are the leading rows of x (the activations
    are drawn after the weights from the same stream, row by row)."""
    fmt, ms, K, N = synth.WORKLOADS[name]
    M = max(ms) if M is None else M
    return (nvfp4_case if fmt == "nvfp4" else fp8_case)(M, K, N, seed)
