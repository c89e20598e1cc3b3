"""Full-size decode workloads quantized by the oracle, with whole-output references.

Test helper (no tests here).  The seeded float32 weights and fp16 activations
come from synth (random numbers only); the compressed weights come from the
oracle's quantizers, and the library's host quantizer is checked to give the
same bytes at the same full shape, so that parity on these inputs also covers
the inputs the benchmark times.  The library only packs the oracle's arrays.

The oracle is plain NumPy; at these sizes (up to 778 M weights) it runs on
column slices in a thread pool: NVFP4 blocks depend only on their own values
and the per-tensor scale, which is computed once from the whole tensor and
passed in (oracle.nvfp4_quantize(w, g=...), pinned to equal the one-shot
quantization); FP8 blocks are 128 x 128 and the slices are whole column
blocks.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
import fp8_quantized_skinny_amd as sk
from fp8_quantized_skinny_amd import synth

THREADS = max(1, min(16, os.cpu_count() or 1))
SLICE = 2048          # columns per slice (a multiple of 128)


def _pool_map(fn, items):
    with ThreadPoolExecutor(THREADS) as ex:
        return list(ex.map(fn, items))


def draw(M, K, N, seed=0):
    rng = np.random.default_rng(seed)
    w = synth.draw_weights(rng, K, N)
    x = synth.draw_activations(rng, M, K)
    return w, x


def nvfp4_quantize(w):
    """oracle.nvfp4_quantize of the whole float32 [K, N] tensor, computed slice by slice."""
    K, N = w.shape
    g = oracle.nvfp4_global_scale(w)
    parts = _pool_map(lambda c0: oracle.nvfp4_quantize(np.ascontiguousarray(w[:, c0:c0 + SLICE]), g=g),
                      range(0, N, SLICE))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]), g


def fp8_quantize(w):
    """oracle.fp8_quantize of the whole tensor, computed on slices of whole 128-column blocks."""
    K, N = w.shape
    parts = _pool_map(lambda c0: oracle.fp8_quantize(np.ascontiguousarray(w[:, c0:c0 + SLICE])),
                      range(0, N, SLICE))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def _column_slices(fn, N):
    parts = _pool_map(lambda c0: fn(np.arange(c0, min(N, c0 + SLICE))), range(0, N, SLICE))
    return np.concatenate(parts, axis=1)


def nvfp4_reference(x, codes, scales, g):
    """The oracle's float64 y = x . dequant(W) over every column."""
    return _column_slices(lambda cols: oracle.nvfp4_gemm(x, codes, scales, g, cols=cols), codes.shape[0])


def fp8_reference(x, codes, scales):
    return _column_slices(lambda cols: oracle.fp8_gemm(x, codes, scales, cols=cols), codes.shape[0])


def swiglu_reference(x, gate, up):
    return _column_slices(lambda cols: oracle.nvfp4_swiglu(x, gate, up, cols=cols), gate[0].shape[0])


def nvfp4_case(M, K, N, seed=0):
    """Oracle-quantized NVFP4 weights, the library's packed blob of them and x.

    Also asserts that the library's own quantizer gives the same bytes."""
    w, x = draw(M, K, N, seed)
    codes, scales, g = nvfp4_quantize(w)
    lc, ls, lg = sk.nvfp4_quantize(w)
    assert lg == g and np.array_equal(lc, codes) and np.array_equal(ls, scales), \
        f"library quantizer differs from the oracle's at {K} x {N}"
    del w, lc, ls
    return {"M": M, "K": K, "N": N, "codes": codes, "scales": scales, "g": g, "x": x,
            "blob": sk.nvfp4_pack(codes, scales, g, K, N)}


def swiglu_case(M, K, F, seed=0):
    """The fused [K, 2F] gate+up weight drawn as for nvfp4_case(M, K, 2F); gate = first F
    columns, up = last F, each with its own per-tensor scale."""
    w, x = draw(M, K, 2 * F, seed)
    gate = nvfp4_quantize(np.ascontiguousarray(w[:, :F]))
    up = nvfp4_quantize(np.ascontiguousarray(w[:, F:]))
    del w
    return {"M": M, "K": K, "F": F, "gate": gate, "up": up, "x": x, "blob": sk.nvfp4_pack_swiglu(gate, up, K, F)}


def fp8_case(M, K, N, seed=0):
    w, x = draw(M, K, N, seed)
    codes, scales = fp8_quantize(w)
    lc, ls = sk.fp8_quantize(w)
    assert np.array_equal(lc, codes) and np.array_equal(ls, scales), \
        f"library FP8 quantizer differs from the oracle's at {K} x {N}"
    del w, lc, ls
    return {"M": M, "K": K, "N": N, "codes": codes, "scales": scales, "x": x}
