"""Plain quantizers that turn float32 weights into the compressed formats.

ORACLE -- test infrastructure only (tests, smoke check, CPU-baseline leg of the
benchmark).  The library has its own host quantizer; the tests require its
output to equal these functions' output byte for byte.

The pages serve checkpoints that were quantized offline (ai-manual article,
section "NVFP4 model conversion": the FP16 model is converted to NVFP4 by a
script; the author's post, section "v1.0 -> v1.1": published FP4 regions stay
FP4 and published FP8 regions stay FP8).  They do not print the rule, so the
standard two-level NVFP4 recipe and the 128x128 block FP8 recipe are used:

NVFP4 (per tensor W[K, N], K-blocks of 16 elements of one output column n):
  g      = fp32(amax(|W|) / (6 * 448))                   per-tensor scale
  t      = (blk_amax / 6) / g            (float64)       per-block target
  s_code = E4M3(t),  s = value(s_code)
  q      = E2M1(W / (s * g))             (float64 ratio; all codes 0 if s == 0)
  W~     = value(q) * s * g
  amax == 0 gives g = 0 and all-zero scales and codes.

FP8 (per 128x128 block of W, K-rows kb*128.., columns nb*128..):
  S      = fp32(blk_amax / 448)
  c      = E4M3(W / S)                   (float64 ratio; all codes 0 if S == 0)
  W~     = value(c) * S

Storage (output-major, the order the GEMM streams it):
  NVFP4 codes  uint8 [N][K/2]   byte j of row n = code(k=2j) | code(k=2j+1) << 4
  NVFP4 scales uint8 [N][K/16]  E4M3FN
  FP8 codes    uint8 [N][K]     E4M3FN
  FP8 scales   fp32  [ceil(N/128)][ceil(K/128)]
"""

import numpy as np

from .formats import e2m1_encode, e4m3_encode, e4m3_decode, E2M1_MAX, E4M3_MAX


def nvfp4_global_scale(w):
    """The per-tensor scale g = fp32(amax(|W|) / (6 * 448)) of float32 W."""
    w = np.asarray(w, dtype=np.float32)
    amax = float(np.abs(w).max()) if w.size else 0.0      # |float32| is exact in float64
    return np.float32(amax / (E2M1_MAX * E4M3_MAX))


def nvfp4_quantize(w, g=None):
    """w: float32 [K, N] (K % 16 == 0) -> (codes [N][K/2] u8, scales [N][K/16] u8, g float32).

    g: the per-tensor scale to quantize with; None computes it from w.  Every
    block depends only on its own 16 values and g, so a column slice of a
    tensor quantized with the whole tensor's g gives that slice of the whole
    tensor's codes and scales."""
    w = np.asarray(w, dtype=np.float32)
    K, N = w.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    wt = w.T.astype(np.float64)                      # [N][K], exact widening
    g = nvfp4_global_scale(w) if g is None else np.float32(g)
    if g == 0:
        return (np.zeros((N, K // 2), np.uint8), np.zeros((N, K // 16), np.uint8), np.float32(0.0))
    blocks = wt.reshape(N, K // 16, 16)
    blk_amax = np.abs(blocks).max(axis=2)            # [N][K/16]
    t = (blk_amax / E2M1_MAX) / np.float64(g)
    s_code = e4m3_encode(t)
    s = e4m3_decode(s_code)                          # >= 0
    denom = s * np.float64(g)                        # exact: <= 4 + 24 significant bits
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = blocks / denom[:, :, None]
    ratio = np.where(denom[:, :, None] == 0, 0.0, ratio)
    q = e2m1_encode(ratio).reshape(N, K)
    q = np.where(np.broadcast_to((denom == 0)[:, :, None], blocks.shape).reshape(N, K), 0, q).astype(np.uint8)
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    return codes, s_code.astype(np.uint8), g


def fp8_quantize(w):
    """w: float32 [K, N] -> (codes [N][K] u8 E4M3FN, scales fp32 [ceil(N/128)][ceil(K/128)])."""
    w = np.asarray(w, dtype=np.float32)
    K, N = w.shape
    KB, NB = -(-K // 128), -(-N // 128)
    wt = w.T.astype(np.float64)                      # [N][K]
    codes = np.zeros((N, K), np.uint8)
    scales = np.zeros((NB, KB), np.float32)
    for nb in range(NB):
        for kb in range(KB):
            blk = wt[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
            S = np.float32(np.abs(blk).max() / E4M3_MAX)
            scales[nb, kb] = S
            if S == 0:
                continue
            codes[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128] = e4m3_encode(blk / np.float64(S))
    return codes, scales
