"""The computation the hot path performs, written as its plain definition.

ORACLE -- test infrastructure only (tests, smoke check, CPU-baseline leg of the
benchmark).  It reads only the canonical compressed arrays and shares no code
with the library.

What is computed (author's post, section "What I actually built": the weights are
read from HBM still compressed and every fragment is turned into fp16 operands
on the fly, with no dequantize-the-model pass; the 8-row tile serves the target
token plus k=7 drafts, post section on why M=8 matters):

  y[m, n]  = sum_k x[m, k] * W~[k, n]                 (float64 here)
  NVFP4:  W~[k, n] = E2M1(q[n, k]) * E4M3(s[n, k//16]) * g
  FP8:    W~[k, n] = E4M3(c[n, k]) * S[n//128, k//128]
  argmax: idx[m] = smallest n with y[m, n] == max over the non-NaN y[m, n'],
          -1 if every y[m, n] is NaN
          (the drafter should propose greedy / local-argmax tokens: post,
           section "This is a server, not a GEMM screenshot"; a NaN logit is
           no token's score, so it never wins)

The method reaches this exact result up to the order of floating-point sums,
so the oracle is the definition: decode, widen to float64, one matmul.
"""

import numpy as np

from .formats import e2m1_decode, e4m3_decode


def nvfp4_unpack_codes(codes, K):
    """codes [N][K/2] u8 -> nibble codes [N][K] (low nibble = even k)."""
    codes = np.asarray(codes, dtype=np.uint8)
    q = np.empty((codes.shape[0], K), np.uint8)
    q[:, 0::2] = codes & 15
    q[:, 1::2] = codes >> 4
    return q


def nvfp4_dequant_unscaled(codes, scales, K, cols=None):
    """E2M1(q) * E4M3(s) as float64 [K, n_cols] -- the weights before the global scale g.

    This product is what the kernels must reproduce exactly (it has at most 6
    significant bits and lies in [2^-10, 2688], so fp16 and fp32 hold it exactly).
    """
    codes = np.asarray(codes)
    scales = np.asarray(scales)
    if cols is not None:
        codes = codes[cols]
        scales = scales[cols]
    q = e2m1_decode(nvfp4_unpack_codes(codes, K))                # [n][K]
    s = np.repeat(e4m3_decode(scales), 16, axis=1)               # [n][K]
    return (q * s).T


def nvfp4_gemm(x, codes, scales, g, cols=None, chunk=1024):
    """y = x @ (E2M1(q) * E4M3(s) * g) in float64.  x: [M, K] (fp16 values).

    cols: optional array of output columns to compute (others are skipped).
    Columns are processed `chunk` at a time to bound memory."""
    x64 = np.asarray(x).astype(np.float64)
    K = x64.shape[1]
    n_all = np.asarray(codes).shape[0] if cols is None else len(cols)
    col_ids = np.arange(n_all) if cols is None else np.asarray(cols)
    y = np.empty((x64.shape[0], n_all), np.float64)
    for c0 in range(0, n_all, chunk):
        sel = col_ids[c0:c0 + chunk]
        deq = nvfp4_dequant_unscaled(codes, scales, K, cols=sel)
        y[:, c0:c0 + len(sel)] = (x64 @ deq) * np.float64(g)
    return y


def fp8_dequant(codes, scales, cols=None):
    """E4M3(c) * S as float64 [K, n_cols]."""
    codes = np.asarray(codes)
    scales = np.asarray(scales, dtype=np.float32).astype(np.float64)
    col_ids = np.arange(codes.shape[0]) if cols is None else np.asarray(cols)
    c = e4m3_decode(codes[col_ids])                               # [n][K]
    K = c.shape[1]
    S = scales[col_ids // 128][:, np.arange(K) // 128]            # [n][K]
    return (c * S).T


def fp8_gemm(x, codes, scales, cols=None, chunk=1024):
    """y = x @ (E4M3(c) * S) in float64."""
    x64 = np.asarray(x).astype(np.float64)
    n_all = np.asarray(codes).shape[0] if cols is None else len(cols)
    col_ids = np.arange(n_all) if cols is None else np.asarray(cols)
    y = np.empty((x64.shape[0], n_all), np.float64)
    for c0 in range(0, n_all, chunk):
        sel = col_ids[c0:c0 + chunk]
        y[:, c0:c0 + len(sel)] = x64 @ fp8_dequant(codes, scales, cols=sel)
    return y


def silu(z):
    """SiLU (sigmoid-weighted linear unit), z * sigmoid(z), in float64.

    The activation of the gated MLP that follows a fused gate+up projection
    (SwiGLU: Shazeer, "GLU Variants Improve Transformer", 2020, with the
    SiLU of Elfwing, Uchibe and Doya, 2018).  Written as z / (1 + exp(-z));
    exp overflows to inf for z below about -709, which gives the correct
    limit -0."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def nvfp4_swiglu(x, gate, up, cols=None, chunk=1024):
    """h = silu(x @ Wg~) * (x @ Wu~) in float64.

    gate, up: (codes [F][K/2], scales [F][K/16], g) -- two NVFP4 weights of
    the same shape, each with its own per-tensor scale.  The GEMMs are the
    plain definitions above; the activation acts on the exact (float64)
    projections, since the kernels apply it to their fp32 sums before any
    rounding to fp16."""
    yg = nvfp4_gemm(x, gate[0], gate[1], gate[2], cols=cols, chunk=chunk)
    yu = nvfp4_gemm(x, up[0], up[1], up[2], cols=cols, chunk=chunk)
    return silu(yg) * yu


def argmax_rows(y):
    """Per-row greedy token: the lowest index holding the largest logit; plus the normalised margin.

    NaN logits never win: the maximum is taken over the logits that are
    numbers (+-inf included), and the index is the first column equal to it.
    A row with no number at all (every logit NaN) has no greedy token: -1.

    margin[m] = (top1 - top2) / RMS of row m, both over its non-NaN logits --
    how far the winner is ahead (NaN where fewer than two logits are numbers)."""
    y = np.asarray(y, dtype=np.float64)
    M = y.shape[0]
    idx = np.full(M, -1, np.int64)
    margin = np.full(M, np.nan)
    for m in range(M):
        row = y[m]
        numbers = row[~np.isnan(row)]
        if numbers.size == 0:
            continue
        top = numbers.max()
        idx[m] = np.flatnonzero(row == top)[0]
        if numbers.size > 1:
            second = np.partition(numbers, -2)[-2]
            with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
                margin[m] = (top - second) / np.sqrt(np.mean(numbers * numbers))
    return idx, margin


def compare(y_test, y_ref):
    """Error metrics of a GEMM result against the float64 definition.

    rel_frob = ||y_test - y_ref||_F / ||y_ref||_F  (whole M x N)
    row_max  = max over rows of  max_n |y_test - y_ref| / RMS_n(y_ref[m, :])"""
    a = np.asarray(y_test, dtype=np.float64)
    b = np.asarray(y_ref, dtype=np.float64)
    diff = a - b
    nb = np.linalg.norm(b)
    rel_frob = np.linalg.norm(diff) / nb if nb > 0 else float(np.linalg.norm(diff))
    rms = np.sqrt(np.mean(b * b, axis=1))
    with np.errstate(divide="ignore", invalid="ignore"):
        row = np.where(rms > 0, np.abs(diff).max(axis=1) / rms, np.abs(diff).max(axis=1))
    return {"rel_frob": float(rel_frob), "row_max": float(row.max()) if row.size else 0.0}
