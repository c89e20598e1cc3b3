"""Property-based pins of the oracle's encoders, quantizer and GEMM (hypothesis).

Each property follows from the definitions alone, not from the oracle's code:
  * round to nearest: no representable value is closer than the chosen one,
    and a tie goes to the code with an even mantissa;
  * the NVFP4 quantizer reconstructs every weight to within half the local
    E2M1 step times the block scale, and never flips a sign;
  * the GEMM is linear in x and in the per-tensor scale.
"""

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle

E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
finite = st.floats(min_value=-1e4, max_value=1e4, allow_nan=False, allow_infinity=False, width=64)


def _e4m3_grid():
    codes = np.arange(0x7F)                                    # positive finite codes 0 .. 126
    return oracle.e4m3_decode(codes.astype(np.uint8)).astype(np.float64)


@settings(max_examples=400, deadline=None)
@given(finite)
def test_e2m1_encode_is_nearest_with_even_ties(v):
    code = int(oracle.e2m1_encode(np.array([v]))[0])
    got = float(oracle.e2m1_decode(np.array([code], np.uint8))[0])
    a = min(abs(v), 6.0)                                       # saturation at 6
    err = abs(abs(got) - a)
    dists = np.abs(E2M1_VALUES - a)
    assert err <= dists.min() + 1e-15
    if np.sum(dists == dists.min()) > 1:                       # a tie: the even code (mantissa bit 0) wins
        assert (code & 1) == 0
    assert got == 0.0 or np.sign(got) == np.sign(v)


@settings(max_examples=400, deadline=None)
@given(st.floats(min_value=0.0, max_value=1000.0, allow_nan=False, width=64))
def test_e4m3_encode_is_nearest_with_even_ties(v):
    grid = _e4m3_grid()
    code = int(oracle.e4m3_encode(np.array([v]))[0])
    got = float(oracle.e4m3_decode(np.array([code], np.uint8))[0])
    a = min(v, 448.0)
    dists = np.abs(grid - a)
    assert abs(got - a) <= dists.min()
    if np.sum(dists == dists.min()) > 1:
        assert (code & 1) == 0


@settings(max_examples=60, deadline=None)
@given(st.integers(min_value=1, max_value=6), st.integers(min_value=1, max_value=5), st.integers(0, 2**31 - 1),
       st.floats(min_value=1e-3, max_value=1e3))
def test_nvfp4_quantizer_reconstruction_bound(nb, n, seed, scale):
    """|w - e2m1(q)·e4m3(s)·g| <= half the E2M1 step at |w|/(s·g), times s·g, and no sign flips."""
    K = 16 * nb
    w = (np.random.default_rng(seed).standard_normal((K, n)) * scale).astype(np.float32)
    codes, scales, g = oracle.nvfp4_quantize(w)
    deq = oracle.nvfp4_dequant_unscaled(codes, scales, K) * np.float64(g)      # [K, n]
    s = np.repeat(oracle.e4m3_decode(scales).astype(np.float64), 16, axis=1).T * np.float64(g)
    r = np.abs(w.astype(np.float64)) / s
    steps = np.diff(E2M1_VALUES)
    idx = np.clip(np.searchsorted(E2M1_VALUES, np.minimum(r, 6.0)) - 1, 0, len(steps) - 1)
    bound = 0.5 * steps[idx] * s * (1 + 1e-12)
    assert np.all(np.abs(deq - w) <= np.maximum(bound, np.abs(w) - 6.0 * s + 1e-300) + 1e-30)
    assert np.all((deq == 0) | (np.sign(deq) == np.sign(w)))


@settings(max_examples=40, deadline=None)
@given(st.integers(min_value=1, max_value=4), st.integers(0, 2**31 - 1))
def test_nvfp4_gemm_is_linear(M, seed):
    """y(a·x1 + b·x2) = a·y(x1) + b·y(x2) up to float64 rounding, and y scales with g."""
    rng = np.random.default_rng(seed)
    K, N = 64, 5
    w = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    codes, scales, g = oracle.nvfp4_quantize(w)
    x1 = rng.standard_normal((M, K)).astype(np.float16)
    x2 = rng.standard_normal((M, K)).astype(np.float16)
    y1, y2 = (oracle.nvfp4_gemm(x, codes, scales, g) for x in (x1, x2))
    comb = (2.0 * x1.astype(np.float64) - 0.5 * x2.astype(np.float64))
    yc = oracle.nvfp4_gemm(comb, codes, scales, g)
    assert np.allclose(yc, 2.0 * y1 - 0.5 * y2, rtol=1e-12, atol=1e-12)
    assert np.allclose(oracle.nvfp4_gemm(x1, codes, scales, 4.0 * g), 4.0 * y1, rtol=1e-14, atol=0)
