"""Pins of the oracle's GEMM, dequantization and argmax (CPU only).

  * exactness of E2M1 x E4M3 products in fp16 and fp32 (all 16 x 254 pairs)
  * brute force with exact rational arithmetic on tiny shapes
  * closed-form special cases: one-hot x, scaling by powers of two, zero
    weights, duplicated columns, constant blocks
"""

from fractions import Fraction

import numpy as np

import oracle
from fp8_quantized_skinny_amd import synth


def test_e2m1_times_e4m3_exact_in_fp16_and_fp32():
    q = oracle.e2m1_decode(np.arange(16))
    s = oracle.e4m3_decode(np.array([c for c in range(256) if c not in (0x7F, 0xFF)]))
    prod = np.outer(q, s)
    assert np.array_equal(prod.astype(np.float16).astype(np.float64), prod)
    assert np.array_equal(prod.astype(np.float32).astype(np.float64), prod)
    nz = np.abs(prod[prod != 0])
    assert nz.min() == 2.0 ** -10 and nz.max() == 2688.0


def _frac_e2m1(c):
    s = -1 if c & 8 else 1
    e, m = (c >> 1) & 3, c & 1
    return s * (Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2)))


def _frac_e4m3(c):
    s = -1 if c & 0x80 else 1
    e, m = (c >> 3) & 15, c & 7
    return s * (Fraction(m, 512) if e == 0 else Fraction(2) ** (e - 7) * (1 + Fraction(m, 8)))


def test_nvfp4_gemm_brute_force_fractions():
    for M, K, N, seed in [(1, 32, 5, 0), (3, 48, 4, 1), (8, 64, 3, 2)]:
        w, x = synth.draw(M, K, N, seed=seed)
        codes, scales, g = oracle.nvfp4_quantize(w)
        y = oracle.nvfp4_gemm(x, codes, scales, g)
        for m in range(M):
            for n in range(N):
                tot = Fraction(0)
                for k in range(K):
                    byte = int(codes[n, k // 2])
                    c = byte & 15 if k % 2 == 0 else byte >> 4
                    tot += Fraction(float(x[m, k])) * _frac_e2m1(c) * _frac_e4m3(int(scales[n, k // 16]))
                exact = tot * Fraction(float(g))
                assert abs(float(exact) - y[m, n]) <= 1e-13 * max(1.0, abs(float(exact)))


def test_fp8_gemm_brute_force_fractions():
    M, K, N = 2, 160, 130
    w, x = synth.draw(M, K, N, seed=9)
    codes, scales = oracle.fp8_quantize(w)
    y = oracle.fp8_gemm(x, codes, scales)
    for m in range(M):
        for n in (0, 1, 127, 128, 129):
            tot = Fraction(0)
            for k in range(K):
                tot += (Fraction(float(x[m, k])) * _frac_e4m3(int(codes[n, k]))
                        * Fraction(float(scales[n // 128, k // 128])))
            assert abs(float(tot) - y[m, n]) <= 1e-13 * max(1.0, abs(float(tot)))


def test_one_hot_rows_recover_dequantized_weights():
    K, N = 64, 16
    w, _ = synth.draw(1, K, N, seed=11)
    codes, scales, g = oracle.nvfp4_quantize(w)
    x = np.eye(K, dtype=np.float16)[:8]
    y = oracle.nvfp4_gemm(x, codes, scales, np.float32(1.0))
    deq = oracle.nvfp4_dequant_unscaled(codes, scales, K)
    assert np.array_equal(y, deq[:8])


def test_power_of_two_scaling_is_exact():
    w, x = synth.draw(2, 128, 24, seed=12)
    codes, scales, g = oracle.nvfp4_quantize(w)
    y1 = oracle.nvfp4_gemm(x, codes, scales, g)
    y2 = oracle.nvfp4_gemm((x.astype(np.float32) * 4).astype(np.float16), codes, scales, g)
    assert np.array_equal(y2, 4 * y1)


def test_constant_block_gives_scaled_code_sum():
    K, N = 32, 2
    w, _ = synth.draw(1, K, N, seed=13)
    codes, scales, g = oracle.nvfp4_quantize(w)
    x = np.zeros((1, K), np.float16)
    x[0, 16:32] = 1.0
    y = oracle.nvfp4_gemm(x, codes, scales, g)
    for n in range(N):
        q = oracle.e2m1_decode(oracle.nvfp4_unpack_codes(codes, K)[n, 16:32]).sum()
        assert y[0, n] == q * oracle.e4m3_decode(scales[n, 1]) * np.float64(g)


def test_zero_weights_and_argmax_ties():
    K, N = 64, 40
    codes = np.zeros((N, K // 2), np.uint8)
    scales = np.zeros((N, K // 16), np.uint8)
    _, x = synth.draw(3, K, N, seed=14)
    y = oracle.nvfp4_gemm(x, codes, scales, np.float32(0.5))
    assert not y.any()
    idx, _ = oracle.argmax_rows(y)
    assert np.array_equal(idx, [0, 0, 0])
    # duplicated best column: lower index wins
    w, _ = synth.draw(1, K, N, seed=15)
    c2, s2, g2 = oracle.nvfp4_quantize(w)
    y = oracle.nvfp4_gemm(x, c2, s2, g2)
    best = np.argmax(y[0])
    c2[N - 1], s2[N - 1] = c2[best], s2[best]
    c2[best - 1 if best > 0 else 0], s2[best - 1 if best > 0 else 0] = c2[best], s2[best]
    y = oracle.nvfp4_gemm(x, c2, s2, g2)
    idx, _ = oracle.argmax_rows(y)
    assert idx[0] == max(best - 1, 0)


def test_argmax_matches_scan():
    rng = np.random.default_rng(16)
    y = rng.integers(-5, 5, size=(6, 50)).astype(np.float64)
    idx, margin = oracle.argmax_rows(y)
    for m in range(6):
        best = 0
        for n in range(50):
            if y[m, n] > y[m, best]:
                best = n
        assert idx[m] == best
    assert np.all(margin >= 0)


def test_column_subset_matches_full():
    w, x = synth.draw(4, 256, 300, seed=17)
    codes, scales, g = oracle.nvfp4_quantize(w)
    full = oracle.nvfp4_gemm(x, codes, scales, g, chunk=64)
    cols = np.array([0, 5, 299, 150])
    assert np.array_equal(oracle.nvfp4_gemm(x, codes, scales, g, cols=cols), full[:, cols])
    c8, s8 = oracle.fp8_quantize(w)
    f8 = oracle.fp8_gemm(x, c8, s8, chunk=100)
    assert np.array_equal(oracle.fp8_gemm(x, c8, s8, cols=cols), f8[:, cols])


def test_compare_metrics():
    ref = np.array([[3.0, 4.0], [0.0, 1.0]])
    m = oracle.compare(ref + np.array([[0.0, 0.1], [0.0, 0.0]]), ref)
    assert abs(m["rel_frob"] - 0.1 / np.sqrt(26)) < 1e-15
    assert abs(m["row_max"] - 0.1 / np.sqrt(12.5)) < 1e-15


def test_silu_closed_forms():
    """SiLU pinned by values and identities that do not use its formula:
    sigmoid(ln 3) = 3/4, silu(z) - silu(-z) = z, silu(z) + silu(-z) =
    z * tanh(z / 2), and the limits z (large z) and -0 (very negative z)."""
    ln3 = np.log(3.0)
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(ln3) - 0.75 * ln3) <= 1e-15
    assert abs(oracle.silu(-ln3) + 0.25 * ln3) <= 1e-15
    z = np.linspace(-30.0, 30.0, 601)
    s, t = oracle.silu(z), oracle.silu(-z)
    assert np.allclose(s - t, z, rtol=0, atol=1e-13)
    assert np.allclose(s + t, z * np.tanh(z / 2), rtol=0, atol=1e-13)
    assert oracle.silu(40.0) == 40.0
    big_neg = oracle.silu(-800.0)
    assert big_neg == 0.0 and np.signbit(big_neg)


def test_nvfp4_swiglu_brute_force():
    """h = silu(gate) * up against exact rational gate and up sums with the
    activation taken in Python's math library, on tiny shapes."""
    import math
    for M, K, F, seed in [(1, 32, 3, 3), (4, 48, 5, 4), (8, 64, 2, 5)]:
        w, x = synth.draw(M, K, 2 * F, seed=seed)
        gate = oracle.nvfp4_quantize(w[:, :F])
        up = oracle.nvfp4_quantize(w[:, F:])
        h = oracle.nvfp4_swiglu(x, gate, up)
        assert h.shape == (M, F)
        for m in range(M):
            for f in range(F):
                val = []
                for codes, scales, g in (gate, up):
                    tot = Fraction(0)
                    for k in range(K):
                        byte = int(codes[f, k // 2])
                        c = byte & 15 if k % 2 == 0 else byte >> 4
                        tot += Fraction(float(x[m, k])) * _frac_e2m1(c) * _frac_e4m3(int(scales[f, k // 16]))
                    val.append(float(tot * Fraction(float(g))))
                a, b = val
                want = a / (1.0 + math.exp(-a)) * b
                assert abs(want - h[m, f]) <= 1e-12 * max(1.0, abs(want))


def test_nvfp4_swiglu_zero_halves():
    """A zero gate gives silu(0) * up = 0; a zero up gives 0 whatever the gate."""
    M, K, F = 3, 64, 4
    w, x = synth.draw(M, K, 2 * F, seed=6)
    gate = oracle.nvfp4_quantize(w[:, :F])
    up = oracle.nvfp4_quantize(w[:, F:])
    zero = oracle.nvfp4_quantize(np.zeros((K, F), np.float32))
    assert np.all(oracle.nvfp4_swiglu(x, zero, up) == 0.0)
    assert np.all(oracle.nvfp4_swiglu(x, gate, zero) == 0.0)


def _scan_argmax(row):
    """Greedy token by a plain scan: skip NaN, keep the first strictly larger logit; -1 if none."""
    best = -1
    for n, v in enumerate(row):
        if v != v:
            continue
        if best < 0 or v > row[best]:
            best = n
    return best


def test_argmax_nan_never_wins():
    """A NaN logit, whatever its sign bit, is no score: the greedy token is the
    first maximum of the numbers in the row (+-inf count), and a row with no
    number at all gives -1."""
    nan, inf = np.nan, np.inf
    neg_nan = np.copysign(np.nan, -1.0)
    assert np.signbit(neg_nan) and not np.signbit(nan)
    rows = [
        ([nan, 1.0, neg_nan, 2.0, 2.0], 3),
        ([nan, nan, nan], -1),
        ([neg_nan, neg_nan], -1),
        ([nan, neg_nan, nan, neg_nan], -1),
        ([nan, -inf, neg_nan], 1),
        ([inf, nan, inf], 0),
        ([neg_nan, -inf, -inf], 1),
        ([nan, -inf, inf, neg_nan, inf], 2),
        ([-0.0, 0.0, nan], 0),
        ([neg_nan, -5.0, 7.0, nan, 7.0], 2),
    ]
    for row, want in rows:
        idx, _ = oracle.argmax_rows(np.array([row]))
        assert idx[0] == want, (row, idx[0], want)
        assert _scan_argmax(row) == want, row


def test_argmax_with_nan_and_inf_matches_scan():
    """Random rows with NaN of both signs, +-inf and exact ties planted, some
    rows all NaN: the oracle equals the plain scan in every row."""
    rng = np.random.default_rng(61)
    specials = np.array([np.nan, np.copysign(np.nan, -1.0), np.inf, -np.inf])
    for trial in range(200):
        M, N = int(rng.integers(1, 9)), int(rng.integers(1, 40))
        y = rng.integers(-3, 4, size=(M, N)).astype(np.float64)
        plant = rng.random((M, N)) < rng.random()
        y[plant] = specials[rng.integers(0, 4, size=int(plant.sum()))]
        if trial % 7 == 0:
            y[int(rng.integers(M))] = specials[rng.integers(0, 2, size=N)]   # an all-NaN row
        idx, margin = oracle.argmax_rows(y)
        for m in range(M):
            assert idx[m] == _scan_argmax(list(y[m])), (y[m], idx[m])
        finite_rows = np.isfinite(y).all(axis=1) & (N > 1)
        assert np.all(margin[finite_rows] >= 0)


def test_gemm_with_non_finite_activations_follows_ieee():
    """Activations holding +-inf and NaN: the oracle's sums equal a plain
    Python loop over IEEE doubles (inf * 0 is NaN, inf plus a finite value
    stays inf, NaN spreads), element by element, NaN where NaN."""
    K, N = 48, 9
    w, _ = synth.draw(1, K, N, seed=62)
    codes, scales, g = oracle.nvfp4_quantize(w)
    q = oracle.nvfp4_unpack_codes(codes, K)
    q[::2, 5] = 0                                   # zero codes under the inf of row 0
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    x = np.zeros((4, K), np.float16)
    x[:] = np.random.default_rng(63).standard_normal((4, K)).astype(np.float16)
    x[0, 5] = np.inf
    x[1, K - 1] = -np.inf
    x[2, 7] = np.nan
    x[3, 3], x[3, 40] = np.inf, -np.inf
    y = oracle.nvfp4_gemm(x, codes, scales, g)
    deq = oracle.nvfp4_dequant_unscaled(codes, scales, K)
    for m in range(4):
        for n in range(N):
            s = 0.0
            for k in range(K):
                s += float(x[m, k]) * float(deq[k, n])
            want = s * float(g)
            if want != want:
                assert np.isnan(y[m, n]), (m, n, y[m, n])
            elif abs(want) == float("inf"):
                assert y[m, n] == want, (m, n, y[m, n], want)
            else:
                assert abs(y[m, n] - want) <= 1e-12 * max(1.0, abs(want)), (m, n)
    assert np.isnan(y[2]).all()
    assert np.isnan(y[0, ::2]).all() and np.isinf(y[0, 1::2]).all()
