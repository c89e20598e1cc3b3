"""Pins of the oracle's quantizers (CPU only): invariants the rules imply."""

import numpy as np

import oracle
from fp8_quantized_skinny_amd import synth

# E2M1 gap below each positive magnitude code (distance to the next lower value).
_E2M1_MAG = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])


def _half_gap(mag):
    """Half of the spacing around |value| on the E2M1 grid (largest neighbour gap)."""
    idx = np.searchsorted(_E2M1_MAG, mag)
    idx = np.clip(idx, 1, 7)
    return (_E2M1_MAG[idx] - _E2M1_MAG[idx - 1]) / 2


def test_nvfp4_global_scale_and_top_block():
    w, _ = synth.draw(1, 256, 64, seed=3)
    codes, scales, g = oracle.nvfp4_quantize(w)
    amax = np.abs(w).max()
    assert g == np.float32(amax / 2688.0)
    # The block holding the global maximum gets scale 448 (0x7E) and code +-6.
    k, n = np.unravel_index(np.argmax(np.abs(w)), w.shape)
    assert scales[n, k // 16] == 0x7E
    q = oracle.nvfp4_unpack_codes(codes, 256)
    assert q[n, k] & 7 == 7
    assert (q[n, k] >> 3) == (w[k, n] < 0)


def test_nvfp4_every_normal_block_uses_code_six():
    # blk_amax / (s*g) = 6 * t / s with t/s within one E4M3 half-ulp of 1, so
    # the block maximum always encodes to magnitude 6.
    w, _ = synth.draw(1, 512, 128, seed=4)
    codes, scales, g = oracle.nvfp4_quantize(w)
    q = oracle.nvfp4_unpack_codes(codes, 512).reshape(128, 32, 16)
    s = oracle.e4m3_decode(scales)
    normal = s >= 2.0 ** -6
    assert normal.mean() > 0.99
    assert np.all((q[normal] & 7).max(axis=-1) == 7)


def test_nvfp4_error_bound():
    w, _ = synth.draw(1, 512, 96, seed=5)
    codes, scales, g = oracle.nvfp4_quantize(w)
    deq = oracle.nvfp4_dequant_unscaled(codes, scales, 512) * np.float64(g)   # [K, N]
    s = np.repeat(oracle.e4m3_decode(scales), 16, axis=1).T * np.float64(g)   # [K, N]
    ratio = np.abs(w.astype(np.float64)) / s
    bound = np.where(ratio >= 6, ratio - 6, _half_gap(np.minimum(ratio, 6))) * s
    assert np.all(np.abs(deq - w) <= bound + 1e-12 * np.abs(w))


def test_nvfp4_zero_cases():
    z = np.zeros((64, 32), np.float32)
    codes, scales, g = oracle.nvfp4_quantize(z)
    assert g == 0 and not codes.any() and not scales.any()
    w, _ = synth.draw(1, 64, 32, seed=6)
    w[16:32, 5] = 0.0                       # one all-zero block
    codes, scales, g = oracle.nvfp4_quantize(w)
    assert scales[5, 1] == 0
    q = oracle.nvfp4_unpack_codes(codes, 64)
    assert not (q[5, 16:32] & 7).any()


def test_nvfp4_code_layout_low_nibble_is_even_k():
    w = np.zeros((16, 1), np.float32)
    w[0, 0], w[1, 0] = 6.0, -3.0            # block max 6 -> s*g = 1 after scaling
    codes, scales, g = oracle.nvfp4_quantize(w)
    assert codes[0, 0] & 15 == 0x7 and codes[0, 0] >> 4 == 0xD


def test_fp8_scales_and_bound():
    w, _ = synth.draw(1, 256, 200, seed=7)
    codes, scales = oracle.fp8_quantize(w)
    assert scales.shape == (2, 2)
    for nb in range(2):
        for kb in range(2):
            blk = w[kb * 128:(kb + 1) * 128, nb * 128:(nb + 1) * 128]
            assert scales[nb, kb] == np.float32(np.abs(blk).max() / 448.0)
    deq = oracle.fp8_dequant(codes, scales)
    S = scales[np.arange(200) // 128][:, np.arange(256) // 128].T.astype(np.float64)
    # E4M3 relative half-ulp is 2^-4 for normals; subnormal spacing 2^-9.
    err = np.abs(deq - w)
    assert np.all(err <= np.maximum(np.abs(w) * 2.0 ** -4, 2.0 ** -10 * S) * (1 + 1e-12))
    # Each block's maximum encodes to +-448 exactly.
    c = oracle.e4m3_decode(codes)
    assert np.abs(c[:128, :128]).max() == 448.0


def test_fp8_zero_block():
    w = np.zeros((128, 256), np.float32)
    w[:, 128:] = 1.0
    codes, scales = oracle.fp8_quantize(w)
    assert scales[0, 0] == 0 and not codes[:128].any()
    assert np.all(oracle.e4m3_decode(codes[128:]) == 448.0)


def test_chunked_draw_equals_one_shot():
    rng1 = np.random.default_rng(0)
    a = (rng1.standard_normal((100, 37)) * 0.02).astype(np.float32)
    xa = rng1.standard_normal((3, 100)).astype(np.float16)
    rng2 = np.random.default_rng(0)
    b = synth.draw_weights(rng2, 100, 37, chunk_rows=7)
    xb = synth.draw_activations(rng2, 3, 100)
    assert np.array_equal(a, b) and np.array_equal(xa, xb)


def test_nvfp4_column_slices_with_the_whole_tensors_scale():
    """Blocks depend only on their own 16 values and g: quantizing column
    slices with the whole tensor's g gives the whole tensor's codes and
    scales, slice by slice; the slice's own g would differ."""
    w, _ = synth.draw(1, 256, 300, seed=64)
    codes, scales, g = oracle.nvfp4_quantize(w)
    assert g == oracle.nvfp4_global_scale(w)
    for c0, c1 in ((0, 7), (7, 130), (130, 300)):
        c, s, g2 = oracle.nvfp4_quantize(np.ascontiguousarray(w[:, c0:c1]), g=g)
        assert g2 == g
        assert np.array_equal(c, codes[c0:c1]) and np.array_equal(s, scales[c0:c1])
    own = oracle.nvfp4_quantize(np.ascontiguousarray(w[:, :7]))
    assert own[2] != g
