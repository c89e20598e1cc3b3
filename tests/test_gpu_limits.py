"""GPU parity at the size limits of the C ABI and in degenerate cases.

  * K = 2^20 (the largest K): every kernel family splits K many ways here.
  * N = 2^24 (the largest N) with K = 16: over a million column tiles; the
    NVFP4 blob pads K to one 1024-K span, so it is 9.7 GB.
  * N = 2^18 with K = 1024 for the lm_head: many tiles per wavefront in the
    streaming kernel, argmax over a quarter million columns.
  * all-zero activations: every output is exactly +0 or -0.
Outputs are compared with the oracle on all columns where that is cheap, on
sampled columns (first and last tiles plus random ones) otherwise.
"""

import time

import numpy as np
import pytest
import torch

import oracle
import fp8_quantized_skinny_amd as sk
from fp8_quantized_skinny_amd import synth

pytestmark = pytest.mark.gpu

REL_FROB = 2e-3
ROW_MAX = 1e-2


def _log(msg):
    print(f"[limits] {time.strftime('%H:%M:%S')} {msg}", flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _ws(op, M, K, N, config=None):
    n = sk.workspace_bytes(op, M, K, N, config)
    return sk.new_workspace(n, fill=0xA5)


def _check(got, ref, what):
    m = oracle.compare(got, ref)
    _log(f"{what}: {m}")
    assert m["rel_frob"] <= REL_FROB and m["row_max"] <= ROW_MAX, (what, m)


def _cols(N, k=512, seed=0):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(min(16, N)), np.arange(max(N - 16, 0), N),
                                     rng.choice(N, min(k, N), replace=False)]))


def _nvfp4(M, K, N, seed):
    w, x = synth.draw(M, K, N, seed=seed)
    codes, scales, g = sk.nvfp4_quantize(w)
    del w
    return x, codes, scales, g


@pytest.mark.timeout(600)
def test_nvfp4_largest_k():
    M, K, N = 8, 1 << 20, 40
    _log("preparing NVFP4 K = 2^20")
    x, codes, scales, g = _nvfp4(M, K, N, seed=31)
    blob = dev(sk.nvfp4_pack(codes, scales, g, K, N))
    ref = oracle.nvfp4_gemm(x, codes, scales, g)
    for Mi, cfg in ((8, None), (1, None), (3, None), (8, (1, 1, 8, 128)), (1, (0, 2, 16, 128))):
        y = torch.empty((Mi, N), dtype=torch.float16, device="cuda")
        sk.nvfp4_gemm(blob, dev(x[:Mi]), y, config=cfg, workspace=_ws(sk.OP_NVFP4, Mi, K, N, cfg))
        torch.cuda.synchronize()
        _check(y.float().cpu().numpy(), ref[:Mi], f"NVFP4 M={Mi} K=2^20 N={N} {cfg or 'default'}")


@pytest.mark.timeout(600)
def test_fp8_largest_k():
    M, K, N = 4, 1 << 20, 20
    _log("preparing FP8 K = 2^20")
    w, x = synth.draw(M, K, N, seed=32)
    codes, scales = sk.fp8_quantize(w)
    del w
    ref = oracle.fp8_gemm(x, codes, scales)
    for Mi in (4, 1):
        y = torch.empty((Mi, N), dtype=torch.float16, device="cuda")
        sk.fp8_gemm(dev(codes), dev(scales), dev(x[:Mi]), y, workspace=_ws(sk.OP_FP8, Mi, K, N))
        torch.cuda.synchronize()
        _check(y.float().cpu().numpy(), ref[:Mi], f"FP8 M={Mi} K=2^20 N={N}")


@pytest.mark.timeout(900)
def test_nvfp4_largest_n():
    M, K, N = 1, 16, 1 << 24
    _log("preparing NVFP4 N = 2^24")
    x, codes, scales, g = _nvfp4(M, K, N, seed=33)
    blob = sk.nvfp4_pack(codes, scales, g, K, N)
    _log(f"blob {blob.nbytes / 1e9:.2f} GB")
    blob_d = dev(blob)
    del blob
    cols = _cols(N)
    ref = oracle.nvfp4_gemm(x, codes, scales, g, cols=cols)
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    sk.nvfp4_gemm(blob_d, dev(x), y, workspace=_ws(sk.OP_NVFP4, M, K, N))
    torch.cuda.synchronize()
    _check(y.float().cpu().numpy()[:, cols], ref, "NVFP4 M=1 K=16 N=2^24 (sampled)")


@pytest.mark.timeout(900)
def test_fp8_largest_n():
    M, K, N = 2, 16, 1 << 24
    _log("preparing FP8 N = 2^24")
    w, x = synth.draw(M, K, N, seed=34)
    codes, scales = sk.fp8_quantize(w)
    del w
    cols = _cols(N)
    ref = oracle.fp8_gemm(x, codes, scales, cols=cols)
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    sk.fp8_gemm(dev(codes), dev(scales), dev(x), y, workspace=_ws(sk.OP_FP8, M, K, N))
    torch.cuda.synchronize()
    _check(y.float().cpu().numpy()[:, cols], ref, "FP8 M=2 K=16 N=2^24 (sampled)")


@pytest.mark.timeout(600)
def test_lm_head_quarter_million_columns():
    M, K, N = 8, 1024, 1 << 18
    _log("preparing lm_head N = 2^18")
    x, codes, scales, g = _nvfp4(M, K, N, seed=35)
    blob = dev(sk.nvfp4_pack(codes, scales, g, K, N))
    ref = oracle.nvfp4_gemm(x, codes, scales, g)
    want, margin = oracle.argmax_rows(ref)
    _log(f"oracle argmax {want}, margins {np.round(margin, 4)}")
    for Mi in (8, 1):
        idx = torch.full((Mi,), -7, dtype=torch.int32, device="cuda")
        sk.lm_head_gemm_argmax(blob, dev(x[:Mi]), idx, N, workspace=_ws(sk.OP_LM_HEAD, Mi, K, N))
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), want[:Mi]), (idx.cpu().numpy(), want[:Mi])


def test_zero_activations_give_zero_outputs():
    """x = 0 makes every output exactly zero, in every engine."""
    M, K, N = 8, 2064, 100
    _, codes, scales, g = _nvfp4(M, K, N, seed=36)
    blob = dev(sk.nvfp4_pack(codes, scales, g, K, N))
    z = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    for Mi, cfg in ((8, None), (1, None), (1, (1, 1, 3, 1)), (8, (1, 2, 2, 3)), (4, (2, 1, 8, 1))):
        y = torch.full((Mi, N), float("nan"), dtype=torch.float16, device="cuda")
        sk.nvfp4_gemm(blob, z[:Mi].contiguous(), y, config=cfg, workspace=_ws(sk.OP_NVFP4, Mi, K, N, cfg))
        torch.cuda.synchronize()
        assert (y == 0).all(), cfg
    w8, _ = synth.draw(1, K, N, seed=37)
    c8, s8 = sk.fp8_quantize(w8)
    y = torch.full((4, N), float("nan"), dtype=torch.float16, device="cuda")
    sk.fp8_gemm(dev(c8), dev(s8), z[:4].contiguous(), y, workspace=_ws(sk.OP_FP8, 4, K, N))
    torch.cuda.synchronize()
    assert (y == 0).all()


def test_read_probe_reads_without_writing():
    """The read probe over a zeroed buffer (a whole number of 9216-byte blocks
    plus a ragged tail it must not read) leaves its sink word untouched: it
    folds what it loads and writes only on a 2^-64 chance that zeros never hit."""
    from fp8_quantized_skinny_amd._lib import lib
    buf = torch.zeros(9216 * 37 + 100, dtype=torch.uint8, device="cuda")
    sink = torch.full((1,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    for nbytes in (9216, 9216 * 37, 9216 * 37 + 100):
        assert lib().skinny_read_probe(buf.data_ptr(), nbytes, sink.data_ptr(), None) == 0
    torch.cuda.synchronize()
    assert int(sink.item()) == 0x5A5A5A5A
