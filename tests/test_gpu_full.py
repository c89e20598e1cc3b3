"""GPU parity at the full decode shapes, in the kernel choice the benchmark times.

Inputs: the seeded weights are quantized by the oracle (full_inputs.py, which
also checks that the library's own quantizer gives the same bytes at each
shape), and the library only packs them.  Every output element is compared
with the oracle's float64 result: rel-Frobenius over the whole M x N output
and the per-row maximum error against the row's RMS.  The lm_head's argmax
must equal the oracle's bit for bit on every row, and each row's margin
(top-1 minus top-2 over the row RMS) must be at least 1e-4 so that
bit-exactness is decidable at fp32; a row below that is reported as
ill-conditioned and fails.

Exactness of the dequantized weights at full K: with g = 1 and one-hot
activation rows the output equals e2m1 * e4m3 exactly, here run in the
library's default kernel choice of each full shape (forced onto a narrow
weight of the same K) and in streaming choices where every wavefront walks
several tiles.

Runs print their steps so that a long input preparation is visible.
"""

import time

import numpy as np
import pytest
import torch

import oracle
import fp8_quantized_skinny_amd as sk
from fp8_quantized_skinny_amd import synth

import full_inputs as fi

pytestmark = pytest.mark.gpu

REL_FROB = 2e-3
ROW_MAX = 1e-2
MIN_MARGIN = 1e-4


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _log(msg):
    print(f"[full] {time.strftime('%H:%M:%S')} {msg}", flush=True)


def _ws(op, M, K, N, cfg=None):
    """Junk-filled workspace for a kernel choice (None if none is needed)."""
    n = sk.workspace_bytes(op, M, K, N, cfg)
    return sk.new_workspace(n, fill=0xA5)


def _whole(got, ref, what):
    m = oracle.compare(got, ref)
    _log(f"{what}: rel_frob {m['rel_frob']:.3e} row_max {m['row_max']:.3e}")
    assert m["rel_frob"] <= REL_FROB and m["row_max"] <= ROW_MAX, (what, m)
    assert np.isfinite(got).all(), what


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,ms", [("up", (1, 4)), ("gate_up", (8, 4)), ("down", (8, 4, 2, 1)),
                                     ("up_tp4", (1, 4, 8)), ("gate_up_tp4", (1, 4, 8)), ("down_tp4", (1, 4, 8))])
def test_nvfp4_full_shape_whole_output(name, ms):
    """The decode shapes in the benchmark's kernel choice, with M = 4 (k = 3
    drafts, the long-context setting) beside the listed M, and one rank's
    share of each shape under 4-way tensor parallelism."""
    _, _, K, N = synth.WORKLOADS[name]
    _log(f"preparing {name} ({K} x {N})")
    case = fi.nvfp4_case(8, K, N)
    ref = fi.nvfp4_reference(case["x"], case["codes"], case["scales"], case["g"])
    blob = dev(case["blob"])
    for M in ms:
        x = dev(case["x"][:M])
        ws = _ws(sk.OP_NVFP4, M, K, N)
        y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        sk.nvfp4_gemm(blob, x, y, workspace=ws)
        y2 = torch.empty_like(y)
        sk.nvfp4_gemm(blob, x, y2, workspace=ws)
        torch.cuda.synchronize()
        # the second call reuses the workspace left behind by the first
        assert torch.equal(y, y2), "not deterministic"
        _whole(y.float().cpu().numpy(), ref[:M], f"{name} M={M} {sk.default_config(sk.OP_NVFP4, M, K, N)}")


@pytest.mark.timeout(600)
def test_swiglu_gate_up_full_shape_whole_output():
    """The fused gate+up shape (K = 5120, 2 x 17408 columns) with the SwiGLU
    epilogue: h[M, 17408], M = 1 and 8, every element against the oracle."""
    _, _, K, N = synth.WORKLOADS["gate_up"]
    F = N // 2
    _log("preparing gate_up SwiGLU pair")
    case = fi.swiglu_case(8, K, F)
    ref = fi.swiglu_reference(case["x"], case["gate"], case["up"])
    blob = dev(case["blob"])
    for M in (1, 8):
        x = dev(case["x"][:M])
        ws = _ws(sk.OP_SWIGLU, M, K, F)
        h = torch.empty((M, F), dtype=torch.float16, device="cuda")
        sk.nvfp4_gemm_swiglu(blob, x, h, workspace=ws)
        h2 = torch.empty_like(h)
        sk.nvfp4_gemm_swiglu(blob, x, h2, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(h, h2), "not deterministic"
        _whole(h.float().cpu().numpy(), ref[:M], f"gate_up SwiGLU M={M}")


@pytest.mark.parametrize("name", ["qkv", "o_proj", "qkv_tp4", "o_proj_tp4"])
def test_fp8_full_shape_whole_output(name):
    _, ms, K, N = synth.WORKLOADS[name]
    _log(f"preparing {name} ({K} x {N})")
    case = fi.fp8_case(max(ms), K, N)
    ref = fi.fp8_reference(case["x"], case["codes"], case["scales"])
    w, s = dev(case["codes"]), dev(case["scales"])
    wp = dev(sk.fp8_pack(case["codes"], K, N))
    for M in ms:
        ws = _ws(sk.OP_FP8, M, K, N)
        x = dev(case["x"][:M])
        y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        sk.fp8_gemm(w, s, x, y, workspace=ws)
        y2 = torch.empty_like(y)
        sk.fp8_gemm(w, s, x, y2, workspace=ws)
        yp = torch.empty_like(y)
        sk.fp8_gemm_packed(wp, s, x, yp, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y, y2), "not deterministic"
        assert torch.equal(y, yp), "packed codes give a different result"
        _whole(y.float().cpu().numpy(), ref[:M], f"{name} M={M} {sk.default_config(sk.OP_FP8, M, K, N)}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["lm_head", "lm_head_tp4"])
def test_lm_head_full_shape_argmax_bit_exact(name):
    _, _, K, N = synth.WORKLOADS[name]
    _log(f"preparing {name} ({K} x {N})")
    case = fi.nvfp4_case(8, K, N)
    blob = dev(case["blob"])
    _log("oracle logits (float64, whole rows)")
    ref = fi.nvfp4_reference(case["x"], case["codes"], case["scales"], case["g"])
    want, margin = oracle.argmax_rows(ref)
    _log(f"oracle argmax {want} margins {np.round(margin, 5)}")
    for M in (1, 8):
        ws = _ws(sk.OP_LM_HEAD, M, K, N)
        idx = torch.empty((M,), dtype=torch.int32, device="cuda")
        lg = torch.empty((M, N), dtype=torch.float16, device="cuda")
        sk.lm_head_gemm_argmax(blob, dev(case["x"][:M]), idx, N, logits=lg, workspace=ws)
        idx2 = torch.empty_like(idx)
        sk.lm_head_gemm_argmax(blob, dev(case["x"][:M]), idx2, N, workspace=ws)
        torch.cuda.synchronize()
        got = idx.cpu().numpy()
        _log(f"{name} M={M} {sk.default_config(sk.OP_LM_HEAD, M, K, N)}: gpu {got}")
        assert torch.equal(idx, idx2)
        _whole(lg.float().cpu().numpy(), ref[:M], f"{name} M={M} logits")
        ill = margin[:M] < MIN_MARGIN
        for m in np.flatnonzero(ill):
            # still a valid choice up to the fp32 error of the sums?
            rms = np.sqrt(np.mean(ref[m] ** 2))
            ok = ref[m, got[m]] >= ref[m].max() - MIN_MARGIN * rms
            _log(f"row {m} ill-conditioned (margin {margin[m]:.2e}); gpu pick valid up to rounding: {ok}")
        assert not ill.any(), f"ill-conditioned rows {np.flatnonzero(ill)}: bit-exactness is not decidable"
        assert np.array_equal(got, want[:M]), (got, want[:M], margin[:M])


# ------------------------------------------------------------ exactness at full K
def _one_hot_exact(K, N, M, cfg, op=sk.OP_NVFP4, seed=81):
    """y over one-hot rows (g = 1) equals e2m1 * e4m3 exactly for every K row and column."""
    w, _ = fi.draw(1, K, N, seed)
    codes, scales, _ = fi.nvfp4_quantize(w)
    blob = dev(sk.nvfp4_pack(codes, scales, 1.0, K, N))
    assert sk.config_supported(op, M, K, N, cfg), cfg
    eye = torch.eye(K, dtype=torch.float16, device="cuda")
    out = torch.empty((K, N), dtype=torch.float16, device="cuda")
    ws = _ws(op, M, K, N, cfg)
    idx = torch.empty((M,), dtype=torch.int32, device="cuda")
    for r0 in range(0, K, M):
        rows = min(M, K - r0)
        if op == sk.OP_LM_HEAD:
            sk.lm_head_gemm_argmax(blob, eye[r0:r0 + rows], idx[:rows], N, logits=out[r0:r0 + rows],
                                   workspace=ws, config=cfg)
        else:
            sk.nvfp4_gemm(blob, eye[r0:r0 + rows], out[r0:r0 + rows], workspace=ws, config=cfg)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    for c0 in range(0, N, 4096):
        cols = np.arange(c0, min(N, c0 + 4096))
        deq = oracle.nvfp4_dequant_unscaled(codes, scales, K, cols=cols)
        bad = np.argwhere(got[:, cols] != deq)
        assert bad.size == 0, f"K={K} N={N} M={M} {cfg}: first mismatches (k, n) {bad[:5]}"
    _log(f"one-hot exact: K={K} N={N} M={M} {cfg}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,M", [("up", 1), ("up", 2), ("up", 8), ("gate_up", 8), ("down", 8), ("down", 2),
                                    ("down", 1), ("lm_head", 1), ("lm_head", 8)])
def test_one_hot_exact_in_the_full_shapes_kernel_choice(name, M):
    """The default choice of each full shape, forced onto a narrow weight of
    the same K (80 columns: five tiles, so tile groups and a partial group
    occur), reproduces the dequantized weights exactly."""
    _, _, K, N = synth.WORKLOADS[name]
    op = sk.OP_LM_HEAD if name == "lm_head" else sk.OP_NVFP4
    cfg = sk.default_config(op, M, K, N)
    _one_hot_exact(K, 80, M, cfg, op=op)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg", [(2, 1, 1, 1), (2, 1, 2, 1), (2, 1, 3, 1)])
def test_one_hot_exact_streaming_several_tiles_per_wavefront(cfg):
    """K = 5120 (five spans, an odd count: tile pairs swap unit buffers) and
    N = 12368 (773 tiles) on 256 CUs: one wavefront per workgroup walks three
    or four tiles (tile pairs and an odd last tile); with two or three per
    workgroup some walk two."""
    _one_hot_exact(5120, 12368, 8, cfg)
