"""GPU parity at the full decode shapes, in the kernel choice the benchmark times.

Outputs are checked on sampled columns, which the oracle computes one by one
(first and last tiles plus 512 random columns); the lm_head argmax is checked
against the oracle's full float64 logit rows.  Runs print their steps so a
long input preparation is visible.
"""

import time

import numpy as np
import pytest
import torch

import oracle
import fp8_quantized_skinny_amd as sk
from fp8_quantized_skinny_amd import workload, synth

pytestmark = pytest.mark.gpu

REL_FROB = 2e-3
ROW_MAX = 1e-2


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _cols(N, seed=0):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(16), np.arange(N - 16, N), rng.choice(N, 512, replace=False)]))


def _log(msg):
    print(f"[full] {time.strftime('%H:%M:%S')} {msg}", flush=True)


def _ws(op, M, K, N):
    """Junk-filled workspace for the library's default kernel choice (None if none is needed)."""
    n = sk.workspace_bytes(op, M, K, N)
    return torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda") if n else None


@pytest.mark.parametrize("name,ms", [("up", (1, 4)), ("gate_up", (8, 4)), ("down", (8, 4)),
                                     ("up_tp4", (1, 4, 8)), ("gate_up_tp4", (1, 4, 8)), ("down_tp4", (1, 4, 8))])
def test_nvfp4_full_shape_sampled(name, ms):
    """The decode shapes in the benchmark's kernel choice, with M = 4 (k = 3
    drafts, the long-context setting) beside the listed M, and one rank's
    share of each shape under 4-way tensor parallelism."""
    _log(f"preparing {name}")
    case = workload.named_case(name, M=8)
    K, N = case["K"], case["N"]
    blob = dev(case["blob"])
    cols = _cols(N)
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
        got = y.float().cpu().numpy()[:, cols]
        ref = oracle.nvfp4_gemm(case["x"][:M], case["codes"], case["scales"], case["g"], cols=cols)
        m = oracle.compare(got, ref)
        _log(f"{name} M={M}: {m}")
        assert m["rel_frob"] <= REL_FROB and m["row_max"] <= ROW_MAX, m
        assert np.isfinite(y.float().cpu().numpy()).all()


def test_swiglu_gate_up_full_shape_sampled():
    """The fused gate+up shape (K = 5120, 2 x 17408 columns) with the SwiGLU
    epilogue: h[M, 17408], M = 1 and 8, against the oracle on sampled columns."""
    fmt, ms, K, N = synth.WORKLOADS["gate_up"]
    F = N // 2
    _log("preparing gate_up SwiGLU pair")
    case = workload.swiglu_case(8, K, F)
    blob = dev(case["blob"])
    cols = _cols(F)
    for M in (1, 8):
        x = dev(case["x"][:M])
        ws = _ws(sk.OP_SWIGLU, M, K, F)
        h = torch.empty((M, F), dtype=torch.float16, device="cuda")
        sk.nvfp4_gemm_swiglu(blob, x, h, workspace=ws)
        h2 = torch.empty_like(h)
        sk.nvfp4_gemm_swiglu(blob, x, h2, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(h, h2), "not deterministic"
        got = h.float().cpu().numpy()[:, cols]
        ref = oracle.nvfp4_swiglu(case["x"][:M], case["gate"], case["up"], cols=cols)
        m = oracle.compare(got, ref)
        _log(f"gate_up SwiGLU M={M}: {m}")
        assert m["rel_frob"] <= REL_FROB and m["row_max"] <= ROW_MAX, m
        assert np.isfinite(h.float().cpu().numpy()).all()


@pytest.mark.parametrize("name", ["qkv", "o_proj", "qkv_tp4", "o_proj_tp4"])
def test_fp8_full_shape_sampled(name):
    _log(f"preparing {name}")
    case = workload.named_case(name)
    K, N = case["K"], case["N"]
    w, s = dev(case["codes"]), dev(case["scales"])
    wp = dev(sk.fp8_pack(case["codes"], K, N))
    cols = _cols(N)
    for M in synth.WORKLOADS[name][1]:
        ws = _ws(sk.OP_FP8, M, K, N)
        y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        sk.fp8_gemm(w, s, dev(case["x"][:M]), y, workspace=ws)
        y2 = torch.empty_like(y)
        sk.fp8_gemm(w, s, dev(case["x"][:M]), y2, workspace=ws)
        yp = torch.empty_like(y)
        sk.fp8_gemm_packed(wp, s, dev(case["x"][:M]), yp, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y, y2), "not deterministic"
        assert torch.equal(y, yp), "packed codes give a different result"
        got = y.float().cpu().numpy()[:, cols]
        ref = oracle.fp8_gemm(case["x"][:M], case["codes"], case["scales"], cols=cols)
        m = oracle.compare(got, ref)
        _log(f"{name} M={M}: {m}")
        assert m["rel_frob"] <= REL_FROB and m["row_max"] <= ROW_MAX, m


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["lm_head", "lm_head_tp4"])
def test_lm_head_full_shape_argmax_bit_exact(name):
    _log(f"preparing {name}")
    case = workload.named_case(name)
    K, N = case["K"], case["N"]
    blob = dev(case["blob"])
    _log("oracle logits (float64, full rows)")
    ref = oracle.nvfp4_gemm(case["x"], case["codes"], case["scales"], case["g"])
    want, margin = oracle.argmax_rows(ref)
    _log(f"oracle argmax {want} margins {np.round(margin, 4)}")
    cols = _cols(N)
    for M in (1, 8):
        ws = _ws(sk.OP_LM_HEAD, M, K, N)
        idx = torch.empty((M,), dtype=torch.int32, device="cuda")
        lg = torch.empty((M, N), dtype=torch.float16, device="cuda")
        sk.lm_head_gemm_argmax(blob, dev(case["x"][:M]), idx, N, logits=lg, workspace=ws)
        idx2 = torch.empty_like(idx)
        sk.lm_head_gemm_argmax(blob, dev(case["x"][:M]), idx2, N, workspace=ws)
        torch.cuda.synchronize()
        got = idx.cpu().numpy()
        _log(f"lm_head M={M}: gpu {got}")
        assert np.array_equal(got, want[:M]), (got, want[:M], margin[:M])
        assert torch.equal(idx, idx2)
        m = oracle.compare(lg.float().cpu().numpy()[:, cols], ref[:M, cols])
        assert m["rel_frob"] <= REL_FROB and m["row_max"] <= ROW_MAX, m
