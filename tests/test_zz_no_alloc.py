"""nvfp4_gemm_noalloc on the GPU: the allocation-free call against nvfp4_gemm with a workspace.

Two calls in a row, the second with a smaller input: the down projection at
M = 8 (K = 17408, N = 5120: the library's choice splits K nine ways, so the
partial sums live in the library's device array) and then a smaller ragged
shape (M = 3, K = 9232, N = 333: a five-way split on the MFMA engine) that
reuses the array the first call left filled.  Each output equals the
workspace call's bit for bit (same kernels, same order of sums) and meets the
oracle's bounds.
"""

import numpy as np
import pytest
import torch

import oracle
import fp8_quantized_skinny_amd as sk
from fp8_quantized_skinny_amd import workload

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _with_workspace(case, M):
    K, N = case["K"], case["N"]
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    n = sk.workspace_bytes(sk.OP_NVFP4, M, K, N)
    ws = sk.new_workspace(n, fill=0xA5)
    sk.nvfp4_gemm(dev(case["blob"]), dev(case["x"][:M]), y, workspace=ws)
    return y


def test_noalloc_matches_the_workspace_call_twice_in_a_row():
    big = workload.nvfp4_case(8, 17408, 5120, seed=91)
    small = workload.nvfp4_case(3, 9232, 333, seed=92)
    assert sk.workspace_bytes(sk.OP_NVFP4, 8, 17408, 5120) > 0
    assert sk.workspace_bytes(sk.OP_NVFP4, 3, 9232, 333) > 0
    outs = []
    for case in (big, small):
        M, N = case["M"], case["N"]
        y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
        sk.nvfp4_gemm_noalloc(dev(case["blob"]), dev(case["x"]), y)
        outs.append(y)
    torch.cuda.synchronize()
    for case, y in zip((big, small), outs):
        want = _with_workspace(case, case["M"])
        torch.cuda.synchronize()
        assert torch.equal(y, want), f"noalloc differs from the workspace call at {case['M']}x{case['K']}x{case['N']}"
        ref = oracle.nvfp4_gemm(case["x"], case["codes"], case["scales"], case["g"])
        m = oracle.compare(y.float().cpu().numpy(), ref)
        assert m["rel_frob"] <= 2e-3 and m["row_max"] <= 1e-2, m
    # and once more on the big shape after the small one
    y = torch.empty((8, 5120), dtype=torch.float16, device="cuda")
    sk.nvfp4_gemm_noalloc(dev(big["blob"]), dev(big["x"]), y)
    torch.cuda.synchronize()
    assert torch.equal(y, outs[0])


def test_noalloc_rejects_shapes_beyond_its_scratch():
    x = torch.zeros((8, 1 << 20), dtype=torch.float16, device="cuda")
    y = torch.empty((8, 4096), dtype=torch.float16, device="cuda")
    blob = torch.zeros(256, dtype=torch.uint8, device="cuda")
    from fp8_quantized_skinny_amd._lib import lib
    st = lib().nvfp4_gemm_noalloc(blob.data_ptr(), x.data_ptr(), y.data_ptr(), 8, 1 << 20, 4096, None)
    assert st == sk.ESIZE


def test_noalloc_balanced_gemv():
    """A GEMV whose library choice is the balanced layout (engine 3: 800 tiles on 256 CUs, the last
    32 cut into two K-split workgroups each, added through counters in the library's array): the
    allocation-free call equals the workspace call bit for bit, twice in a row."""
    case = workload.nvfp4_case(1, 2048, 12800, seed=93)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert sk.default_config(sk.OP_NVFP4, 1, 2048, 12800)[0] == 3
    ys = []
    for _ in range(2):
        y = torch.full((1, 12800), float("nan"), dtype=torch.float16, device="cuda")
        sk.nvfp4_gemm_noalloc(dev(case["blob"]), dev(case["x"]), y)
        ys.append(y)
    want = _with_workspace(case, 1)
    torch.cuda.synchronize()
    assert torch.equal(ys[0], want) and torch.equal(ys[1], want)
    ref = oracle.nvfp4_gemm(case["x"], case["codes"], case["scales"], case["g"])
    m = oracle.compare(want.float().cpu().numpy(), ref)
    assert m["rel_frob"] <= 2e-3 and m["row_max"] <= 1e-2, m
