"""GPU parity with non-finite activations: NaN and +-inf in x.

The greedy token of a row is the lowest column holding its largest logit,
over the logits that are numbers; a NaN logit never wins and a row with no
number gives -1 (the oracle's argmax_rows).  The logits themselves follow
IEEE arithmetic of the definition: inf times a zero weight is NaN, inf plus
finite values stays inf, a NaN activation makes the whole row NaN.

Rows of x (M = 8, K = 2064: the last K span holds 16 real K, so every engine
meets K padding; N = 700, ragged):
  0  finite (an ordinary greedy token)
  1  one NaN                         -> every logit NaN, token -1
  2  +inf where half the columns have a zero code -> +-inf and NaN logits
  3  -inf at the last K (k = K - 1)   -> +-inf and NaN logits
  4  +inf and -inf at two K           -> inf, -inf or NaN per column
  5  finite
  6  all NaN                          -> token -1
  7  +inf where every column's code is zero -> every logit NaN, token -1
Each engine runs it: the VALU GEMV (rows one and two at a time), the
one-unit MFMA engine, the streaming engine and K-split choices (argmax in the
split reduction).  Logits: NaN exactly where the oracle has NaN, the same
infinity where it has one, the usual bounds elsewhere.
"""

import numpy as np
import pytest
import torch

import oracle
import fp8_quantized_skinny_amd as sk
from fp8_quantized_skinny_amd import workload

pytestmark = pytest.mark.gpu

K, N = 2064, 700


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _case():
    c = workload.nvfp4_case(8, K, N, seed=71)
    q = oracle.nvfp4_unpack_codes(c["codes"], K)
    k2, k7 = 11, 1500
    q[::2, k2] = 0                  # row 2: half the columns have a zero code under the inf
    q[:, k7] = 0                    # row 7: every column does
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    x = c["x"].copy()
    x[1, 700] = np.nan
    x[2, k2] = np.inf
    x[3, K - 1] = -np.inf
    x[4, 20], x[4, 2000] = np.inf, -np.inf
    x[6, :] = np.nan
    x[7, k7] = np.inf
    blob = sk.nvfp4_pack(codes, c["scales"], c["g"], K, N)
    return dict(c, codes=codes, x=x, blob=blob)


@pytest.fixture(scope="module")
def case():
    c = _case()
    with np.errstate(invalid="ignore"):
        c["ref"] = oracle.nvfp4_gemm(c["x"], c["codes"], c["scales"], c["g"])
    c["want"], _ = oracle.argmax_rows(c["ref"])
    return c


def _check_logits(got, ref, what):
    nan = np.isnan(ref)
    inf = np.isinf(ref)
    assert np.array_equal(np.isnan(got), nan), f"{what}: NaN pattern differs"
    assert np.array_equal(got[inf], ref[inf]), f"{what}: infinities differ"
    fin = ~(nan | inf)
    for m in range(ref.shape[0]):
        if not fin[m].any():
            continue
        d = np.abs(got[m][fin[m]] - ref[m][fin[m]])
        rms = np.sqrt(np.mean(ref[m][fin[m]] ** 2))
        assert d.max() <= 1e-2 * rms, f"{what}: row {m} max error {d.max()} vs rms {rms}"


def test_oracle_side_of_the_case(case):
    """The planted rows give what the definition says, before any GPU call."""
    ref, want = case["ref"], case["want"]
    assert np.isfinite(ref[[0, 5]]).all()
    assert np.isnan(ref[[1, 6, 7]]).all() and list(want[[1, 6, 7]]) == [-1, -1, -1]
    for m in (2, 3):
        assert np.isnan(ref[m]).any() and np.isinf(ref[m]).any()
    assert np.isinf(ref[2][1::2]).any() and np.isnan(ref[2][::2]).all()
    assert want[2] >= 0 and ref[2, want[2]] == np.inf
    assert want[3] >= 0 and ref[3, want[3]] == np.inf


def _lm_head(case, rows, cfg):
    M = len(rows)
    idx = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    lg = torch.empty((M, N), dtype=torch.float16, device="cuda")
    n = sk.workspace_bytes(sk.OP_LM_HEAD, M, K, N, cfg)
    ws = sk.new_workspace(n, fill=0xA5)
    sk.lm_head_gemm_argmax(dev(case["blob"]), dev(case["x"][rows]), idx, N, logits=lg, workspace=ws, config=cfg)
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    n = sk.workspace_bytes(sk.OP_NVFP4, M, K, N, cfg)
    ws = sk.new_workspace(n, fill=0xA5)
    sk.nvfp4_gemm(dev(case["blob"]), dev(case["x"][rows]), y, workspace=ws, config=cfg)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), lg.float().cpu().numpy(), y.float().cpu().numpy()


CHOICES_8 = [None, (1, 1, 3, 1), (1, 4, 12, 1), (1, 2, 4, 2), (1, 1, 1, 3), (2, 1, 16, 1), (2, 1, 4, 1)]
CHOICES_1 = [None, (0, 1, 3, 1), (0, 2, 6, 1), (0, 1, 1, 3), (0, 2, 4, 2), (1, 1, 3, 1), (1, 2, 4, 2), (2, 1, 16, 1)]


def test_nan_and_inf_activations_eight_rows(case):
    for cfg in CHOICES_8:
        assert cfg is None or sk.config_supported(sk.OP_LM_HEAD, 8, K, N, cfg), cfg
        idx, lg, y = _lm_head(case, list(range(8)), cfg)
        assert np.array_equal(idx, case["want"]), (cfg, idx, case["want"])
        _check_logits(lg, case["ref"], f"{cfg} logits")
        _check_logits(y, case["ref"], f"{cfg} y")


def test_nan_and_inf_activations_one_and_two_rows(case):
    """M = 1 runs the one-row key reduction; M = 2 the two-row VALU engine."""
    for cfg in CHOICES_1:
        for m in range(8):
            assert cfg is None or sk.config_supported(sk.OP_LM_HEAD, 1, K, N, cfg), cfg
            idx, lg, y = _lm_head(case, [m], cfg)
            assert idx[0] == case["want"][m], (cfg, m, idx[0], case["want"][m])
            _check_logits(lg, case["ref"][m:m + 1], f"{cfg} row {m} logits")
            _check_logits(y, case["ref"][m:m + 1], f"{cfg} row {m} y")
    for cfg in [c for c in CHOICES_1 if c is None or c[0] == 0]:
        for rows in ([0, 1], [2, 3], [4, 6], [7, 5]):
            idx, lg, _ = _lm_head(case, rows, cfg)
            assert np.array_equal(idx, case["want"][rows]), (cfg, rows, idx)
            _check_logits(lg, case["ref"][rows], f"{cfg} rows {rows} logits")


def test_fp8_inf_activation_at_the_last_k():
    """FP8 with K = 400 (the last 512-K unit holds 16 real K): -inf at k = K - 1
    and a NaN elsewhere, through the canonical and packed codes, VALU (M = 1, 2)
    and MFMA (M = 4) engines: the same NaN/inf pattern as the oracle."""
    Kf, Nf = 400, 300
    c = workload.fp8_case(4, Kf, Nf, seed=72)
    x = c["x"].copy()
    x[0, Kf - 1] = -np.inf
    x[1, 100] = np.nan
    x[2, Kf - 1] = np.inf
    with np.errstate(invalid="ignore"):
        ref = oracle.fp8_gemm(x, c["codes"], c["scales"])
    wp = dev(sk.fp8_pack(c["codes"], Kf, Nf))
    for M, cfg in [(1, None), (1, (0, 1, 1, 1)), (2, None), (4, None), (4, (1, 1, 1, 1)), (3, (0, 1, 1, 1))]:
        rows = [0, 1, 2, 3][:M]
        for packed in (False, True):
            y = torch.empty((M, Nf), dtype=torch.float16, device="cuda")
            if packed:
                sk.fp8_gemm_packed(wp, dev(c["scales"]), dev(x[rows]), y, config=cfg)
            else:
                sk.fp8_gemm(dev(c["codes"]), dev(c["scales"]), dev(x[rows]), y, config=cfg)
            torch.cuda.synchronize()
            _check_logits(y.float().cpu().numpy(), ref[rows], f"fp8 M={M} {cfg} packed={packed}")
