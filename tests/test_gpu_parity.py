"""GPU parity of the HIP kernels against the CPU oracle at small and ragged shapes.

Bars (element by element, same seeded inputs on both sides):
  * dequantized weights before the global scale: exact (one-hot activations)
  * GEMM outputs: rel. Frobenius error <= 2e-3 and, per row,
    max |error| <= 1e-2 * RMS of the oracle's row
  * argmax indices: identical
Every kernel variant (engine, column tiles per workgroup, wavefronts per
workgroup) is covered, at shapes that span several tiles and chunks and leave
ragged tails in K (not a multiple of 128) and N (not a multiple of 16).
"""

import itertools

import numpy as np
import pytest
import torch

import oracle
import fp8_quantized_skinny_amd as sk
from fp8_quantized_skinny_amd import workload

pytestmark = pytest.mark.gpu

REL_FROB = 2e-3
ROW_MAX = 1e-2
def cfgs(engine, K, unit_k=1024, splits=(1, 2, 3), cts=(1, 2, 4, 8)):
    """(engine, ct, nw, ksplit) choices valid for this K.

    A workgroup covers S = nw / ct K units of ct tiles; ksplit workgroups must
    cover all ku units of K and each must get some.  Besides the tight S, one
    more span than needed is tried too (it leaves idle wavefronts)."""
    ku = -(-K // unit_k)
    out = []
    for ct in cts:
        for ks in splits:
            S = -(-ku // ks)
            for s in (S, S + 1):
                if ks * s >= ku and (ks - 1) * s < ku and ct * s <= 16:
                    out.append((engine, ct, ct * s, ks))
    return sorted(set(out))


STREAM = [(2, 1, 16, 1), (2, 1, 4, 1), (2, 2, 8, 1), (2, 1, 1, 1)]


def stream_cfgs(op, M, K, N):
    """Streaming-engine choices (x resident in LDS, whole tiles per wavefront) supported here."""
    return [c for c in STREAM if sk.config_supported(op, M, K, N, c)]


def ws_for(op, M, K, N, config):
    """Workspace for a call, filled with junk: the library must not rely on its contents."""
    n = sk.workspace_bytes(op, M, K, N, config)
    return sk.new_workspace(n, fill=0xA5)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _check(y_gpu, y_ref, what):
    m = oracle.compare(y_gpu, y_ref)
    assert m["rel_frob"] <= REL_FROB and m["row_max"] <= ROW_MAX, f"{what}: {m}"
    return m


def run_nvfp4(case, M=None, config=None, guard=0):
    M = case["M"] if M is None else M
    K, N = case["K"], case["N"]
    blob = dev(case["blob"])
    x = dev(case["x"][:M])
    buf = torch.full((M * N + 2 * guard,), float("nan"), dtype=torch.float16, device="cuda")
    y = buf[guard:guard + M * N].view(M, N)
    sk.nvfp4_gemm(blob, x, y, config=config, workspace=ws_for(sk.OP_NVFP4, M, K, N, config))
    torch.cuda.synchronize()
    if guard:
        assert torch.isnan(buf[:guard]).all() and torch.isnan(buf[guard + M * N:]).all(), "guard overwritten"
    return y.float().cpu().numpy()


def run_fp8(case, M=None, config=None, packed=False):
    M = case["M"] if M is None else M
    K, N = case["K"], case["N"]
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    ws = ws_for(sk.OP_FP8, M, K, N, config)
    if packed:
        sk.fp8_gemm_packed(dev(sk.fp8_pack(case["codes"], K, N)), dev(case["scales"]), dev(case["x"][:M]), y,
                           config=config, workspace=ws)
    else:
        sk.fp8_gemm(dev(case["codes"]), dev(case["scales"]), dev(case["x"][:M]), y, config=config, workspace=ws)
    torch.cuda.synchronize()
    return y.float().cpu().numpy()


def ref_nvfp4(case, M=None):
    M = case["M"] if M is None else M
    return oracle.nvfp4_gemm(case["x"][:M], case["codes"], case["scales"], case["g"])


def ref_fp8(case, M=None):
    M = case["M"] if M is None else M
    return oracle.fp8_gemm(case["x"][:M], case["codes"], case["scales"])


SMALL_NVFP4 = [(1, 256, 512), (1, 272, 100), (3, 400, 300), (8, 1040, 1000), (8, 2064, 48), (1, 3088, 200), (2, 16, 7),
               (2, 2064, 333)]


@pytest.fixture(scope="module")
def small_nvfp4():
    return {s: workload.nvfp4_case(*s, seed=sum(s)) for s in SMALL_NVFP4}


# ------------------------------------------------------------ exactness
@pytest.mark.parametrize("K,N", [(256, 512), (272, 100)])
def test_nvfp4_one_hot_reproduces_dequantized_weights_exactly(K, N):
    """With g = 1 and one-hot rows, y equals e2m1(q) * e4m3(s) exactly (fp16 holds it)."""
    case = workload.nvfp4_case(1, K, N, seed=5)
    blob = dev(sk.nvfp4_pack(case["codes"], case["scales"], 1.0, K, N))
    deq = oracle.nvfp4_dequant_unscaled(case["codes"], case["scales"], K)       # [K, N]
    assert np.array_equal(deq.astype(np.float16).astype(np.float64), deq)
    eye = torch.eye(K, dtype=torch.float16, device="cuda")
    for cfg in cfgs(1, K) + cfgs(0, K) + stream_cfgs(sk.OP_NVFP4, 8, K, N):
        for rows in ((1, 2) if cfg[0] == 0 else (8,)):
            out = np.empty((K, N))
            ws = ws_for(sk.OP_NVFP4, rows, K, N, cfg)
            for r0 in range(0, K, rows):
                y = torch.empty((rows, N), dtype=torch.float16, device="cuda")
                sk.nvfp4_gemm(blob, eye[r0:r0 + rows].contiguous(), y, config=cfg, workspace=ws)
                out[r0:r0 + rows] = y.float().cpu().numpy()
            assert np.array_equal(out, deq), f"config {cfg} rows {rows}: {np.argwhere(out != deq)[:5]}"


def test_nvfp4_one_hot_exact_in_the_balanced_gemv():
    """The balanced GEMV (engine 3) over several spans with a ragged last span (K = 3088)
    and 257 tiles, so 256 whole-K tiles and one tile cut into K-split workgroups added
    inside the kernel: with g = 1 and one-hot rows, every weight comes out exactly, at
    M = 1 and 2."""
    K, N = 3088, 4112
    case = workload.nvfp4_case(1, K, N, seed=9)
    blob = dev(sk.nvfp4_pack(case["codes"], case["scales"], 1.0, K, N))
    deq = oracle.nvfp4_dequant_unscaled(case["codes"], case["scales"], K)       # [K, N]
    assert np.array_equal(deq.astype(np.float16).astype(np.float64), deq)
    cfg = (3, 1, -(-K // 1024), 1)
    eye = torch.eye(K, dtype=torch.float16, device="cuda")
    for rows in (1, 2):
        assert sk.config_supported(sk.OP_NVFP4, rows, K, N, cfg)
        ws = ws_for(sk.OP_NVFP4, rows, K, N, cfg)
        out = torch.empty((K, N), dtype=torch.float16, device="cuda")
        for r0 in range(0, K, rows):
            sk.nvfp4_gemm(blob, eye[r0:r0 + rows].contiguous(), out[r0:r0 + rows], config=cfg, workspace=ws)
        got = out.float().cpu().numpy()
        assert np.array_equal(got, deq), f"rows {rows}: {np.argwhere(got != deq)[:5]}"
        assert not ws[:sk.WORKSPACE_SYNC_BYTES].any().item(), "arrival counters not back at zero"


def test_fp8_one_hot_reproduces_codes_exactly():
    """Random finite E4M3 codes, power-of-two block scales: y = e4m3(c) * S exactly."""
    K, N = 272, 200
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C
    scales = np.ldexp(1.0, rng.integers(-6, 2, size=(2, 3))).astype(np.float32)
    case = {"codes": codes, "scales": scales, "K": K, "N": N}
    deq = oracle.fp8_dequant(codes, scales)
    assert np.array_equal(deq.astype(np.float16).astype(np.float64), deq)
    eye = np.eye(K, dtype=np.float16)
    for packed in (False, True):
        for cfg in cfgs(1, K, unit_k=512):
            out = np.empty((K, N))
            for r0 in range(0, K, 8):
                case["x"] = eye[r0:r0 + 8]
                out[r0:r0 + 8] = run_fp8(case, M=8, config=cfg, packed=packed)
            assert np.array_equal(out, deq), f"config {cfg} packed={packed}"
        # the VALU engine (M <= 4): one and three rows at a time (three rows run
        # as four, the fourth a copy never stored), a sample of rows in every chunk
        for cfg in cfgs(0, K, unit_k=512):
            for r0 in list(range(0, K, 7)) + [K - 1]:
                case["x"] = eye[r0:r0 + 1]
                got = run_fp8(case, M=1, config=cfg, packed=packed)
                assert np.array_equal(got[0], deq[r0]), f"VALU config {cfg} packed={packed} row {r0}"
            for r0 in list(range(0, K - 2, 11)) + [K - 3]:
                case["x"] = eye[r0:r0 + 3]
                got = run_fp8(case, M=3, config=cfg, packed=packed)
                assert np.array_equal(got, deq[r0:r0 + 3]), f"VALU config {cfg} packed={packed} rows {r0}..+3"


def test_fp8_one_hot_exact_over_several_units():
    """The same over three 512-K units with a ragged last unit (K = 1040) and a
    ragged last tile (N = 40): every K row of every unit, chunk and piece lands
    on its own column, canonical and packed, in the MFMA engine (every row) and
    the VALU engine (a sample of rows)."""
    K, N = 1040, 40
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C
    scales = np.ldexp(1.0, rng.integers(-6, 2, size=(1, 9))).astype(np.float32)
    case = {"codes": codes, "scales": scales, "K": K, "N": N}
    deq = oracle.fp8_dequant(codes, scales)
    assert np.array_equal(deq.astype(np.float16).astype(np.float64), deq)
    eye = np.eye(K, dtype=np.float16)
    for packed in (False, True):
        for cfg in cfgs(1, K, unit_k=512, cts=(1, 4)):
            out = np.empty((K, N))
            for r0 in range(0, K, 8):
                case["x"] = eye[r0:r0 + 8]
                out[r0:r0 + 8] = run_fp8(case, M=8, config=cfg, packed=packed)
            assert np.array_equal(out, deq), f"config {cfg} packed={packed}: {np.argwhere(out != deq)[:5]}"
        for cfg in cfgs(0, K, unit_k=512, cts=(1, 2)):
            for r0 in list(range(0, K, 5)) + [K - 1]:
                case["x"] = eye[r0:r0 + 1]
                got = run_fp8(case, M=1, config=cfg, packed=packed)
                assert np.array_equal(got[0], deq[r0]), f"VALU config {cfg} packed={packed} row {r0}"


# -------------------------------------------------------- tolerance parity
@pytest.mark.parametrize("shape", SMALL_NVFP4)
def test_nvfp4_parity_all_configs(small_nvfp4, shape):
    case = small_nvfp4[shape]
    ref = ref_nvfp4(case)
    choices = (cfgs(1, case["K"]) + (cfgs(0, case["K"]) if case["M"] <= 2 else [])
               + stream_cfgs(sk.OP_NVFP4, case["M"], case["K"], case["N"]))
    for cfg in choices:
        _check(run_nvfp4(case, config=cfg), ref, f"{shape} {cfg}")
    _check(run_nvfp4(case, guard=8), ref, f"{shape} default")


def test_nvfp4_every_m():
    case = workload.nvfp4_case(8, 1152, 520, seed=11)
    for M in range(1, 9):
        ref = ref_nvfp4(case, M)
        _check(run_nvfp4(case, M=M), ref, f"M={M} default")
        _check(run_nvfp4(case, M=M, config=(1, 2, 2, 2)), ref, f"M={M} mfma split")
        _check(run_nvfp4(case, M=M, config=(2, 1, 16, 1)), ref, f"M={M} streaming")
        if M <= 2:
            _check(run_nvfp4(case, M=M, config=(0, 1, 1, 2)), ref, f"M={M} VALU split")
            _check(run_nvfp4(case, M=M, config=(0, 2, 4, 1)), ref, f"M={M} VALU")


# ------------------------------------------------------------ SwiGLU pair
SMALL_SWIGLU = [(1, 256, 8), (1, 272, 13), (3, 400, 100), (8, 1040, 500), (8, 2064, 21), (1, 3088, 40), (2, 16, 5),
                (2, 2064, 40)]


def run_swiglu(case, M=None, config=None, guard=0):
    M = case["M"] if M is None else M
    K, F = case["K"], case["F"]
    buf = torch.full((M * F + 2 * guard,), float("nan"), dtype=torch.float16, device="cuda")
    h = buf[guard:guard + M * F].view(M, F)
    sk.nvfp4_gemm_swiglu(dev(case["blob"]), dev(case["x"][:M]), h, config=config,
                         workspace=ws_for(sk.OP_SWIGLU, M, K, F, config))
    torch.cuda.synchronize()
    if guard:
        assert torch.isnan(buf[:guard]).all() and torch.isnan(buf[guard + M * F:]).all(), "guard overwritten"
    return h.float().cpu().numpy()


@pytest.mark.parametrize("shape", SMALL_SWIGLU)
def test_nvfp4_swiglu_parity_all_configs(shape):
    """h = silu(x.Wg) * (x.Wu) from the interleaved pair, in every engine, against the oracle."""
    M, K, F = shape
    case = workload.swiglu_case(M, K, F, seed=sum(shape) + 7)
    ref = oracle.nvfp4_swiglu(case["x"], case["gate"], case["up"])
    choices = (cfgs(1, K) + (cfgs(0, K) if M <= 2 else [])
               + stream_cfgs(sk.OP_SWIGLU, M, K, F))
    assert choices
    for cfg in choices:
        _check(run_swiglu(case, config=cfg), ref, f"swiglu {shape} {cfg}")
    _check(run_swiglu(case, guard=8), ref, f"swiglu {shape} default")


def test_nvfp4_swiglu_every_m_and_shared_scale():
    """Every row count, and a pair quantized with one scale for the fused tensor."""
    K, F = 1152, 72
    case = workload.swiglu_case(8, K, F, seed=21)
    for M in range(1, 9):
        ref = oracle.nvfp4_swiglu(case["x"][:M], case["gate"], case["up"])
        _check(run_swiglu(case, M=M), ref, f"swiglu M={M} default")
        _check(run_swiglu(case, M=M, config=(1, 2, 2, 2)), ref, f"swiglu M={M} mfma split")
        _check(run_swiglu(case, M=M, config=(2, 1, 16, 1)), ref, f"swiglu M={M} streaming")
    w, x = workload.synth.draw(4, K, 2 * F, seed=22)
    codes, scales, g = sk.nvfp4_quantize(w)       # one g for the fused [K, 2F] tensor
    gate, up = (codes[:F], scales[:F], g), (codes[F:], scales[F:], g)
    shared = {"M": 4, "K": K, "F": F, "x": x, "blob": sk.nvfp4_pack_swiglu(gate, up, K, F)}
    ref = oracle.nvfp4_swiglu(x, gate, up)
    for cfg in (None, (1, 1, 2, 1), (2, 2, 8, 1)):
        _check(run_swiglu(shared, config=cfg), ref, f"swiglu shared g {cfg}")


SMALL_FP8 = [(1, 256, 256), (2, 272, 100), (4, 400, 300), (8, 1040, 1000), (3, 16, 129)]


@pytest.mark.parametrize("shape", SMALL_FP8)
def test_fp8_parity_all_configs(shape):
    """Canonical and packed codes, every kernel choice: within the bounds of the
    oracle, and the packed path equal to the canonical one bit for bit (same
    pieces in the same registers, only the byte order in memory differs)."""
    case = workload.fp8_case(*shape, seed=sum(shape))
    ref = ref_fp8(case)
    valu = cfgs(0, case["K"], unit_k=512) if case["M"] <= 4 else []
    for cfg in cfgs(1, case["K"], unit_k=512) + valu + [None]:
        y = run_fp8(case, config=cfg)
        _check(y, ref, f"{shape} {cfg}")
        assert np.array_equal(run_fp8(case, config=cfg, packed=True), y), f"{shape} {cfg} packed"


@pytest.mark.parametrize("groups", [1024, 1025])
def test_in_kernel_split_reduction_group_limit(groups):
    """A plain MFMA call with a K split adds the splits inside the GEMM kernel
    when it has at most 1024 tile groups (one arrival counter each in the
    workspace's first 128 KiB), and through the split-reduction kernel beyond;
    both at the limit, against the oracle, and twice in a row on one workspace
    (the counters must be back at zero after the first call)."""
    M, K, N = 3, 2048, 16 * groups
    cfg = (1, 1, 1, 2)
    case = workload.nvfp4_case(M, K, N, seed=groups)
    ref = ref_nvfp4(case)
    blob, x = dev(case["blob"]), dev(case["x"])
    ws = ws_for(sk.OP_NVFP4, M, K, N, cfg)
    ys = []
    for _ in range(2):
        y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
        sk.nvfp4_gemm(blob, x, y, config=cfg, workspace=ws)
        ys.append(y)
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1])
    _check(ys[0].float().cpu().numpy(), ref, f"{groups} tile groups")
    assert not ws[:sk.WORKSPACE_SYNC_BYTES].any().item(), "arrival counters not back at zero"


def balanced_layout(nt, ku, cus):
    """The library's split of a one-tile-whole-K GEMV over `cus` CUs (engine 3): the largest
    multiple of cus of tiles stay whole; each other tile becomes `splits` workgroups of `spans`
    K spans, at most one per CU.  None when the tiles divide evenly or there are more than four
    whole tiles per CU."""
    if nt % cus == 0 or nt // cus > 4:
        return None
    rest = nt % cus
    for spans in range(1, ku + 1):
        splits = -(-ku // spans)
        if rest * splits <= min(cus, 1024):
            return nt - rest, spans, splits
    return None


@pytest.mark.parametrize("M,K,N", [(1, 5120, 4688), (2, 3088, 8272), (2, 9008, 1008), (1, 1024, 4112),
                                   (1, 2048, 4096)])
def test_balanced_gemv(M, K, N):
    """Engine 3 (one tile of whole K per workgroup, balanced over the CUs): the tiles past the
    largest multiple of the CU count are cut into K-split workgroups, added inside the kernel.
    Whole tiles give the bits of (0, 1, ku, 1) and split tiles those of (0, 1, spans, splits),
    which add the same sums in the same order; against the oracle too, twice in a row on one
    workspace (the arrival counters must be back at zero)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ku, nt = -(-K // 1024), -(-N // 16)
    cfg = (3, 1, ku, 1)
    assert sk.config_supported(sk.OP_NVFP4, M, K, N, cfg)
    case = workload.nvfp4_case(M, K, N, seed=N)
    blob, x = dev(case["blob"]), dev(case["x"])
    ws = ws_for(sk.OP_NVFP4, M, K, N, cfg)
    ys = []
    for _ in range(2):
        y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
        sk.nvfp4_gemm(blob, x, y, config=cfg, workspace=ws)
        ys.append(y)
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1])
    assert not ws[:sk.WORKSPACE_SYNC_BYTES].any().item(), "arrival counters not back at zero"
    got = ys[0].float().cpu().numpy()
    _check(got, ref_nvfp4(case), f"balanced {M}x{K}x{N}")
    whole = run_nvfp4(case, config=(0, 1, ku, 1))
    lay = balanced_layout(nt, ku, cus)
    if lay is None:
        assert np.array_equal(got, whole)
        return
    w, spans, splits = lay
    assert np.array_equal(got[:, :16 * w], whole[:, :16 * w])
    split = run_nvfp4(case, config=(0, 1, spans, splits))
    assert np.array_equal(got[:, 16 * w:], split[:, 16 * w:])


def test_deterministic_repeats(small_nvfp4):
    case = small_nvfp4[(8, 1040, 1000)]
    a = run_nvfp4(case)
    b = run_nvfp4(case)
    assert np.array_equal(a, b)
    c1 = small_nvfp4[(1, 272, 100)]
    assert np.array_equal(run_nvfp4(c1), run_nvfp4(c1))
    s1 = run_nvfp4(case, config=(2, 1, 16, 1))
    assert np.array_equal(s1, run_nvfp4(case, config=(2, 1, 16, 1)))


# ------------------------------------------------------------------ argmax
def run_lm_head(case, M, config=None, logits=False, ws=None):
    K, N = case["K"], case["N"]
    idx = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    ws = ws if ws is not None else ws_for(sk.OP_LM_HEAD, M, K, N, config)
    lg = torch.empty((M, N), dtype=torch.float16, device="cuda") if logits else None
    sk.lm_head_gemm_argmax(dev(case["blob"]), dev(case["x"][:M]), idx, N, logits=lg, workspace=ws, config=config)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), (lg.float().cpu().numpy() if logits else None)


@pytest.mark.parametrize("shape", [(1, 256, 1000), (8, 512, 3000), (5, 272, 777), (8, 1024, 16), (2, 2064, 1500)])
def test_lm_head_argmax_and_logits(shape):
    M, K, N = shape
    case = workload.nvfp4_case(*shape, seed=sum(shape))
    ref = ref_nvfp4(case)
    want, margin = oracle.argmax_rows(ref)
    valu = cfgs(0, K) if M <= 2 else []
    for cfg in valu + cfgs(1, K) + stream_cfgs(sk.OP_LM_HEAD, M, K, N):
        idx, lg = run_lm_head(case, M, config=cfg, logits=True)
        assert np.array_equal(idx, want), f"{shape} {cfg}: {idx} vs {want} (margins {margin})"
        _check(lg, ref, f"{shape} {cfg} logits")
    idx, _ = run_lm_head(case, M)
    assert np.array_equal(idx, want)


@pytest.mark.parametrize("M,K", [(4, 256), (8, 2048), (1, 2048), (2, 1024)])
def test_lm_head_ties_go_to_lowest_column(M, K):
    """Exact ties in every row; M = 8 fills both four-row groups of the MFMA
    output, K = 2048 adds K-split choices (argmax in the split reduction) and
    M = 1 and 2 add the VALU engine's candidates, M = 1 the one-row key
    reduction."""
    N = 700
    case = workload.nvfp4_case(M, K, N, seed=21)
    ref = ref_nvfp4(case)
    best = oracle.argmax_rows(ref)[0]
    codes, scales = case["codes"].copy(), case["scales"].copy()
    # Copy each row's winning column into a lower and a higher column: exact ties.
    for m, b in enumerate(best):
        for dst in (max(int(b) - 37, 0) if m % 2 else 3 + m, N - 1 - m):
            codes[dst], scales[dst] = codes[b], scales[b]
    case2 = dict(case, codes=codes, scales=scales, blob=sk.nvfp4_pack(codes, scales, case["g"], K, N))
    ref2 = ref_nvfp4(case2)
    want, _ = oracle.argmax_rows(ref2)
    valu = cfgs(0, K) if M <= 2 else []
    for cfg in valu + cfgs(1, K) + stream_cfgs(sk.OP_LM_HEAD, M, K, N):
        idx, _ = run_lm_head(case2, M, config=cfg)
        assert np.array_equal(idx, want), f"{cfg}: {idx} vs {want}"


def test_lm_head_one_row_with_more_candidates_than_one_reduction_round():
    """M = 1 on one 16-column tile per workgroup: 18750 candidates, more than
    the 16384 that the one-row key reduction reads in one round.  The winning
    column is moved into the last tile, so it is found only in the second
    round; the logits are checked too."""
    M, K, N = 1, 256, 300000
    case = workload.nvfp4_case(M, K, N, seed=24)
    b = int(oracle.argmax_rows(ref_nvfp4(case))[0][0])
    dst = N - 5
    codes, scales = case["codes"].copy(), case["scales"].copy()
    codes[[b, dst]], scales[[b, dst]] = codes[[dst, b]], scales[[dst, b]]
    case2 = dict(case, codes=codes, scales=scales, blob=sk.nvfp4_pack(codes, scales, case["g"], K, N))
    ref2 = ref_nvfp4(case2)
    want, margin = oracle.argmax_rows(ref2)
    assert want[0] == dst
    for cfg in [(0, 1, 1, 1), (0, 2, 2, 1), None]:
        idx, lg = run_lm_head(case2, M, config=cfg, logits=True)
        assert np.array_equal(idx, want), (cfg, idx, want, margin)
        _check(lg, ref2, f"{cfg} logits")


def test_lm_head_zero_weights_and_shared_workspace():
    M, K, N = 8, 256, 300
    case = workload.nvfp4_case(M, K, N, seed=22)
    zc = np.zeros_like(case["codes"])
    zs = np.zeros_like(case["scales"])
    zero = dict(case, codes=zc, scales=zs, blob=sk.nvfp4_pack(zc, zs, case["g"], K, N))
    idx, lg = run_lm_head(zero, M, logits=True)
    assert np.array_equal(idx, np.zeros(M)) and not lg.any()
    # one workspace reused across calls with different M
    ws = ws_for(sk.OP_LM_HEAD, 8, K, N, None)
    for Mi in (8, 1, 5, 8):
        want, _ = oracle.argmax_rows(ref_nvfp4(case, Mi))
        idx, _ = run_lm_head(case, Mi, ws=ws)
        assert np.array_equal(idx, want), Mi


# ------------------------------------------------------ speculative verify
def run_verify(case, M, drafts, config=None):
    K, N = case["K"], case["N"]
    idx = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    res = torch.full((M + 1,), -9, dtype=torch.int32, device="cuda")
    d = dev(np.asarray(drafts, np.int32)) if M > 1 else None
    sk.lm_head_verify_greedy(dev(case["blob"]), dev(case["x"][:M]), d, idx, res, N,
                             workspace=ws_for(sk.OP_LM_HEAD, M, K, N, config), config=config)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), res.cpu().numpy()


def test_lm_head_verify_greedy_rounds():
    """Rounds of k = 7 drafts that are accepted in full, cut at every position,
    or rejected at once, plus M = 1: the device's accepted length and committed
    tokens equal the oracle's verification of the oracle's argmax, bit for bit."""
    M, K, N = 8, 2048, 3000
    case = workload.nvfp4_case(M, K, N, seed=23)
    want_idx, margin = oracle.argmax_rows(ref_nvfp4(case))
    rng = np.random.default_rng(5)
    rounds = [list(want_idx[:M - 1])]
    for cut in range(M - 1):                      # first wrong draft at position `cut`
        d = list(want_idx[:M - 1])
        d[cut] = (d[cut] + 1 + int(rng.integers(N - 1))) % N
        rounds.append(d)
    choices = [None, (1, 2, 2, 2), (2, 1, 16, 1), (1, 1, 1, 2), (1, 4, 8, 1)]
    assert all(c is None or sk.config_supported(sk.OP_LM_HEAD, M, K, N, c) for c in choices)
    for cfg in choices:
        for drafts in rounds:
            idx, res = run_verify(case, M, drafts, config=cfg)
            assert np.array_equal(idx, want_idx), (cfg, idx, want_idx, margin)
            L, committed = oracle.verify_greedy(want_idx, drafts)
            want_res = [L] + committed + [-1] * (M - 1 - L)
            assert list(res) == want_res, (cfg, drafts, list(res), want_res)
    idx, res = run_verify(case, 1, [])
    assert list(res) == [0, int(want_idx[0])]
    # M = 2 (one draft), accepted and rejected, on the VALU engine and the default choice
    for cfg in [(0, 1, 2, 1), (0, 2, 2, 2), None]:
        for d in ([int(want_idx[0])], [(int(want_idx[0]) + 1) % N]):
            idx, res = run_verify(case, 2, d, config=cfg)
            assert np.array_equal(idx, want_idx[:2]), (cfg, idx, want_idx[:2])
            L, committed = oracle.verify_greedy(want_idx[:2], d)
            assert list(res) == [L] + committed + [-1] * (1 - L), (cfg, d, list(res))


def test_calls_on_two_streams_do_not_interfere():
    """The library keeps no state between calls: a K-split NVFP4 GEMM (GEMM
    kernel plus split reduction) and an lm_head argmax (streaming kernel plus
    key reduction) issued together on two streams, each with its own
    workspace, four rounds in a row, give bit for bit what each gives alone."""
    a = workload.nvfp4_case(8, 4096, 3000, seed=41)       # default choice splits K four ways
    b = workload.nvfp4_case(8, 1024, 20000, seed=42)      # streaming engine, argmax epilogue
    assert sk.workspace_bytes(sk.OP_NVFP4, 8, 4096, 3000) > 0
    wa, xa, wb, xb = dev(a["blob"]), dev(a["x"]), dev(b["blob"]), dev(b["x"])
    wsa = ws_for(sk.OP_NVFP4, 8, 4096, 3000, None)
    wsb = ws_for(sk.OP_LM_HEAD, 8, 1024, 20000, None)
    ya_ref = torch.empty((8, 3000), dtype=torch.float16, device="cuda")
    ib_ref = torch.empty((8,), dtype=torch.int32, device="cuda")
    sk.nvfp4_gemm(wa, xa, ya_ref, workspace=wsa)
    sk.lm_head_gemm_argmax(wb, xb, ib_ref, 20000, workspace=wsb)
    torch.cuda.synchronize()
    assert np.array_equal(ib_ref.cpu().numpy(), oracle.argmax_rows(ref_nvfp4(b))[0])
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for s in (s1, s2):
        s.wait_stream(torch.cuda.current_stream())
    ya = [torch.full((8, 3000), float("nan"), dtype=torch.float16, device="cuda") for _ in range(4)]
    ib = [torch.full((8,), -7, dtype=torch.int32, device="cuda") for _ in range(4)]
    torch.cuda.synchronize()
    for r in range(4):
        sk.nvfp4_gemm(wa, xa, ya[r], workspace=wsa, stream=s1)
        sk.lm_head_gemm_argmax(wb, xb, ib[r], 20000, workspace=wsb, stream=s2)
    torch.cuda.synchronize()
    for r in range(4):
        assert torch.equal(ya[r], ya_ref), f"round {r}: GEMM on a second stream differs"
        assert torch.equal(ib[r], ib_ref), f"round {r}: argmax on a second stream differs"


# ------------------------------------------------------ mixed-allocation table
def test_layer_table_mixed_allocation():
    """A stack of FP4, FP8 and SwiGLU-pair layers run through one table call:
    every layer's output against that layer's oracle, at M = 1 and 8, and a
    chained pair whose second layer reads the first one's output."""
    nv = workload.nvfp4_case(8, 1040, 300, seed=41)
    f8 = workload.fp8_case(8, 512, 384, seed=42)
    sw = workload.swiglu_case(8, 1040, 100, seed=43)
    dn = workload.nvfp4_case(8, 2064, 48, seed=44)
    f8b = workload.fp8_case(8, 400, 300, seed=45)
    layers = [(sk.LAYER_NVFP4, dev(nv["blob"]), None, 1040, 300),
              (sk.LAYER_FP8, dev(f8["codes"]), dev(f8["scales"]), 512, 384),
              (sk.LAYER_SWIGLU, dev(sw["blob"]), None, 1040, 100),
              (sk.LAYER_NVFP4, dev(dn["blob"]), None, 2064, 48),
              (sk.LAYER_FP8, dev(f8b["codes"]), dev(f8b["scales"]), 400, 300),
              (sk.LAYER_FP8_PACKED, dev(sk.fp8_pack(f8b["codes"], 400, 300)), dev(f8b["scales"]), 400, 300)]
    for M in (8, 1):
        refs = [ref_nvfp4(nv, M), ref_fp8(f8, M), oracle.nvfp4_swiglu(sw["x"][:M], sw["gate"], sw["up"]),
                ref_nvfp4(dn, M), ref_fp8(f8b, M), ref_fp8(f8b, M)]
        xs = [dev(c["x"][:M]) for c in (nv, f8, sw, dn, f8b, f8b)]
        ys = [torch.full((M, l[4]), float("nan"), dtype=torch.float16, device="cuda") for l in layers]
        n = sk.layers_workspace_bytes(layers, M)
        ws = sk.new_workspace(n, fill=0xA5)
        sk.layers_run(layers, xs, ys, workspace=ws)
        torch.cuda.synchronize()
        for i, (y, ref) in enumerate(zip(ys, refs)):
            _check(y.float().cpu().numpy(), ref, f"layer {i} M={M}")
        assert torch.equal(ys[4], ys[5]), "packed FP8 layer differs from the canonical one"
    # chain: NVFP4 1040 -> 512, then FP8 512 -> 384 on the first layer's fp16 output
    a = workload.nvfp4_case(4, 1040, 512, seed=46)
    b = workload.fp8_case(4, 512, 384, seed=47)
    chain = [(sk.LAYER_NVFP4, dev(a["blob"]), None, 1040, 512), (sk.LAYER_FP8, dev(b["codes"]), dev(b["scales"]), 512, 384)]
    mid = torch.empty((4, 512), dtype=torch.float16, device="cuda")
    out = torch.empty((4, 384), dtype=torch.float16, device="cuda")
    n = sk.layers_workspace_bytes(chain, 4)
    sk.layers_run(chain, [dev(a["x"]), mid], [mid, out],
                  workspace=sk.new_workspace(n))
    torch.cuda.synchronize()
    _check(mid.float().cpu().numpy(), ref_nvfp4(a), "chain layer 0")
    _check(out.float().cpu().numpy(), oracle.fp8_gemm(mid.cpu().numpy(), b["codes"], b["scales"]), "chain layer 1")


# ------------------------------------------------------------- graph replay
def test_hip_graph_replays_match_eager():
    """Every entry point captured in one HIP graph (K-split choices with their
    workspaces included, the balanced GEMV, packed FP8 and a two-layer table too) and replayed three times, with the outputs cleared by
    eager fills between replays: each replay equals the eager results bit for
    bit.  The benchmark times graph replays, and the library records no memset
    into a stream (workspaces are written before they are read)."""
    nv = workload.nvfp4_case(8, 2064, 1000, seed=51)
    f8 = workload.fp8_case(4, 1040, 640, seed=52)
    sw = workload.swiglu_case(8, 2064, 72, seed=53)
    lm = workload.nvfp4_case(8, 1024, 3000, seed=54)
    bal = workload.nvfp4_case(2, 2064, 4800, seed=55)      # 300 tiles: engine 3 cuts the last 44 along K
    want_idx = oracle.argmax_rows(ref_nvfp4(lm))[0]
    drafts = dev(np.asarray(want_idx[:7], np.int32))
    bufs = {"nv": dev(nv["blob"]), "nvx": dev(nv["x"]), "f8c": dev(f8["codes"]), "f8s": dev(f8["scales"]),
            "f8x": dev(f8["x"]), "sw": dev(sw["blob"]), "swx": dev(sw["x"]), "lm": dev(lm["blob"]), "lmx": dev(lm["x"]),
            "f8p": dev(sk.fp8_pack(f8["codes"], 1040, 640)), "nvx4": dev(nv["x"][:4]),
            "bal": dev(bal["blob"]), "balx": dev(bal["x"])}
    # a two-layer table at M = 4: NVFP4 then packed FP8 (independent inputs)
    layers = [(sk.LAYER_NVFP4, bufs["nv"], None, 2064, 1000), (sk.LAYER_FP8_PACKED, bufs["f8p"], bufs["f8s"], 1040, 640)]
    outs = {"y_nv": torch.empty((8, 1000), dtype=torch.float16, device="cuda"),
            "y_nv_split": torch.empty((8, 1000), dtype=torch.float16, device="cuda"),
            "y_f8": torch.empty((4, 640), dtype=torch.float16, device="cuda"),
            "h": torch.empty((8, 72), dtype=torch.float16, device="cuda"),
            "h_split": torch.empty((8, 72), dtype=torch.float16, device="cuda"),
            "idx": torch.empty((8,), dtype=torch.int32, device="cuda"),
            "vidx": torch.empty((8,), dtype=torch.int32, device="cuda"),
            "res": torch.empty((9,), dtype=torch.int32, device="cuda"),
            "y_f8p": torch.empty((4, 640), dtype=torch.float16, device="cuda"),
            "ly_nv": torch.empty((4, 1000), dtype=torch.float16, device="cuda"),
            "ly_f8p": torch.empty((4, 640), dtype=torch.float16, device="cuda"),
            "y_bal": torch.empty((2, 4800), dtype=torch.float16, device="cuda")}
    split = (1, 2, 4, 2)                                   # three K spans over two workgroups
    f8split = (1, 1, 1, 3)
    wss = {k: ws_for(op, M, K, N, cfg) for k, (op, M, K, N, cfg) in {
        "nv": (sk.OP_NVFP4, 8, 2064, 1000, None), "nv_split": (sk.OP_NVFP4, 8, 2064, 1000, split),
        "f8": (sk.OP_FP8, 4, 1040, 640, f8split), "sw": (sk.OP_SWIGLU, 8, 2064, 72, None),
        "sw_split": (sk.OP_SWIGLU, 8, 2064, 72, split), "lm": (sk.OP_LM_HEAD, 8, 1024, 3000, None),
        "lmv": (sk.OP_LM_HEAD, 8, 1024, 3000, None), "f8p": (sk.OP_FP8, 4, 1040, 640, f8split),
        "bal": (sk.OP_NVFP4, 2, 2064, 4800, (3, 1, 3, 1))}.items()}
    n_layers = sk.layers_workspace_bytes(layers, 4)
    wss["layers"] = sk.new_workspace(n_layers)
    assert wss["nv_split"] is not None and wss["f8"] is not None and wss["sw_split"] is not None
    assert sk.config_supported(sk.OP_NVFP4, 8, 2064, 1000, split) and sk.config_supported(sk.OP_SWIGLU, 8, 2064, 72, split)
    assert sk.config_supported(sk.OP_FP8, 4, 1040, 640, f8split)

    def calls(stream):
        sk.nvfp4_gemm(bufs["nv"], bufs["nvx"], outs["y_nv"], workspace=wss["nv"], stream=stream)
        sk.nvfp4_gemm(bufs["nv"], bufs["nvx"], outs["y_nv_split"], config=split, workspace=wss["nv_split"], stream=stream)
        sk.fp8_gemm(bufs["f8c"], bufs["f8s"], bufs["f8x"], outs["y_f8"], config=f8split, workspace=wss["f8"], stream=stream)
        sk.nvfp4_gemm_swiglu(bufs["sw"], bufs["swx"], outs["h"], workspace=wss["sw"], stream=stream)
        sk.nvfp4_gemm_swiglu(bufs["sw"], bufs["swx"], outs["h_split"], config=split, workspace=wss["sw_split"], stream=stream)
        sk.lm_head_gemm_argmax(bufs["lm"], bufs["lmx"], outs["idx"], 3000, workspace=wss["lm"], stream=stream)
        sk.lm_head_verify_greedy(bufs["lm"], bufs["lmx"], drafts, outs["vidx"], outs["res"], 3000,
                                 workspace=wss["lmv"], stream=stream)
        sk.fp8_gemm_packed(bufs["f8p"], bufs["f8s"], bufs["f8x"], outs["y_f8p"], config=f8split, workspace=wss["f8p"],
                           stream=stream)
        sk.layers_run(layers, [bufs["nvx4"], bufs["f8x"]], [outs["ly_nv"], outs["ly_f8p"]], workspace=wss["layers"],
                      stream=stream)
        sk.nvfp4_gemm(bufs["bal"], bufs["balx"], outs["y_bal"], config=(3, 1, 3, 1), workspace=wss["bal"], stream=stream)

    calls(torch.cuda.current_stream())
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in outs.items()}
    _check(eager["y_nv"].float().cpu().numpy(), ref_nvfp4(nv), "graph test eager nvfp4")
    _check(eager["y_nv_split"].float().cpu().numpy(), ref_nvfp4(nv), "graph test eager nvfp4 split")
    _check(eager["h_split"].float().cpu().numpy(), oracle.nvfp4_swiglu(sw["x"], sw["gate"], sw["up"]), "graph test eager swiglu split")
    assert list(eager["res"].cpu().numpy()) == [7] + [int(v) for v in want_idx] and np.array_equal(eager["idx"].cpu().numpy(), want_idx)
    assert torch.equal(eager["y_f8p"], eager["y_f8"]), "packed FP8 differs from canonical FP8"
    _check(eager["ly_nv"].float().cpu().numpy(), ref_nvfp4(nv, 4), "graph test eager layer table, NVFP4 layer")
    _check(eager["ly_f8p"].float().cpu().numpy(), ref_fp8(f8), "graph test eager layer table, packed FP8 layer")
    _check(eager["y_bal"].float().cpu().numpy(), ref_nvfp4(bal), "graph test eager balanced GEMV")
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            calls(cap)
    for rep in range(3):
        for k, v in outs.items():                          # eager clears between replays
            v.fill_(-1) if v.dtype == torch.int32 else v.fill_(float("nan"))
        for w in wss.values():
            if w is not None:
                w[sk.WORKSPACE_SYNC_BYTES:].fill_(0x5A)   # the counters stay zero at rest
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(v, eager[k]), f"replay {rep}: {k} differs from the eager call"
