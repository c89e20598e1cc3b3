"""C ABI checks that need no GPU: exports, argument validation, packer, quantizers.

Every error path here returns before the library makes any HIP call, so these
tests run on machines without a GPU.  Fake device pointers are plain integers
and are never dereferenced.
"""

import ctypes
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import fp8_quantized_skinny_amd as sk
from fp8_quantized_skinny_amd import synth
from fp8_quantized_skinny_amd._lib import lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A = 0x10000          # fake, 16-byte aligned "device" address (never touched)
MIS = 0x10008        # 8-byte aligned only


def _header_functions():
    text = open(os.path.join(ROOT, "include", "skinny.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(?:int|size_t|const char\*)\s+(\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = _header_functions()
    assert {"nvfp4_pack", "nvfp4_gemm", "fp8_gemm", "lm_head_gemm_argmax"} <= set(names)
    L = lib()
    for n in names:
        assert hasattr(L, n), n


def test_strerror_covers_all_codes():
    for s in range(7):
        assert sk.strerror(s) and sk.strerror(s) != "unknown status"
    assert sk.strerror(99) == "unknown status"


def _gemm(M=1, K=256, N=512, w=A, x=A, y=A, ws=None, wsb=0):
    return lib().nvfp4_gemm(w, x, y, M, K, N, ws, wsb, None)


def test_nvfp4_gemm_argument_errors():
    assert _gemm(w=None) == sk.EINVAL
    assert _gemm(x=None) == sk.EINVAL
    assert _gemm(y=None) == sk.EINVAL
    for M in (0, 9, -1):
        assert _gemm(M=M) == sk.ESHAPE
    for K in (0, 8, 24, 100, (1 << 20) + 16):
        assert _gemm(K=K) == sk.ESHAPE
    assert _gemm(N=0) == sk.ESHAPE
    assert _gemm(w=MIS) == sk.EALIGN
    assert _gemm(x=MIS) == sk.EALIGN
    assert _gemm(y=MIS) == sk.EALIGN


def test_explicit_config_rejections():
    L = lib()
    cfg = lambda *c: L.nvfp4_gemm_config(A, A, A, c[0], 256, 512, None, 0, None, *c[1:])
    # VALU engine is M <= 2 only; unknown engine / tile counts / wave counts / splits are rejected.
    assert cfg(3, 0, 1, 4, 1) == sk.EINVAL
    assert cfg(1, 3, 1, 4, 1) == sk.EINVAL
    # streaming engine: no K split, 1 or 2 workgroups per CU, at most 9 K spans, NVFP4 calls only
    assert cfg(1, 2, 1, 4, 2) == sk.EINVAL
    assert cfg(1, 2, 3, 4, 1) == sk.EINVAL
    assert L.nvfp4_gemm_config(A, A, A, 1, 10240, 512, None, 0, None, 2, 1, 16, 1) == sk.EINVAL
    assert L.fp8_gemm_config(A, A, A, A, 1, 256, 512, None, 0, None, 2, 1, 4, 1) == sk.EINVAL
    assert sk.config_supported(sk.OP_NVFP4, 8, 9216, 512, (2, 1, 16, 1))
    assert not sk.config_supported(sk.OP_NVFP4, 8, 9216, 512, (2, 2, 16, 1))      # 2 x 147 KB of LDS
    assert sk.config_supported(sk.OP_LM_HEAD, 8, 5120, 151936, (2, 1, 16, 1))
    assert not sk.config_supported(sk.OP_FP8, 1, 5120, 7168, (2, 1, 16, 1))
    assert cfg(1, 1, 3, 4, 1) == sk.EINVAL
    assert cfg(1, 1, 1, 17, 1) == sk.EINVAL         # at most 16 wavefronts
    assert cfg(1, 1, 2, 3, 1) == sk.EINVAL          # nw must be a multiple of ct
    assert cfg(1, 1, 1, 0, 1) == sk.EINVAL
    assert cfg(1, 1, 1, 4, 0) == sk.EINVAL
    assert cfg(1, 1, 1, 4, 2) == sk.EINVAL          # K = 256 has one K span: no split possible
    # FP8 VALU engine: M <= 4
    assert L.fp8_gemm_config(A, A, A, A, 5, 256, 512, None, 0, None, 0, 1, 4, 1) == sk.EINVAL
    assert sk.config_supported(sk.OP_FP8, 1, 5120, 7168, (0, 1, 10, 1))
    assert sk.config_supported(sk.OP_FP8, 4, 5120, 7168, (0, 1, 10, 1))
    assert not sk.config_supported(sk.OP_FP8, 5, 5120, 7168, (0, 1, 10, 1))
    # NVFP4 VALU engine: M <= 2
    assert L.lm_head_gemm_argmax_config(A, A, A, None, 3, 256, 512, A, 256, None, 0, 1, 4, 1) == sk.EINVAL
    assert L.nvfp4_gemm_config(A, A, A, 3, 256, 512, None, 0, None, 0, 1, 4, 1) == sk.EINVAL
    assert sk.config_supported(sk.OP_LM_HEAD, 1, 5120, 151936, (0, 1, 5, 1))
    assert sk.config_supported(sk.OP_LM_HEAD, 2, 5120, 151936, (0, 1, 5, 1))
    assert sk.config_supported(sk.OP_SWIGLU, 2, 5120, 17408, (0, 1, 5, 1))
    assert not sk.config_supported(sk.OP_NVFP4, 3, 5120, 17408, (0, 1, 5, 1))
    # engine 3 (VALU GEMV balanced over the CUs): plain nvfp4_gemm, M <= 2, one tile of whole K per workgroup
    for M in (1, 2):
        assert sk.config_supported(sk.OP_NVFP4, M, 5120, 17408, (3, 1, 5, 1))
        assert sk.workspace_bytes(sk.OP_NVFP4, M, 5120, 17408, (3, 1, 5, 1)) == \
            sk.WORKSPACE_SYNC_BYTES + 1024 * M * 16 * 4
    assert not sk.config_supported(sk.OP_NVFP4, 3, 5120, 17408, (3, 1, 5, 1))
    for c in ((3, 2, 10, 1), (3, 1, 3, 2), (3, 1, 4, 1)):
        assert not sk.config_supported(sk.OP_NVFP4, 1, 5120, 17408, c), c
    assert not sk.config_supported(sk.OP_LM_HEAD, 1, 5120, 17408, (3, 1, 5, 1))
    assert not sk.config_supported(sk.OP_SWIGLU, 1, 5120, 8704, (3, 1, 5, 1))
    assert L.nvfp4_gemm_swiglu_config(A, A, A, 1, 5120, 8704, A, 1 << 20, None, 3, 1, 5, 1) == sk.EINVAL
    # a K split needs its workspace
    big = lambda ws, wsb: L.nvfp4_gemm_config(A, A, A, 8, 17408, 5120, ws, wsb, None, 1, 1, 4, 5)
    need = sk.workspace_bytes(sk.OP_NVFP4, 8, 17408, 5120, (1, 1, 4, 5))
    assert need >= 5 * 320 * 512
    assert big(None, 0) == sk.EINVAL
    assert big(A, need - 1) == sk.ESIZE
    assert big(MIS, need) == sk.EALIGN


def test_verify_argument_errors():
    L = lib()
    v = lambda M=8, d=A, i=A, r=A, x=A, w=A: L.lm_head_verify_greedy(w, x, d, i, r, M, 256, 512, None, 0, None)
    assert v(d=None) == sk.EINVAL and v(r=None) == sk.EINVAL and v(i=None) == sk.EINVAL
    assert v(M=9) == sk.ESHAPE
    assert v(d=A + 2) == sk.EALIGN and v(r=A + 2) == sk.EALIGN
    # M = 1 needs no drafts: the call gets past that check and stops at the missing workspace
    assert sk.workspace_bytes(sk.OP_LM_HEAD, 1, 256, 512) > 0
    assert v(M=1, d=None) == sk.EINVAL and v(M=1, d=None, r=A + 2) == sk.EALIGN


def test_layer_table_checks_every_layer_first():
    """A table is rejected as a whole, before anything is enqueued, by the
    checks of the call each layer maps to; the workspace serves the largest layer."""
    from fp8_quantized_skinny_amd._lib import SkinnyLayer
    L = lib()

    def table(*layers):
        t = (SkinnyLayer * len(layers))()
        for i, (kind, w, sc, K, N) in enumerate(layers):
            t[i].kind, t[i].weights, t[i].scales, t[i].K, t[i].N = kind, w, sc, K, N
        return t

    ok = [(sk.LAYER_NVFP4, A, None, 256, 512), (sk.LAYER_FP8, A, A, 256, 256), (sk.LAYER_SWIGLU, A, None, 256, 40)]
    t = table(*ok)
    ptrs = (ctypes.c_void_p * 4)(A, A, A, A)
    need = max(sk.workspace_bytes(sk.OP_NVFP4, 8, 17408, 5120), sk.workspace_bytes(sk.OP_FP8, 8, 256, 256))
    big = table((sk.LAYER_NVFP4, A, None, 17408, 5120), (sk.LAYER_FP8, A, A, 256, 256))
    assert L.skinny_layers_workspace_bytes(big, 2, 8) == need > 0
    assert L.skinny_layers_workspace_bytes(t, 3, 1) == max(sk.workspace_bytes(sk.OP_NVFP4, 1, 256, 512),
                                                          sk.workspace_bytes(sk.OP_FP8, 1, 256, 256),
                                                          sk.workspace_bytes(sk.OP_SWIGLU, 1, 256, 40))
    run = lambda t, n, M=1, x=ptrs, y=ptrs, ws=None, wsb=0: L.skinny_layers_run(t, n, x, y, M, ws, wsb, None)
    assert run(None, 1) == sk.EINVAL and run(t, 0) == sk.EINVAL
    for bad, code in [((7, A, None, 256, 512), sk.EINVAL),                 # unknown kind
                      ((sk.LAYER_FP8, A, None, 256, 256), sk.EINVAL),      # FP8 without scales
                      ((sk.LAYER_NVFP4, MIS, None, 256, 512), sk.EALIGN),
                      ((sk.LAYER_NVFP4, A, None, 250, 512), sk.ESHAPE),
                      ((sk.LAYER_SWIGLU, A, None, 256, 0), sk.ESHAPE)]:
        # the bad layer last: the good ones before it must not have been enqueued either,
        # which holds because every check runs before the first launch
        assert run(table(*ok, bad), 4) == code, bad
    assert run(big, 2, M=8) == sk.EINVAL                                   # missing workspace
    assert run(t, 3, M=9) == sk.ESHAPE
    mis = (ctypes.c_void_p * 4)(A, MIS, A, A)
    assert run(t, 3, x=mis) == sk.EALIGN


def test_fp8_gemm_argument_errors():
    L = lib()
    f = lambda **k: L.fp8_gemm(k.get("w", A), k.get("s", A), k.get("x", A), k.get("y", A), k.get("M", 1),
                               k.get("K", 256), k.get("N", 256), None, 0, None)
    assert f(w=None) == sk.EINVAL and f(s=None) == sk.EINVAL
    assert f(M=9) == sk.ESHAPE and f(K=40) == sk.ESHAPE and f(N=0) == sk.ESHAPE
    assert f(w=MIS) == sk.EALIGN and f(s=A + 2) == sk.EALIGN


def test_read_probe_argument_errors():
    """The read probe checks its arguments on the host: no buffer or sink,
    misalignment and buffers smaller than one 9216-byte block are refused
    before anything reaches the GPU (the pointers here are never touched)."""
    L = lib()
    P = 0x10000
    assert L.skinny_read_probe(None, 9216, P, None) == sk.EINVAL
    assert L.skinny_read_probe(P, 9216, None, None) == sk.EINVAL
    assert L.skinny_read_probe(P + 8, 9216, P, None) == sk.EALIGN
    assert L.skinny_read_probe(P, 9216, P + 2, None) == sk.EALIGN
    assert L.skinny_read_probe(P, 9215, P, None) == sk.ESIZE
    assert L.skinny_read_probe(P, 0, P, None) == sk.ESIZE
    assert L.skinny_read_probe(P, 9216 << 31, P, None) == sk.ESIZE     # 2^31 single-wavefront groups


def test_read_probe_pattern_argument_errors():
    """Every pattern's arguments are checked on the host before any launch."""
    L = lib()
    P = 0x10000
    n = ctypes.c_size_t(0)
    call = lambda *a: L.skinny_read_probe_pattern(*a, ctypes.byref(n), None)
    assert call(None, 9216, 0, 1, 0, P) == sk.EINVAL
    assert call(P, 9216, 0, 1, 0, None) == sk.EINVAL
    assert call(P + 8, 9216, 0, 1, 0, P) == sk.EALIGN
    for pattern, a, b in ((0, 0, 0), (0, 17, 0), (1, 0, 0), (2, 17, 0), (3, 0, 0), (3, 17, 0), (4, 0, 1),
                          (4, 65536, 1), (4, 1, 0), (4, 1, 17), (5, 0, 1), (6, 1, 17), (7, 1, 1), (-1, 1, 1)):
        assert call(P, 1 << 20, pattern, a, b, P) == sk.EINVAL, (pattern, a, b)
    assert call(P, 9215, 0, 1, 0, P) == sk.ESIZE
    assert call(P, 4095, 1, 1, 0, P) == sk.ESIZE
    assert call(P, 18431, 2, 4, 0, P) == sk.ESIZE
    assert call(P, 5 * 9216 - 1, 3, 5, 0, P) == sk.ESIZE
    for pattern in (4, 5, 6):
        assert call(P, 9215, pattern, 1, 1, P) == sk.ESIZE


def test_lm_head_argument_errors():
    L = lib()
    need = sk.workspace_bytes(sk.OP_LM_HEAD, 1, 256, 512)
    assert need >= 8 * 8 + 4
    f = lambda **k: L.lm_head_gemm_argmax(k.get("w", A), k.get("x", A), k.get("idx", A), k.get("lg", None),
                                          k.get("M", 1), 256, 512, k.get("ws", A), k.get("wsb", need), None)
    assert f(idx=None) == sk.EINVAL
    assert f(ws=None) == sk.EINVAL
    assert f(wsb=need - 1) == sk.ESIZE
    assert f(ws=MIS) == sk.EALIGN
    assert f(lg=MIS) == sk.EALIGN
    assert f(idx=A + 2) == sk.EALIGN
    assert f(M=9) == sk.ESHAPE


def test_workspace_sizes():
    # no split, no argmax: no workspace
    assert sk.workspace_bytes(sk.OP_NVFP4, 1, 5120, 17408, (0, 1, 5, 1)) == 0
    assert sk.workspace_bytes(sk.OP_FP8, 4, 5120, 7168, (1, 1, 10, 1)) == 0
    # argmax: one 64-bit candidate per workgroup and row
    assert sk.workspace_bytes(sk.OP_LM_HEAD, 8, 5120, 151936, (1, 1, 5, 1)) >= 9496 * 8 * 8
    # every workspace that is not empty starts with the 128 KiB of arrival counters
    SYNC = sk.WORKSPACE_SYNC_BYTES
    assert SYNC == 1024 * 128
    # K split: fp32 partials of every split, row and column
    assert sk.workspace_bytes(sk.OP_NVFP4, 8, 17408, 5120, (1, 2, 10, 4)) == SYNC + 4 * 8 * 5120 * 4
    assert sk.workspace_bytes(sk.OP_FP8, 3, 6144, 5120, (1, 1, 4, 3)) == SYNC + 3 * 3 * 5120 * 4
    # columns rounded up to whole tile groups for the in-kernel split (2 groups of 4 tiles for 100 columns)
    assert sk.workspace_bytes(sk.OP_NVFP4, 8, 2048, 100, (1, 4, 4, 2)) == SYNC + 2 * 8 * 128 * 4
    # K split with argmax: candidates of each 256-column block of the split reduction, then the partials
    # (partials of 5 x 2 x 1008 columns: 63 whole tiles; 40320 rounded up to 256)
    assert sk.workspace_bytes(sk.OP_LM_HEAD, 2, 5120, 1000, (1, 1, 1, 5)) == SYNC + 256 + 40448
    # spans that do not cover K, or a split that leaves a workgroup without spans, are unsupported
    assert sk.workspace_bytes(sk.OP_NVFP4, 8, 17408, 5120, (1, 2, 4, 4)) == 0
    assert sk.workspace_bytes(sk.OP_NVFP4, 8, 17408, 5120, (1, 1, 9, 2)) > 0
    assert sk.workspace_bytes(sk.OP_NVFP4, 8, 17408, 5120, (1, 1, 9, 3)) == 0
    # the MFMA engine's LDS copy of x must fit: 8 rows x 16 spans do not
    assert sk.workspace_bytes(sk.OP_NVFP4, 8, 17408, 5120, (1, 1, 16, 2)) == 0
    # defaults are consistent with some explicit choice and zero for bad shapes or ops
    assert sk.workspace_bytes(sk.OP_LM_HEAD, 0, 5120, 7168) == 0
    assert sk.workspace_bytes(7, 1, 5120, 7168) == 0
    assert sk.workspace_bytes(sk.OP_NVFP4, 1, 5120, 17408, (1, 3, 4, 1)) == 0      # bad ct -> unsupported


# ------------------------------------------------------------------- packer
def _pack_raw(codes, scales, g, K, N, out, size):
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p) if a is not None else None
    sz = ctypes.c_size_t(size)
    st = lib().nvfp4_pack(p(codes), p(scales), g, K, N, p(out), ctypes.byref(sz))
    return st, sz.value


def _geom(K, N):
    ku, nt = -(-K // 1024), -(-N // 16)
    return ku, nt


def test_pack_size_and_header():
    for K, N in [(256, 512), (272, 100), (5120, 17408), (16, 1), (17408, 5120)]:
        ku, nt = _geom(K, N)
        assert sk.packed_bytes(K, N) == 256 + nt * ku * 9216
    codes = np.zeros((100, 136), np.uint8)
    scales = np.zeros((100, 17), np.uint8)
    blob = sk.nvfp4_pack(codes, scales, 0.125, 272, 100)
    h = blob[:64]
    assert bytes(h[:4]) == b"SKN4"
    assert list(h[4:28].view(np.uint32)) == [4, 272, 100, 1, 7, 9216]
    assert h[28:32].view(np.float32)[0] == np.float32(0.125)
    assert list(h[32:48].view(np.uint64)) == [256, 7 * 9216]
    assert h[48:52].view(np.float32)[0] == np.float32(0.125)          # g2 = g for a plain blob
    assert list(h[52:60].view(np.uint32)) == [0, 0]                    # kind plain, F unused


def _interleave(gate, up, F):
    """Canonical arrays of the packed SwiGLU columns, built column by column:
    packed column 16t + c is gate column 8t + c (c < 8) or up column 8t + c - 8."""
    Np = 16 * -(-F // 8)
    codes = np.zeros((Np, gate[0].shape[1]), np.uint8)
    scales = np.zeros((Np, gate[1].shape[1]), np.uint8)
    for n in range(Np):
        t, c = divmod(n, 16)
        f = 8 * t + c % 8
        if f < F:
            src = gate if c < 8 else up
            codes[n], scales[n] = src[0][f], src[1][f]
    return codes, scales


@pytest.mark.parametrize("K,F", [(256, 8), (272, 13), (2064, 3), (1024, 40)])
def test_pack_swiglu_interleaves_gate_and_up(K, F):
    rng = np.random.default_rng(K * F)
    gate = (rng.integers(0, 256, (F, K // 2), dtype=np.uint8), rng.integers(0, 0x7F, (F, K // 16), dtype=np.uint8), 0.5)
    up = (rng.integers(0, 256, (F, K // 2), dtype=np.uint8), rng.integers(0, 0x7F, (F, K // 16), dtype=np.uint8), 0.25)
    blob = sk.nvfp4_pack_swiglu(gate, up, K, F)
    Np = sk.swiglu_packed_cols(F)
    assert Np == 16 * -(-F // 8) and blob.size == sk.packed_bytes(K, Np)
    codes, scales = _interleave(gate, up, F)
    plain = sk.nvfp4_pack(codes, scales, 0.5, K, Np)
    assert np.array_equal(blob[256:], plain[256:])
    h = blob[:64]
    assert bytes(h[:4]) == b"SKN4" and list(h[4:16].view(np.uint32)) == [4, K, Np]
    assert h[28:32].view(np.float32)[0] == np.float32(0.5)
    assert h[48:52].view(np.float32)[0] == np.float32(0.25)
    assert list(h[52:60].view(np.uint32)) == [1, F]


def test_swiglu_argument_errors():
    L = lib()
    c = np.zeros((4, 128), np.uint8)
    s = np.zeros((4, 16), np.uint8)
    size = ctypes.c_size_t(0)
    P = lambda a: a.ctypes.data if a is not None else None
    pack = lambda gc=c, gs=s, gg=1.0, uc=c, us=s, ug=1.0, K=256, F=4: L.nvfp4_pack_swiglu(
        P(gc), P(gs), gg, P(uc), P(us), ug, K, F, None, ctypes.byref(size))
    assert pack() == sk.OK and size.value == sk.packed_bytes(256, 16)
    assert pack(uc=None) == sk.EINVAL
    assert pack(ug=float("nan")) == sk.EINVAL and pack(gg=-1.0) == sk.EINVAL
    assert pack(F=0) == sk.ESHAPE and pack(K=250) == sk.ESHAPE and pack(F=(1 << 23) + 1) == sk.ESHAPE
    bad = s.copy()
    bad[2, 3] = 0xFF
    out = np.zeros(size.value, np.uint8)
    assert L.nvfp4_pack_swiglu(P(c), P(s), 1.0, P(c), P(bad), 1.0, 256, 4, P(out), ctypes.byref(size)) == sk.EFORMAT
    gemm = lambda M=1, K=256, F=100, w=A, x=A, h=A: L.nvfp4_gemm_swiglu(w, x, h, M, K, F, None, 0, None)
    assert gemm(w=None) == sk.EINVAL and gemm(h=None) == sk.EINVAL
    assert gemm(M=9) == sk.ESHAPE and gemm(F=0) == sk.ESHAPE and gemm(K=24) == sk.ESHAPE
    assert gemm(F=(1 << 23) + 1) == sk.ESHAPE
    assert gemm(h=MIS) == sk.EALIGN and gemm(x=MIS) == sk.EALIGN
    # lm_head / split workspace rules carry over to the packed column count
    assert L.nvfp4_gemm_swiglu_config(A, A, A, 8, 256, 100, None, 0, None, 0, 1, 1, 1) == sk.EINVAL  # VALU is M = 1
    need = sk.workspace_bytes(sk.OP_SWIGLU, 8, 17408, 5120)
    assert need == sk.workspace_bytes(sk.OP_NVFP4, 8, 17408, 10240)
    assert gemm(M=8, K=17408, F=5120) == sk.EINVAL                     # no workspace for the K split
    assert sk.workspace_bytes(sk.OP_SWIGLU, 1, 256, 0) == 0


def test_pack_errors():
    c = np.zeros((4, 128), np.uint8)
    s = np.zeros((4, 16), np.uint8)
    out = np.zeros(sk.packed_bytes(256, 4), np.uint8)
    assert _pack_raw(c, s, 1.0, 256, 4, out, out.size)[0] == sk.OK
    assert _pack_raw(c, s, 1.0, 256, 4, out, out.size - 1)[0] == sk.ESIZE
    assert _pack_raw(None, s, 1.0, 256, 4, out, out.size)[0] == sk.EINVAL
    assert _pack_raw(c, s, float("nan"), 256, 4, out, out.size)[0] == sk.EINVAL
    assert _pack_raw(c, s, -1.0, 256, 4, out, out.size)[0] == sk.EINVAL
    assert _pack_raw(c, s, 1.0, 250, 4, out, out.size)[0] == sk.ESHAPE
    for bad in (0x7F, 0xFF):
        s2 = s.copy()
        s2[3, 15] = bad
        assert _pack_raw(c, s2, 1.0, 256, 4, out, out.size)[0] == sk.EFORMAT


@pytest.mark.parametrize("K,N", [(256, 32), (272, 20), (2064, 17)])
def test_pack_places_every_byte_once(K, N):
    """Distinct byte patterns go exactly where the documented unit layout says."""
    rng = np.random.default_rng(K + N)
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, size=(N, K // 16), dtype=np.uint8)   # no NaN codes
    blob = sk.nvfp4_pack(codes, scales, 1.0, K, N)
    ku, nt = _geom(K, N)
    units = blob[256:].reshape(ku, nt, 9, 4, 16, 16).transpose(1, 0, 2, 3, 4, 5)   # span-major -> [tile, span, ...]
    seen_c = np.zeros(codes.shape, np.int64)
    seen_s = np.zeros(scales.shape, np.int64)
    for n in range(N):
        t, c = divmod(n, 16)
        for k in range(0, K, 2):
            g, r = divmod(k, 1024)
            j, r = divmod(r, 128)
            grp, i = divmod(r, 32)
            assert units[t, g, j, grp, c, i // 2] == codes[n, k // 2]
            seen_c[n, k // 2] += 1
        for b in range(K // 16):
            g, r = divmod(16 * b, 1024)
            j, r = divmod(r, 128)
            grp, h = divmod(r, 32)
            assert units[t, g, 8, grp, c, 2 * j + h // 16] == scales[n, b]
            seen_s[n, b] += 1
    assert (seen_c == 1).all() and (seen_s == 1).all()
    # every byte of the padding (columns >= N, K >= real K) is zero
    mask = np.zeros(units.shape, bool)
    for n in range(N):
        t, c = divmod(n, 16)
        for k in range(0, K, 2):
            g, r = divmod(k, 1024)
            j, r = divmod(r, 128)
            grp, i = divmod(r, 32)
            mask[t, g, j, grp, c, i // 2] = True
        for b in range(K // 16):
            g, r = divmod(16 * b, 1024)
            j, r = divmod(r, 128)
            grp, h = divmod(r, 32)
            mask[t, g, 8, grp, c, 2 * j + h // 16] = True
    assert not units[~mask].any()


@pytest.mark.parametrize("K,N", [(512, 16), (400, 20), (1040, 33), (16, 1)])
def test_fp8_pack_places_every_byte_once(K, N):
    """Every code lands where the documented FP8 unit layout says; the rest is zero."""
    rng = np.random.default_rng(K * 7 + N)
    codes = rng.integers(1, 256, size=(N, K), dtype=np.uint8)          # no zero code, so padding is visible
    blob = sk.fp8_pack(codes, K, N)
    ku, nt = -(-K // 512), -(-N // 16)
    assert blob.size == 256 + ku * nt * 8192 == sk.fp8_packed_bytes(K, N)
    h = blob[:64]
    assert bytes(h[:4]) == b"SKF8" and list(h[4:32].view(np.uint32)) == [2, K, N, ku, nt, 8192, 0]
    units = blob[256:].reshape(ku, nt, 8, 4, 16, 16)                   # [span][tile][piece][grp][c][byte]
    seen = np.zeros(codes.shape, np.int64)
    mask = np.zeros(units.shape, bool)
    for n in range(N):
        t, col = divmod(n, 16)
        c = 2 * (col % 8) + col // 8                                     # lane c holds column 8(c%2) + c//2
        for k in range(K):
            u, r = divmod(k, 512)
            j, r = divmod(r, 128)
            grp, r = divmod(r, 32)
            hh, i = divmod(r, 16)
            assert units[u, t, 2 * j + hh, grp, c, i] == codes[n, k]
            seen[n, k] += 1
            mask[u, t, 2 * j + hh, grp, c, i] = True
    assert (seen == 1).all() and not units[~mask].any()


def test_fp8_pack_errors_and_packed_gemm_arguments():
    L = lib()
    c = np.zeros((4, 256), np.uint8)
    size = ctypes.c_size_t(0)
    assert L.fp8_pack(c.ctypes.data, 256, 4, None, ctypes.byref(size)) == sk.OK and size.value == 256 + 8192
    assert L.fp8_pack(None, 256, 4, None, ctypes.byref(size)) == sk.EINVAL
    assert L.fp8_pack(c.ctypes.data, 250, 4, None, ctypes.byref(size)) == sk.ESHAPE
    out = np.zeros(256 + 8192 - 1, np.uint8)
    size.value = out.size
    assert L.fp8_pack(c.ctypes.data, 256, 4, out.ctypes.data, ctypes.byref(size)) == sk.ESIZE
    g = lambda M=1, K=256, N=256, w=A, s=A, x=A, y=A: L.fp8_gemm_packed(w, s, x, y, M, K, N, None, 0, None)
    assert g(w=None) == sk.EINVAL and g(s=None) == sk.EINVAL
    assert g(M=9) == sk.ESHAPE and g(K=24) == sk.ESHAPE
    assert g(w=MIS) == sk.EALIGN and g(y=MIS) == sk.EALIGN and g(s=A + 2) == sk.EALIGN
    assert L.fp8_gemm_packed_config(A, A, A, A, 5, 256, 256, None, 0, None, 0, 1, 1, 1) == sk.EINVAL  # VALU: M <= 4


def test_pack_is_deterministic():
    w, _ = synth.draw(1, 384, 48, seed=2)
    c, s, g = sk.nvfp4_quantize(w)
    assert np.array_equal(sk.nvfp4_pack(c, s, g, 384, 48), sk.nvfp4_pack(c, s, g, 384, 48))


# --------------------------------------------------------------- quantizers
@pytest.mark.parametrize("K,N,seed", [(256, 512, 0), (272, 100, 1), (16, 1, 2), (1040, 129, 3)])
def test_host_quantizers_match_oracle_bit_exact(K, N, seed):
    w, _ = synth.draw(1, K, N, seed=seed)
    w[:16, 0] = 0.0                            # one all-zero block
    w[min(20, K - 1), :] = -0.0                # negative zeros
    c1, s1, g1 = sk.nvfp4_quantize(w)
    c2, s2, g2 = oracle.nvfp4_quantize(w)
    assert g1 == g2 and np.array_equal(c1, c2) and np.array_equal(s1, s2)
    a1, b1 = sk.fp8_quantize(w)
    a2, b2 = oracle.fp8_quantize(w)
    assert np.array_equal(a1, a2) and np.array_equal(b1, b2)


def test_host_quantizer_special_inputs():
    z = np.zeros((32, 8), np.float32)
    c, s, g = sk.nvfp4_quantize(z)
    assert g == 0 and not c.any() and not s.any()
    bad = np.ones((32, 8), np.float32)
    bad[3, 3] = np.inf
    with pytest.raises(sk.SkinnyError):
        sk.nvfp4_quantize(bad)
    with pytest.raises(sk.SkinnyError):
        sk.fp8_quantize(bad)
    # huge dynamic range: saturation paths agree with the oracle
    w = np.geomspace(1e-30, 1e30, 32 * 16).astype(np.float32).reshape(32, 16)
    w[::3] *= -1
    c1, s1, g1 = sk.nvfp4_quantize(w)
    c2, s2, g2 = oracle.nvfp4_quantize(w)
    assert g1 == g2 and np.array_equal(c1, c2) and np.array_equal(s1, s2)
    a1, b1 = sk.fp8_quantize(w)
    a2, b2 = oracle.fp8_quantize(w)
    assert np.array_equal(a1, a2) and np.array_equal(b1, b2)


@settings(max_examples=60, deadline=None)
@given(st.integers(1, 16), st.integers(1, 40), st.integers(0, 2**31 - 1),
       st.floats(-40.0, 26.0), st.floats(0.0, 12.0), st.floats(0.0, 0.5))
def test_host_quantizers_match_oracle_random_shapes_and_ranges(k_blocks, N, seed, lo, span, zero_frac):
    """Host quantizers against the oracle, bit for bit, on random shapes, dynamic
    ranges (magnitudes log-uniform over [10^lo, 10^(lo+span)], from float32
    subnormals up to 10^38), signs and zeros."""
    K = 16 * k_blocks
    rng = np.random.default_rng(seed)
    mag = 10.0 ** rng.uniform(lo, lo + span, size=(K, N))
    w = (np.where(rng.random((K, N)) < 0.5, -1.0, 1.0) * mag).astype(np.float32)
    w[rng.random((K, N)) < zero_frac] = 0.0
    assert np.isfinite(w).all()                # 10^38 is below the float32 maximum
    c1, s1, g1 = sk.nvfp4_quantize(w)
    c2, s2, g2 = oracle.nvfp4_quantize(w)
    assert g1 == g2 and np.array_equal(c1, c2) and np.array_equal(s1, s2)
    a1, b1 = sk.fp8_quantize(w)
    a2, b2 = oracle.fp8_quantize(w)
    assert np.array_equal(a1, a2) and np.array_equal(b1, b2)


def _has_gpu():
    import torch
    return torch.cuda.device_count() > 0      # counts devices without initialising one


@pytest.mark.skipif(_has_gpu(), reason="launches with fake device pointers: only where no GPU is present")
def test_default_kernel_choice_is_always_supported():
    """For every op and a spread of shapes, the library's own pick passes its checks.

    With fake device pointers a call that passes every host check fails only at
    the launch (no GPU here: SKINNY_EHIP); an unsupported pick would be EINVAL.
    On a machine with a GPU the launch would read the fake addresses, so the
    test is skipped there."""
    L = lib()
    big = 1 << 40
    for M in range(1, 9):
        for K in (16, 256, 1040, 5120, 9216, 10240, 17408, 1 << 20):
            for N in (1, 16, 17, 40, 5120, 151936):
                assert L.nvfp4_gemm(A, A, A, M, K, N, A, big, None) == sk.EHIP, (M, K, N)
                assert L.fp8_gemm(A, A, A, A, M, K, N, A, big, None) == sk.EHIP, (M, K, N)
                assert L.lm_head_gemm_argmax(A, A, A, None, M, K, N, A, big, None) == sk.EHIP, (M, K, N)
                assert L.nvfp4_gemm_swiglu(A, A, A, M, K, N, A, big, None) == sk.EHIP, (M, K, N)


def test_default_config_query():
    """skinny_default_config returns a choice the library supports for the same op, M and K,
    and rejects bad ops, shapes and NULL outputs before touching them."""
    for op in (sk.OP_NVFP4, sk.OP_FP8, sk.OP_LM_HEAD, sk.OP_SWIGLU):
        for M in (1, 2, 4, 8):
            for K, N in ((256, 512), (5120, 17408), (17408, 5120), (5120, 151936), (1040, 40)):
                cfg = sk.default_config(op, M, K, N)
                assert sk.config_supported(op, M, K, N, cfg), (op, M, K, N, cfg)
                assert sk.workspace_bytes(op, M, K, N, cfg) == sk.workspace_bytes(op, M, K, N)
    # 1088 tiles on 256 CUs (the count assumed without a GPU, and MI355X's): the balanced GEMV
    # at M <= 2; 1024 tiles divide evenly and keep the plain whole-K choice at M = 1.
    for M in (1, 2):
        assert sk.default_config(sk.OP_NVFP4, M, 5120, 17408) == (3, 1, 5, 1)
    assert sk.default_config(sk.OP_NVFP4, 1, 5120, 16384) == (0, 1, 5, 1)
    assert sk.default_config(sk.OP_SWIGLU, 1, 5120, 8704)[0] != 3
    L = lib()
    v = [ctypes.c_int() for _ in range(4)]
    refs = [ctypes.byref(c) for c in v]
    assert L.skinny_default_config(4, 1, 256, 512, *refs) == sk.EINVAL
    assert L.skinny_default_config(0, 9, 256, 512, *refs) == sk.ESHAPE
    assert L.skinny_default_config(0, 1, 250, 512, *refs) == sk.ESHAPE
    assert L.skinny_default_config(0, 1, 256, 512, None, *refs[1:]) == sk.EINVAL


def test_noalloc_argument_errors_before_any_hip_call():
    """nvfp4_gemm_noalloc rejects bad arguments, and shapes whose kernel choice
    needs more scratch than its device array holds, on the host (no GPU here)."""
    L = lib()
    assert L.nvfp4_gemm_noalloc(None, A, A, 1, 256, 512, None) == sk.EINVAL
    assert L.nvfp4_gemm_noalloc(A, A, A, 9, 256, 512, None) == sk.ESHAPE
    assert L.nvfp4_gemm_noalloc(A, A, A, 1, 250, 512, None) == sk.ESHAPE
    assert L.nvfp4_gemm_noalloc(A + 8, A, A, 1, 256, 512, None) == sk.EALIGN
    assert L.nvfp4_gemm_noalloc(A, A, A + 2, 1, 256, 512, None) == sk.EALIGN
    big = (8, 1 << 20, 4096)
    assert sk.workspace_bytes(sk.OP_NVFP4, *big) > sk.NOALLOC_SCRATCH_BYTES
    assert L.nvfp4_gemm_noalloc(A, A, A, *big, None) == sk.ESIZE
    # the down projection at M = 8 (a nine-way K split) fits
    assert 0 < sk.workspace_bytes(sk.OP_NVFP4, 8, 17408, 5120) <= sk.NOALLOC_SCRATCH_BYTES
    if not _has_gpu():      # with a GPU the fake pointers would reach a kernel
        assert L.nvfp4_gemm_noalloc(A, A, A, 8, 17408, 5120, None) == sk.EHIP
