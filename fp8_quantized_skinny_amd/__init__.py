"""Weight-only quantized skinny GEMM for MI355X (gfx950): Python binding.

The functions below have the names of the C ABI in include/skinny.h and only
marshal arguments: host arrays are NumPy, device buffers are torch tensors
(torch is used for device memory and streams only).  Every GEMM runs in the
HIP kernels of libskinny.so; there is no other code path.  If the library
cannot be loaded, the first call raises.

    y = x . dequant(W),   x fp16 [M, K] (M = 1..8),  y fp16 [M, N]
"""

import ctypes

import numpy as np

from ._lib import lib

OK, EINVAL, ESHAPE, EALIGN, ESIZE, EHIP, EFORMAT = range(7)
OP_NVFP4, OP_FP8, OP_LM_HEAD, OP_SWIGLU = 0, 1, 2, 3
LAYER_NVFP4, LAYER_FP8, LAYER_SWIGLU, LAYER_FP8_PACKED = 0, 1, 2, 3
ENGINE_VALU, ENGINE_MFMA, ENGINE_STREAM = 0, 1, 2


class SkinnyError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = lib().skinny_strerror(status).decode()
        super().__init__(f"{where}: status {status} ({msg})")


def _check(status, where):
    if status != OK:
        raise SkinnyError(status, where)


def _host_ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dev(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA (HIP) torch tensor")
    if t.device.index != torch.cuda.current_device():
        # The kernels run on the current device; a buffer of another device
        # would be passed to them as a foreign address.
        raise ValueError(f"{name} is on {t.device}, but the current device is cuda:{torch.cuda.current_device()}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def workspace_bytes(op, M, K, N, config=None):
    """Workspace bytes of a call; config = (engine, ct, nw, ksplit) or None for the library's pick."""
    if config is None:
        return int(lib().skinny_workspace_bytes(op, M, K, N))
    return int(lib().skinny_workspace_bytes_config(op, M, K, N, *config))


def default_config(op, M, K, N):
    """The library's own kernel choice (engine, ct, nw, ksplit) for this op and shape."""
    v = [ctypes.c_int() for _ in range(4)]
    _check(lib().skinny_default_config(op, M, K, N, *[ctypes.byref(c) for c in v]), "skinny_default_config")
    return tuple(c.value for c in v)


def config_supported(op, M, K, N, config):
    """True if the explicit kernel choice (engine, ct, nw, ksplit) is supported for this op and shape."""
    return bool(lib().skinny_config_supported(op, M, K, N, *config))


def _workspace(workspace, need, where):
    import torch
    if need == 0 and workspace is None:
        return None, 0
    if workspace is None or workspace.numel() < need:
        raise ValueError(f"{where}: a workspace of at least {need} bytes is required")
    return _dev(workspace, torch.uint8, "workspace"), workspace.numel()


def new_workspace(nbytes, fill=None, device=None):
    """A device workspace of nbytes (None if nbytes is 0), ready for its first call: its leading
    WORKSPACE_SYNC_BYTES are zero (the arrival counters of the in-kernel K-split reduction, which
    every call leaves zero).  fill: byte value for the rest (default zero); calls write every other
    byte they read, so any value works there."""
    import torch
    if not nbytes:
        return None
    if fill is None:
        return torch.zeros(nbytes, dtype=torch.uint8, device=device or "cuda")
    ws = torch.full((nbytes,), fill, dtype=torch.uint8, device=device or "cuda")
    ws[:WORKSPACE_SYNC_BYTES].zero_()
    return ws


def strerror(status):
    return lib().skinny_strerror(status).decode()


# ---------------------------------------------------------------- host-side
def nvfp4_quantize(w):
    """w float32 [K, N] (host) -> (codes u8 [N, K/2], scales u8 [N, K/16], g float)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    K, N = w.shape
    codes = np.empty((N, K // 2), np.uint8)
    scales = np.empty((N, max(K // 16, 1)), np.uint8)
    g = ctypes.c_float()
    _check(lib().nvfp4_quantize(_host_ptr(w), K, N, _host_ptr(codes), _host_ptr(scales), ctypes.byref(g)),
           "nvfp4_quantize")
    return codes, scales, np.float32(g.value)


def fp8_quantize(w):
    """w float32 [K, N] (host) -> (codes u8 [N, K] E4M3FN, scales f32 [ceil(N/128), ceil(K/128)])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    K, N = w.shape
    codes = np.empty((N, K), np.uint8)
    scales = np.empty((-(-N // 128), -(-K // 128)), np.float32)
    _check(lib().fp8_quantize(_host_ptr(w), K, N, _host_ptr(codes), _host_ptr(scales)), "fp8_quantize")
    return codes, scales


def nvfp4_pack(codes, scales, g, K, N):
    """Canonical NVFP4 arrays (host) -> packed blob (host uint8 array) for the GEMM calls."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    if codes.size < N * (K // 2) or scales.size < N * (K // 16):
        raise ValueError("codes/scales smaller than N x K/2 / N x K/16")
    size = ctypes.c_size_t(0)
    _check(lib().nvfp4_pack(_host_ptr(codes), _host_ptr(scales), float(g), K, N, None, ctypes.byref(size)),
           "nvfp4_pack")
    out = np.zeros(size.value, np.uint8)
    _check(lib().nvfp4_pack(_host_ptr(codes), _host_ptr(scales), float(g), K, N, _host_ptr(out),
                            ctypes.byref(size)), "nvfp4_pack")
    return out


def nvfp4_pack_swiglu(gate, up, K, F):
    """Pack a gate/up pair for nvfp4_gemm_swiglu.  gate, up: (codes [F][K/2], scales [F][K/16], g)
    canonical NVFP4 arrays (host) with their own per-tensor scales.  Returns the host uint8 blob of
    N = 16 * ceil(F / 8) columns, gate and up interleaved by eight (see nvfp4_pack_swiglu in skinny.h)."""
    arrs = []
    for codes, scales, g in (gate, up):
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        scales = np.ascontiguousarray(scales, dtype=np.uint8)
        if codes.size < F * (K // 2) or scales.size < F * (K // 16):
            raise ValueError("codes/scales smaller than F x K/2 / F x K/16")
        arrs.append((codes, scales, float(g)))
    (gc, gs, gg), (uc, us, ug) = arrs
    size = ctypes.c_size_t(0)
    args = (_host_ptr(gc), _host_ptr(gs), gg, _host_ptr(uc), _host_ptr(us), ug, K, F)
    _check(lib().nvfp4_pack_swiglu(*args, None, ctypes.byref(size)), "nvfp4_pack_swiglu")
    out = np.zeros(size.value, np.uint8)
    _check(lib().nvfp4_pack_swiglu(*args, _host_ptr(out), ctypes.byref(size)), "nvfp4_pack_swiglu")
    return out


def swiglu_packed_cols(F):
    """Columns of the packed blob of a SwiGLU pair of F columns each."""
    return 16 * (-(-F // 8))


def packed_bytes(K, N):
    size = ctypes.c_size_t(0)
    dummy = np.zeros(1, np.uint8)
    _check(lib().nvfp4_pack(_host_ptr(dummy), _host_ptr(dummy), 0.0, K, N, None, ctypes.byref(size)),
           "nvfp4_pack")
    return size.value


# -------------------------------------------------------------- device calls
def _shape_checks(x, M, K, out, N, name):
    if x.dim() != 2 or x.shape[0] != M or x.shape[1] != K:
        raise ValueError(f"x must be [M, K] = [{M}, {K}]")
    if out is not None and out.numel() < M * N:
        raise ValueError(f"{name} must hold M x N = {M} x {N} elements")


def nvfp4_gemm(w_packed, x, y, K=None, N=None, workspace=None, stream=None, config=None):
    """y[M, N] fp16 = x[M, K] fp16 . dequant(W); w_packed: CUDA uint8 blob from nvfp4_pack.

    config: optional (engine, ct, nw, ksplit) kernel choice; default lets the library pick.
    workspace: CUDA uint8 tensor of at least workspace_bytes(OP_NVFP4, ...) bytes when that is > 0,
    from new_workspace() (its first WORKSPACE_SYNC_BYTES zero before the first call; every call
    leaves them zero; the rest scratch); not shared by calls that overlap in time."""
    import torch
    M, Kx = x.shape
    K = Kx if K is None else K
    N = y.shape[-1] if N is None else N
    _shape_checks(x, M, K, y, N, "y")
    if w_packed.numel() < packed_bytes(K, N):
        raise ValueError("w_packed is smaller than the blob for this K, N")
    wp = _dev(w_packed, torch.uint8, "w_packed")
    xp, yp = _dev(x, torch.float16, "x"), _dev(y, torch.float16, "y")
    ws, wsb = _workspace(workspace, workspace_bytes(OP_NVFP4, M, K, N, config), "nvfp4_gemm")
    if config is None:
        st = lib().nvfp4_gemm(wp, xp, yp, M, K, N, ws, wsb, _stream(stream))
    else:
        st = lib().nvfp4_gemm_config(wp, xp, yp, M, K, N, ws, wsb, _stream(stream), *config)
    _check(st, "nvfp4_gemm")
    return y


NOALLOC_SCRATCH_BYTES = 8 << 20
WORKSPACE_SYNC_BYTES = 128 << 10   # the leading bytes of a workspace that must be zero before its first use


def nvfp4_gemm_noalloc(w_packed, x, y, K=None, N=None, stream=None):
    """nvfp4_gemm without a workspace, for callers that cannot allocate: a K split's
    partial sums go to the library's own device array (NOALLOC_SCRATCH_BYTES per GPU).
    Calls that overlap in time on one GPU race.  Shapes whose kernel choice needs more
    scratch raise SkinnyError (ESIZE)."""
    import torch
    M, Kx = x.shape
    K = Kx if K is None else K
    N = y.shape[-1] if N is None else N
    _shape_checks(x, M, K, y, N, "y")
    if w_packed.numel() < packed_bytes(K, N):
        raise ValueError("w_packed is smaller than the blob for this K, N")
    wp = _dev(w_packed, torch.uint8, "w_packed")
    xp, yp = _dev(x, torch.float16, "x"), _dev(y, torch.float16, "y")
    _check(lib().nvfp4_gemm_noalloc(wp, xp, yp, M, K, N, _stream(stream)), "nvfp4_gemm_noalloc")
    return y


def nvfp4_gemm_swiglu(w_packed, x, h, workspace=None, stream=None, config=None):
    """h[M, F] fp16 = silu(x . Wg~) * (x . Wu~); w_packed: CUDA uint8 blob from nvfp4_pack_swiglu.

    config: optional (engine, ct, nw, ksplit) for the packed blob's 16 * ceil(F / 8) columns.
    workspace: CUDA uint8 tensor of at least workspace_bytes(OP_SWIGLU, M, K, F, config) bytes,
    from new_workspace() (as for nvfp4_gemm)."""
    import torch
    M, K = x.shape
    F = h.shape[-1]
    _shape_checks(x, M, K, h, F, "h")
    if w_packed.numel() < packed_bytes(K, swiglu_packed_cols(F)):
        raise ValueError("w_packed is smaller than the SwiGLU blob for this K, F")
    wp = _dev(w_packed, torch.uint8, "w_packed")
    xp, hp = _dev(x, torch.float16, "x"), _dev(h, torch.float16, "h")
    ws, wsb = _workspace(workspace, workspace_bytes(OP_SWIGLU, M, K, F, config), "nvfp4_gemm_swiglu")
    if config is None:
        st = lib().nvfp4_gemm_swiglu(wp, xp, hp, M, K, F, ws, wsb, _stream(stream))
    else:
        st = lib().nvfp4_gemm_swiglu_config(wp, xp, hp, M, K, F, ws, wsb, _stream(stream), *config)
    _check(st, "nvfp4_gemm_swiglu")
    return h


def fp8_pack(codes, K, N):
    """Canonical FP8 codes [N][K] (host) -> packed blob (host uint8 array) for fp8_gemm_packed."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    if codes.size < N * K:
        raise ValueError("codes smaller than N x K")
    size = ctypes.c_size_t(0)
    _check(lib().fp8_pack(_host_ptr(codes), K, N, None, ctypes.byref(size)), "fp8_pack")
    out = np.zeros(size.value, np.uint8)
    _check(lib().fp8_pack(_host_ptr(codes), K, N, _host_ptr(out), ctypes.byref(size)), "fp8_pack")
    return out


def fp8_packed_bytes(K, N):
    size = ctypes.c_size_t(0)
    dummy = np.zeros(1, np.uint8)
    _check(lib().fp8_pack(_host_ptr(dummy), K, N, None, ctypes.byref(size)), "fp8_pack")
    return size.value


def fp8_gemm_packed(w_packed, block_scales, x, y, workspace=None, stream=None, config=None):
    """y[M, N] fp16 = x . (E4M3(c) * S) with the codes as an fp8_pack blob (CUDA uint8)."""
    import torch
    M, K = x.shape
    N = y.shape[-1]
    _shape_checks(x, M, K, y, N, "y")
    if w_packed.numel() < fp8_packed_bytes(K, N) or block_scales.numel() < (-(-N // 128)) * (-(-K // 128)):
        raise ValueError("w_packed or block_scales smaller than the shape requires")
    wp = _dev(w_packed, torch.uint8, "w_packed")
    sp = _dev(block_scales, torch.float32, "block_scales")
    xp, yp = _dev(x, torch.float16, "x"), _dev(y, torch.float16, "y")
    ws, wsb = _workspace(workspace, workspace_bytes(OP_FP8, M, K, N, config), "fp8_gemm_packed")
    if config is None:
        st = lib().fp8_gemm_packed(wp, sp, xp, yp, M, K, N, ws, wsb, _stream(stream))
    else:
        st = lib().fp8_gemm_packed_config(wp, sp, xp, yp, M, K, N, ws, wsb, _stream(stream), *config)
    _check(st, "fp8_gemm_packed")
    return y


def fp8_gemm(w, block_scales, x, y, workspace=None, stream=None, config=None):
    """y[M, N] fp16 = x . (E4M3(w) * S); w CUDA uint8 [N, K], block_scales CUDA f32 [N/128, K/128]."""
    import torch
    M, K = x.shape
    N = w.shape[0]
    _shape_checks(x, M, K, y, N, "y")
    if w.numel() < N * K or block_scales.numel() < (-(-N // 128)) * (-(-K // 128)):
        raise ValueError("w or block_scales smaller than the shape requires")
    wp = _dev(w, torch.uint8, "w")
    sp = _dev(block_scales, torch.float32, "block_scales")
    xp, yp = _dev(x, torch.float16, "x"), _dev(y, torch.float16, "y")
    ws, wsb = _workspace(workspace, workspace_bytes(OP_FP8, M, K, N, config), "fp8_gemm")
    if config is None:
        st = lib().fp8_gemm(wp, sp, xp, yp, M, K, N, ws, wsb, _stream(stream))
    else:
        st = lib().fp8_gemm_config(wp, sp, xp, yp, M, K, N, ws, wsb, _stream(stream), *config)
    _check(st, "fp8_gemm")
    return y


def lm_head_gemm_argmax(w_packed, x, idx, N, logits=None, workspace=None, stream=None, config=None):
    """idx[M] int32 = per-row argmax over the fp32 logits of x . dequant(W) (ties -> lowest n).

    workspace: CUDA uint8 tensor of at least workspace_bytes(OP_LM_HEAD, ...) bytes, from
    new_workspace() (as for nvfp4_gemm)."""
    import torch
    M, K = x.shape
    _shape_checks(x, M, K, logits, N, "logits")
    if idx.numel() < M:
        raise ValueError("idx must hold M elements")
    if w_packed.numel() < packed_bytes(K, N):
        raise ValueError("w_packed is smaller than the blob for this K, N")
    ws, wsb = _workspace(workspace, workspace_bytes(OP_LM_HEAD, M, K, N, config), "lm_head_gemm_argmax")
    wp = _dev(w_packed, torch.uint8, "w_packed")
    xp, ip = _dev(x, torch.float16, "x"), _dev(idx, torch.int32, "idx")
    lp = None if logits is None else _dev(logits, torch.float16, "logits")
    if config is None:
        st = lib().lm_head_gemm_argmax(wp, xp, ip, lp, M, K, N, ws, wsb, _stream(stream))
    else:
        st = lib().lm_head_gemm_argmax_config(wp, xp, ip, lp, M, K, N, ws, wsb, _stream(stream), *config)
    _check(st, "lm_head_gemm_argmax")
    return idx


def lm_head_verify_greedy(w_packed, x, drafts, idx, result, N, workspace=None, stream=None, config=None):
    """Greedy verification of one speculative round on the device.

    x: CUDA fp16 [M, K] (row 0 after the last accepted token, row m after draft m);
    drafts: CUDA int32 [M - 1] (None if M == 1); idx: CUDA int32 [M] (per-row argmax);
    result: CUDA int32 [M + 1] -> [L, committed tokens (L + 1), -1 ...].
    workspace: as lm_head_gemm_argmax (op OP_LM_HEAD)."""
    import torch
    M, K = x.shape
    _shape_checks(x, M, K, None, N, "x")
    if idx.numel() < M or result.numel() < M + 1 or (M > 1 and (drafts is None or drafts.numel() < M - 1)):
        raise ValueError("idx must hold M, result M + 1 and drafts M - 1 elements")
    if w_packed.numel() < packed_bytes(K, N):
        raise ValueError("w_packed is smaller than the blob for this K, N")
    ws, wsb = _workspace(workspace, workspace_bytes(OP_LM_HEAD, M, K, N, config), "lm_head_verify_greedy")
    wp = _dev(w_packed, torch.uint8, "w_packed")
    xp = _dev(x, torch.float16, "x")
    dp = None if drafts is None else _dev(drafts, torch.int32, "drafts")
    ip, rp = _dev(idx, torch.int32, "idx"), _dev(result, torch.int32, "result")
    if config is None:
        st = lib().lm_head_verify_greedy(wp, xp, dp, ip, rp, M, K, N, ws, wsb, _stream(stream))
    else:
        st = lib().lm_head_verify_greedy_config(wp, xp, dp, ip, rp, M, K, N, ws, wsb, _stream(stream), *config)
    _check(st, "lm_head_verify_greedy")
    return result


def _layer_table(layers):
    """[(kind, weights, scales or None, K, N)] -> ctypes array of skinny_layer (weights/scales: CUDA tensors)."""
    import torch
    from ._lib import SkinnyLayer
    table = (SkinnyLayer * len(layers))()
    for i, (kind, w, sc, K, N) in enumerate(layers):
        table[i].kind = kind
        table[i].weights = _dev(w, torch.uint8, f"layers[{i}].weights").value
        table[i].scales = None if sc is None else _dev(sc, torch.float32, f"layers[{i}].scales").value
        table[i].K, table[i].N = K, N
    return table


def layers_workspace_bytes(layers, M):
    """Workspace bytes that serve every layer of a mixed-allocation table at M rows."""
    return int(lib().skinny_layers_workspace_bytes(_layer_table(layers), len(layers), M))


def layers_run(layers, xs, ys, workspace=None, stream=None):
    """Run a mixed-allocation layer table: layer i maps xs[i] (CUDA fp16 [M, K_i]) to ys[i]
    ([M, N_i]) with nvfp4_gemm, fp8_gemm or nvfp4_gemm_swiglu according to its kind.

    layers: [(kind, weights, scales or None, K, N)], kind LAYER_NVFP4, LAYER_FP8 or LAYER_SWIGLU;
    weights: the packed blob or the FP8 codes (CUDA uint8), scales: FP8 block scales (CUDA f32)."""
    import torch
    n = len(layers)
    if len(xs) != n or len(ys) != n:
        raise ValueError("one x and one y per layer")
    M = xs[0].shape[0]
    for i, ((kind, w, sc, K, N), x, y) in enumerate(zip(layers, xs, ys)):
        _shape_checks(x, M, K, y, N, f"ys[{i}]")
        if kind in (LAYER_FP8, LAYER_FP8_PACKED):
            need = N * K if kind == LAYER_FP8 else fp8_packed_bytes(K, N)
            small = w.numel() < need or sc is None or sc.numel() < (-(-N // 128)) * (-(-K // 128))
        else:
            small = w.numel() < packed_bytes(K, swiglu_packed_cols(N) if kind == LAYER_SWIGLU else N)
        if small:
            raise ValueError(f"layers[{i}]: weights or scales smaller than its shape requires")
    table = _layer_table(layers)
    xp = (ctypes.c_void_p * n)(*[_dev(x, torch.float16, "x").value for x in xs])
    yp = (ctypes.c_void_p * n)(*[_dev(y, torch.float16, "y").value for y in ys])
    ws, wsb = _workspace(workspace, int(lib().skinny_layers_workspace_bytes(table, n, M)), "skinny_layers_run")
    _check(lib().skinny_layers_run(table, n, xp, yp, M, ws, wsb, _stream(stream)), "skinny_layers_run")
    return ys
