"""Python binding of ``libssnvfp4.so`` — NVFP4 / 2:4 weight-quantised GEMM for MI355X (gfx950).

Argument marshalling only: every step runs in the library's HIP kernels. PyTorch supplies
device memory and the current stream. The functions have the names of the C entry points
declared in ``include/ssnvfp4.h``; outputs are allocated here with torch when not given.
If the shared library is missing, every call raises (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssnvfp4.so")

SSN_OK, SSN_E_NULL, SSN_E_SHAPE, SSN_E_ALIGN, SSN_E_DTYPE, SSN_E_ALGO, SSN_E_HIP, SSN_E_RANGE = range(8)
SSN_F32, SSN_BF16 = 0, 1
ALGO_AUTO, ALGO_VALU, ALGO_MFMA, ALGO_SMFMAC, ALGO_GATHER, ALGO_DECOMPRESS_MFMA, ALGO_STREAM = 0, 1, 2, 3, 4, 5, 6
ALGO_NAMES = {ALGO_AUTO: "auto", ALGO_VALU: "valu", ALGO_MFMA: "mfma", ALGO_SMFMAC: "smfmac", ALGO_GATHER: "gather",
              ALGO_DECOMPRESS_MFMA: "decompress_mfma", ALGO_STREAM: "stream"}
EPI_NONE, EPI_SILU_GATE = 0, 1
MX_ROWS, MX_TILED = 0, 1
WLAYOUT_ROWS, WLAYOUT_KTILE64 = 0, 1
PROBE_BF16, PROBE_FP4 = 0, 1

_vp, _i64, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
_SIGS = {
    "ssn_last_error": ([], ctypes.c_char_p),
    "ssn_version": ([], _int),
    "nvfp4_quantize": ([_vp, _int, _i64, _i64, _vp, _vp, _vp, _vp, _vp], _int),
    "nvfp4_dequantize": ([_vp, _vp, _vp, _i64, _i64, _vp, _int, _vp], _int),
    "nvfp4_sp24_produce": ([_vp, _int, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp], _int),
    "sp24_prune": ([_vp, _int, _i64, _i64, _vp, _vp, _vp], _int),
    "sp24_check": ([_vp, _i64, _i64, _vp, _vp, _vp], _int),
    "sp24_compress": ([_vp, _i64, _i64, _vp, _vp, _vp, _vp], _int),
    "sp24_decompress": ([_vp, _vp, _i64, _i64, _vp, _vp], _int),
    "gemm_nvfp4_dense": ([_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _int, _int, _vp, _vp], _int),
    "gemm_nvfp4_sp24": ([_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _int, _int, _vp, _vp], _int),
    "moe_route_workspace_bytes": ([_i64, _int, _int], _i64),
    "moe_route": ([_vp, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp], _int),
    "moe_grouped_gemm_nvfp4": ([_vp, _i64, _vp, _vp, _int, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp,
                                _int, _vp, _int, _int, _vp, _vp], _int),
    "moe_pack_ktiles": ([_vp, _i64, _i64, _i64, _i64, _vp, _vp], _int),
    "moe_combine": ([_vp, _int, _i64, _vp, _vp, _i64, _int, _i64, _vp, _vp], _int),
    "moe_ffn_workspace_bytes": ([_i64, _int, _int, _i64, _i64], _i64),
    "moe_nvfp4_ffn": ([_vp, _i64, _i64, _vp, _vp, _int, _int, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp, _vp,
                       _vp, _vp, _vp, _vp, _vp, _i64, _vp], _int),
    "mxfp4_tiled_bytes": ([_i64, _i64, _vp], _i64),
    "mxfp4_quantize": ([_vp, _int, _i64, _i64, _int, _vp, _vp, _vp], _int),
    "gemm_mxfp4": ([_vp, _vp, _i64, _vp, _vp, _i64, _i64, _vp, _int, _int, _vp, _vp], _int),
    "moe_nvfp4_ffn_noalloc": ([_vp, _i64, _i64, _vp, _vp, _int, _int, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp,
                               _vp, _vp, _vp, _vp, _vp, _vp], _int),
    "mfma_probe_sink_floats": ([], _i64),
    "mfma_probe": ([_int, _int, _int, ctypes.c_uint32, _vp, _vp, _vp], _int),
}

_lib = None


class SsnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[status {status}] {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded shared library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python structured_sparse_nvfp4_amd/build.py` (no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes, f.restype = args, res
        _lib = L
    return _lib


def _check(status: int):
    if status != SSN_OK:
        raise SsnError(status, lib().ssn_last_error().decode())


class Prepared:
    """A call with its arguments already marshalled (tensors, sizes, stream): calling it issues
    the C entry point with no per-call Python work beyond the ctypes call itself. Used to keep the
    host ahead of the GPU when timing short kernels. The tensors must stay alive."""

    def __init__(self, fname, cargs, keep):
        self.f = getattr(lib(), fname)
        self.cargs = cargs
        self.keep = keep

    def __call__(self):
        st = self.f(*self.cargs)
        if st:
            _check(st)


def _run(fname, cargs, prepare, keep, result):
    if prepare:   # the prepared call holds its outputs too: they must outlive every later call
        return Prepared(fname, cargs, (keep, result)), result
    _check(getattr(lib(), fname)(*cargs))
    return result


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev=None):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t, dtype, name, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _wdt(W):
    if W.dtype == torch.float32:
        return SSN_F32
    if W.dtype == torch.bfloat16:
        return SSN_BF16
    raise TypeError(f"weights must be float32 or bfloat16, got {W.dtype}")


def version() -> int:
    return lib().ssn_version()


def nvfp4_quantize(W, tensor_scale_in=None, codes=None, scales=None, tensor_scale_out=None, prepare=False):
    """NVFP4-quantise W [N, K] (f32 or bf16). Returns (codes u8 [N,K/2], scales u8 [N,K/16], s_t f32 [1])."""
    N, K = W.shape
    _need(W, W.dtype, "W")
    dev = W.device
    codes = codes if codes is not None else torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    scales = scales if scales is not None else torch.empty((N, K // 16), dtype=torch.uint8, device=dev)
    ts = tensor_scale_out if tensor_scale_out is not None else torch.empty(1, dtype=torch.float32, device=dev)
    _need(codes, torch.uint8, "codes", (N, K // 2)); _need(scales, torch.uint8, "scales", (N, K // 16))
    _need(ts, torch.float32, "tensor_scale_out", (1,))
    if tensor_scale_in is not None:
        _need(tensor_scale_in, torch.float32, "tensor_scale_in", (1,))
    cargs = (_ptr(W), _wdt(W), N, K, _ptr(tensor_scale_in), _ptr(codes), _ptr(scales), _ptr(ts), _stream(dev))
    return _run("nvfp4_quantize", cargs, prepare, (W, tensor_scale_in), (codes, scales, ts))


def nvfp4_dequantize(codes, scales, tensor_scale, out_dtype=torch.float32, out=None):
    N, Kh = codes.shape
    K = 2 * Kh
    _need(codes, torch.uint8, "codes"); _need(scales, torch.uint8, "scales", (N, K // 16))
    _need(tensor_scale, torch.float32, "tensor_scale", (1,))
    out = out if out is not None else torch.empty((N, K), dtype=out_dtype, device=codes.device)
    dt = SSN_F32 if out.dtype == torch.float32 else SSN_BF16 if out.dtype == torch.bfloat16 else None
    if dt is None:
        raise TypeError("out must be float32 or bfloat16")
    _need(out, out.dtype, "out", (N, K))
    _check(lib().nvfp4_dequantize(_ptr(codes), _ptr(scales), _ptr(tensor_scale), N, K, _ptr(out), dt,
                                  _stream(codes.device)))
    return out


def nvfp4_sp24_produce(W, tensor_scale_in=None, vals=None, meta=None, scales=None, tensor_scale_out=None,
                       codes=None, want_codes=False, bad_groups=None, prepare=False):
    """Prune -> quantise -> compress W [N, K] (f32 or bf16) in one pass, bit-identical to sp24_prune,
    nvfp4_quantize and sp24_compress in turn. Returns (vals u8 [N,K/4], meta u8 [N,K/8], scales u8
    [N,K/16], s_t f32 [1], bad_groups int64 [1] device, codes u8 [N,K/2] of the pruned tensor or None)."""
    N, K = W.shape
    _need(W, W.dtype, "W")
    dev = W.device
    u8 = dict(dtype=torch.uint8, device=dev)
    vals = vals if vals is not None else torch.empty((N, K // 4), **u8)
    meta = meta if meta is not None else torch.empty((N, K // 8), **u8)
    scales = scales if scales is not None else torch.empty((N, K // 16), **u8)
    ts = tensor_scale_out if tensor_scale_out is not None else torch.empty(1, dtype=torch.float32, device=dev)
    bad = bad_groups if bad_groups is not None else torch.empty(1, dtype=torch.int64, device=dev)
    if codes is None and want_codes:
        codes = torch.empty((N, K // 2), **u8)
    _need(vals, torch.uint8, "vals", (N, K // 4)); _need(meta, torch.uint8, "meta", (N, K // 8))
    _need(scales, torch.uint8, "scales", (N, K // 16)); _need(ts, torch.float32, "tensor_scale_out", (1,))
    _need(bad, torch.int64, "bad_groups", (1,))
    if codes is not None:
        _need(codes, torch.uint8, "codes", (N, K // 2))
    if tensor_scale_in is not None:
        _need(tensor_scale_in, torch.float32, "tensor_scale_in", (1,))
    cargs = (_ptr(W), _wdt(W), N, K, _ptr(tensor_scale_in), _ptr(vals), _ptr(meta), _ptr(scales), _ptr(ts),
             _ptr(codes), _ptr(bad), _stream(dev))
    return _run("nvfp4_sp24_produce", cargs, prepare, (W, tensor_scale_in), (vals, meta, scales, ts, bad, codes))


def sp24_prune(W, out=None, tensor_scale_out=None, prepare=False):
    """2:4 magnitude prune along K (keep the two largest |w| of every group of four). With
    tensor_scale_out (f32 [1]) it also receives s_t of W, which is s_t of the pruned tensor too."""
    N, K = W.shape
    _need(W, W.dtype, "W")
    out = out if out is not None else torch.empty_like(W)
    _need(out, W.dtype, "out", (N, K))
    if tensor_scale_out is not None:
        _need(tensor_scale_out, torch.float32, "tensor_scale_out", (1,))
    cargs = (_ptr(W), _wdt(W), N, K, _ptr(out), _ptr(tensor_scale_out), _stream(W.device))
    return _run("sp24_prune", cargs, prepare, (W, tensor_scale_out), out)


def sp24_check(codes, bad_groups=None, first_bad=None, prepare=False):
    """Per-group 2:4 check. Returns device int64 tensors (bad_groups [1], first_bad [1])."""
    N, Kh = codes.shape
    _need(codes, torch.uint8, "codes")
    dev = codes.device
    bad = bad_groups if bad_groups is not None else torch.empty(1, dtype=torch.int64, device=dev)
    first = first_bad if first_bad is not None else torch.empty(1, dtype=torch.int64, device=dev)
    cargs = (_ptr(codes), N, 2 * Kh, _ptr(bad), _ptr(first), _stream(dev))
    return _run("sp24_check", cargs, prepare, (codes,), (bad, first))


def sp24_compress(codes, vals=None, meta=None, bad_groups=None, raise_if_bad=False, prepare=False):
    """2:4 compression. Returns (vals u8 [N,K/4], meta u8 [N,K/8], bad_groups int64 [1] device)."""
    N, Kh = codes.shape
    K = 2 * Kh
    _need(codes, torch.uint8, "codes")
    dev = codes.device
    vals = vals if vals is not None else torch.empty((N, K // 4), dtype=torch.uint8, device=dev)
    meta = meta if meta is not None else torch.empty((N, K // 8), dtype=torch.uint8, device=dev)
    bad = bad_groups if bad_groups is not None else torch.empty(1, dtype=torch.int64, device=dev)
    _need(vals, torch.uint8, "vals", (N, K // 4)); _need(meta, torch.uint8, "meta", (N, K // 8))
    cargs = (_ptr(codes), N, K, _ptr(vals), _ptr(meta), _ptr(bad), _stream(dev))
    if prepare:
        return _run("sp24_compress", cargs, True, (codes,), (vals, meta, bad))
    _check(lib().sp24_compress(*cargs))
    if raise_if_bad:
        nb = int(bad.item())
        if nb:
            raise ValueError(f"sp24_compress: {nb} group(s) of four have fewer than two zeros")
    return vals, meta, bad


def sp24_decompress(vals, meta, codes=None):
    N, G = vals.shape
    K = 4 * G
    _need(vals, torch.uint8, "vals"); _need(meta, torch.uint8, "meta", (N, K // 8))
    codes = codes if codes is not None else torch.empty((N, K // 2), dtype=torch.uint8, device=vals.device)
    _need(codes, torch.uint8, "codes", (N, K // 2))
    _check(lib().sp24_decompress(_ptr(vals), _ptr(meta), N, K, _ptr(codes), _stream(vals.device)))
    return codes


def _gemm_out(X, N, y_dtype, Y):
    M = X.shape[0]
    Y = Y if Y is not None else torch.empty((M, N), dtype=y_dtype, device=X.device)
    dt = SSN_F32 if Y.dtype == torch.float32 else SSN_BF16 if Y.dtype == torch.bfloat16 else None
    if dt is None:
        raise TypeError("Y must be float32 or bfloat16")
    _need(Y, Y.dtype, "Y", (M, N))
    return Y, dt


def gemm_nvfp4_dense(X, codes, scales, tensor_scale, y_dtype=torch.float32, algo=ALGO_AUTO, Y=None, prepare=False):
    """Y = X . W_hat^T for dense NVFP4 weights. Returns (Y, algorithm that ran)."""
    M, K = X.shape
    N = codes.shape[0]
    _need(X, torch.bfloat16, "X"); _need(codes, torch.uint8, "codes", (N, K // 2))
    _need(scales, torch.uint8, "scales", (N, K // 16)); _need(tensor_scale, torch.float32, "tensor_scale", (1,))
    Y, dt = _gemm_out(X, N, y_dtype, Y)
    used = ctypes.c_int(-1)
    cargs = (_ptr(X), M, N, K, _ptr(codes), _ptr(scales), _ptr(tensor_scale), _ptr(Y), dt, algo,
             ctypes.byref(used), _stream(X.device))
    if prepare:
        return Prepared("gemm_nvfp4_dense", cargs, (X, codes, scales, tensor_scale, used, Y)), (Y, used)
    _check(lib().gemm_nvfp4_dense(*cargs))
    return Y, used.value


def gemm_nvfp4_sp24(X, vals, meta, scales, tensor_scale, y_dtype=torch.float32, algo=ALGO_AUTO, Y=None,
                    prepare=False):
    """Y = X . W_hat^T from 2:4-compressed NVFP4 weights. Returns (Y, algorithm that ran)."""
    M, K = X.shape
    N = vals.shape[0]
    _need(X, torch.bfloat16, "X"); _need(vals, torch.uint8, "vals", (N, K // 4))
    _need(meta, torch.uint8, "meta", (N, K // 8)); _need(scales, torch.uint8, "scales", (N, K // 16))
    _need(tensor_scale, torch.float32, "tensor_scale", (1,))
    Y, dt = _gemm_out(X, N, y_dtype, Y)
    used = ctypes.c_int(-1)
    cargs = (_ptr(X), M, N, K, _ptr(vals), _ptr(meta), _ptr(scales), _ptr(tensor_scale), _ptr(Y), dt, algo,
             ctypes.byref(used), _stream(X.device))
    if prepare:
        return Prepared("gemm_nvfp4_sp24", cargs, (X, vals, meta, scales, tensor_scale, used, Y)), (Y, used)
    _check(lib().gemm_nvfp4_sp24(*cargs))
    return Y, used.value


# ------------------------------------------------------------------------------------------------
# grouped-expert (MoE) path


def moe_route(topk_ids, E, prepare=False):
    """Routing bookkeeping for topk_ids int32 [T, k]. Returns device tensors
    (expert_offsets [E+1], row_token [T*k], row_slot [T*k], row_of [T*k], bad_ids [1])."""
    T, k = topk_ids.shape
    _need(topk_ids, torch.int32, "topk_ids")
    dev = topk_ids.device
    F = T * k
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    row_token = torch.empty(max(F, 1), dtype=torch.int32, device=dev)[:F]
    row_slot = torch.empty(max(F, 1), dtype=torch.int32, device=dev)[:F]
    row_of = torch.empty(max(F, 1), dtype=torch.int32, device=dev)[:F]
    bad = torch.empty(1, dtype=torch.int64, device=dev)
    nws = lib().moe_route_workspace_bytes(T, k, E)
    if nws < 0:
        _check(lib().moe_route(None, T, k, E, None, None, None, None, None, None, 0, None))
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)
    cargs = (_ptr(topk_ids), T, k, E, _ptr(offsets), _ptr(row_token), _ptr(row_slot), _ptr(row_of), _ptr(bad),
             _ptr(ws), nws, _stream(dev))
    return _run("moe_route", cargs, prepare, (topk_ids, ws), (offsets, row_token, row_slot, row_of, bad))


def moe_grouped_gemm_nvfp4(X, row_token, expert_offsets, R, w_main, w_scales, tensor_scales, w_meta=None,
                           epilogue=EPI_NONE, y_dtype=torch.float32, algo=ALGO_AUTO, Y=None, prepare=False,
                           w_layout=WLAYOUT_ROWS):
    """Every expert's product in one launch. X bf16 [x_rows, K]; row_token int32 [R] or None
    (identity); expert_offsets int32 [E+1]; dense weights w_main [E, N, K/2] (w_meta None) or
    2:4 w_main [E, N, K/4] with w_meta [E, N, K/8]; w_scales [E, N, K/16]; tensor_scales f32 [E].
    w_layout WLAYOUT_KTILE64 when the weight arrays come from moe_pack_weights.
    Returns (Y [R, N] or [R, N/2] for EPI_SILU_GATE, algorithm that ran)."""
    x_rows, K = X.shape
    E, N = w_main.shape[0], w_main.shape[1]
    sparse = w_meta is not None
    _need(X, torch.bfloat16, "X"); _need(expert_offsets, torch.int32, "expert_offsets", (E + 1,))
    if row_token is not None:
        _need(row_token, torch.int32, "row_token", (R,))
    _need(w_main, torch.uint8, "w_main", (E, N, K // 4 if sparse else K // 2))
    if sparse:
        _need(w_meta, torch.uint8, "w_meta", (E, N, K // 8))
    _need(w_scales, torch.uint8, "w_scales", (E, N, K // 16)); _need(tensor_scales, torch.float32, "tensor_scales", (E,))
    ncols = N // 2 if epilogue == EPI_SILU_GATE else N
    Y = Y if Y is not None else torch.empty((R, ncols), dtype=y_dtype, device=X.device)
    dt = SSN_F32 if Y.dtype == torch.float32 else SSN_BF16 if Y.dtype == torch.bfloat16 else None
    if dt is None:
        raise TypeError("Y must be float32 or bfloat16")
    _need(Y, Y.dtype, "Y", (R, ncols))
    used = ctypes.c_int(-1)
    cargs = (_ptr(X), x_rows, _ptr(row_token), _ptr(expert_offsets), E, R, N, K, int(sparse), int(w_layout),
             _ptr(w_main), _ptr(w_meta), _ptr(w_scales), _ptr(tensor_scales), epilogue, _ptr(Y), dt, algo,
             ctypes.byref(used), _stream(X.device))
    if prepare:
        return Prepared("moe_grouped_gemm_nvfp4", cargs, (X, row_token, expert_offsets, w_main, w_meta, w_scales,
                                                          tensor_scales, used, Y)), (Y, used)
    _check(lib().moe_grouped_gemm_nvfp4(*cargs))
    return Y, used.value


def moe_pack_ktiles(src, piece_bytes, out=None, prepare=False):
    """64-k tiled copy of one expert weight array [E, N, row_bytes] (uint8): out[e][kt][n] =
    src[e][n][kt*P:(kt+1)*P] with P = piece_bytes (codes 32, vals 16, meta 8, scales 4). The
    result keeps the shape [E, N, row_bytes]; only the byte order inside each expert changes."""
    _need(src, torch.uint8, "src")
    if src.dim() != 3:
        raise ValueError("src must be [E, N, row_bytes]")
    E, N, rb = src.shape
    out = out if out is not None else torch.empty_like(src)
    _need(out, torch.uint8, "out", (E, N, rb))
    cargs = (_ptr(src), E, N, rb, int(piece_bytes), _ptr(out), _stream(src.device))
    return _run("moe_pack_ktiles", cargs, prepare, (src,), out)


def moe_pack_weights(w):
    """(main, meta or None, scales, ts) in the row layout -> the same tuple in the 64-k tiled
    layout (WLAYOUT_KTILE64)."""
    main, meta, scales, ts = w
    sparse = meta is not None
    return (moe_pack_ktiles(main, 16 if sparse else 32), moe_pack_ktiles(meta, 8) if sparse else None,
            moe_pack_ktiles(scales, 4), ts)


def moe_combine(Yd, row_of, topk_weights, out=None, prepare=False):
    """out[t] = sum_j topk_weights[t, j] * Yd[row_of[t*k + j]] (f32 [T, D])."""
    R, D = Yd.shape
    T, k = topk_weights.shape
    dt = SSN_F32 if Yd.dtype == torch.float32 else SSN_BF16 if Yd.dtype == torch.bfloat16 else None
    if dt is None:
        raise TypeError("Yd must be float32 or bfloat16")
    _need(Yd, Yd.dtype, "Yd"); _need(row_of, torch.int32, "row_of", (T * k,))
    _need(topk_weights, torch.float32, "topk_weights")
    out = out if out is not None else torch.empty((T, D), dtype=torch.float32, device=Yd.device)
    _need(out, torch.float32, "out", (T, D))
    cargs = (_ptr(Yd), dt, R, _ptr(row_of), _ptr(topk_weights), T, k, D, _ptr(out), _stream(Yd.device))
    return _run("moe_combine", cargs, prepare, (Yd, row_of, topk_weights), out)


def moe_nvfp4_ffn(X, topk_ids, topk_weights, E, up, down, out=None, prepare=False, w_layout=WLAYOUT_ROWS):
    """The whole grouped-expert FFN. up = (main [E, 2I, D/2 or D/4], meta or None, scales
    [E, 2I, D/16], ts [E]); down = (main [E, D, I/2 or I/4], meta or None, scales [E, D, I/16],
    ts [E]); w_layout WLAYOUT_KTILE64 when both come from moe_pack_weights.
    Returns (out f32 [T, D], bad_ids int64 [1] device)."""
    T, D = X.shape
    _, k = topk_ids.shape
    I = up[2].shape[1] // 2
    sparse = up[1] is not None
    _need(X, torch.bfloat16, "X"); _need(topk_ids, torch.int32, "topk_ids", (T, k))
    _need(topk_weights, torch.float32, "topk_weights", (T, k))
    dev = X.device
    out = out if out is not None else torch.empty((T, D), dtype=torch.float32, device=dev)
    bad = torch.empty(1, dtype=torch.int64, device=dev)
    nws = lib().moe_ffn_workspace_bytes(T, k, E, I, D)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=dev)
    cargs = (_ptr(X), T, D, _ptr(topk_ids), _ptr(topk_weights), k, E, I, int(sparse), int(w_layout), _ptr(up[0]),
             _ptr(up[1]),
             _ptr(up[2]), _ptr(up[3]), _ptr(down[0]), _ptr(down[1]), _ptr(down[2]), _ptr(down[3]), _ptr(out),
             _ptr(bad), _ptr(ws), nws, _stream(dev))
    return _run("moe_nvfp4_ffn", cargs, prepare, (X, topk_ids, topk_weights, up, down, ws), (out, bad))



# ------------------------------------------------------------------------------------------------
# W4A4 variant (MXFP4 activations and weights)


def mxfp4_tiled_bytes(R, K):
    """(code bytes, scale bytes) of the MX_TILED layout of [R, K]."""
    sb = ctypes.c_int64(0)
    cb = lib().mxfp4_tiled_bytes(R, K, ctypes.byref(sb))
    if cb < 0:
        raise ValueError(f"invalid MXFP4 sizes R={R}, K={K}")
    return cb, sb.value


def mxfp4_quantize(V, layout=MX_TILED, codes=None, scales=None, prepare=False):
    """MXFP4 quantisation of V [R, K] (f32 or bf16). Returns (codes, scales) as uint8 tensors:
    [R, K/2] and [R, K/32] for MX_ROWS, flat arrays of mxfp4_tiled_bytes for MX_TILED."""
    R, K = V.shape
    _need(V, V.dtype, "V")
    dev = V.device
    if layout == MX_ROWS:
        cshape, sshape = (R, K // 2), (R, K // 32)
    else:
        cb, sb = mxfp4_tiled_bytes(R, K)
        cshape, sshape = (cb,), (sb,)
    codes = codes if codes is not None else torch.empty(cshape, dtype=torch.uint8, device=dev)
    scales = scales if scales is not None else torch.empty(sshape, dtype=torch.uint8, device=dev)
    _need(codes, torch.uint8, "codes", cshape); _need(scales, torch.uint8, "scales", sshape)
    cargs = (_ptr(V), _wdt(V), R, K, int(layout), _ptr(codes), _ptr(scales), _stream(dev))
    return _run("mxfp4_quantize", cargs, prepare, (V,), (codes, scales))


def gemm_mxfp4(x_codes, x_scales, M, w_codes, w_scales, N, K, y_dtype=torch.float32, algo=ALGO_AUTO, Y=None,
               prepare=False):
    """W4A4 product Y [M, N] = X_hat . W_hat^T from MX_TILED operands. Returns (Y, algorithm)."""
    for t, n, (R, ) in ((x_codes, "x_codes", (M,)), (w_codes, "w_codes", (N,))):
        _need(t, torch.uint8, n, (mxfp4_tiled_bytes(R, K)[0],))
    _need(x_scales, torch.uint8, "x_scales", (mxfp4_tiled_bytes(M, K)[1],))
    _need(w_scales, torch.uint8, "w_scales", (mxfp4_tiled_bytes(N, K)[1],))
    dev = x_codes.device
    Y = Y if Y is not None else torch.empty((M, N), dtype=y_dtype, device=dev)
    dt = SSN_F32 if Y.dtype == torch.float32 else SSN_BF16 if Y.dtype == torch.bfloat16 else None
    if dt is None:
        raise TypeError("Y must be float32 or bfloat16")
    _need(Y, Y.dtype, "Y", (M, N))
    used = ctypes.c_int(-1)
    cargs = (_ptr(x_codes), _ptr(x_scales), M, _ptr(w_codes), _ptr(w_scales), N, K, _ptr(Y), dt, algo,
             ctypes.byref(used), _stream(dev))
    if prepare:
        return Prepared("gemm_mxfp4", cargs, (x_codes, x_scales, w_codes, w_scales, used, Y)), (Y, used)
    _check(lib().gemm_mxfp4(*cargs))
    return Y, used.value

def moe_nvfp4_ffn_noalloc(X, topk_ids, topk_weights, E, up, down, out, bad_ids, w_layout=WLAYOUT_ROWS):
    """moe_nvfp4_ffn with the library's static per-GPU workspace instead of a caller-provided
    one: the call itself allocates nothing (out f32 [T, D] and bad_ids int64 [1] are the
    caller's). Routings needing more than the static workspace are refused."""
    T, D = X.shape
    _, k = topk_ids.shape
    I = up[2].shape[1] // 2
    sparse = up[1] is not None
    _need(X, torch.bfloat16, "X"); _need(topk_ids, torch.int32, "topk_ids", (T, k))
    _need(topk_weights, torch.float32, "topk_weights", (T, k))
    _need(out, torch.float32, "out", (T, D)); _need(bad_ids, torch.int64, "bad_ids", (1,))
    _check(lib().moe_nvfp4_ffn_noalloc(_ptr(X), T, D, _ptr(topk_ids), _ptr(topk_weights), k, E, I, int(sparse),
                                       int(w_layout), _ptr(up[0]), _ptr(up[1]), _ptr(up[2]), _ptr(up[3]),
                                       _ptr(down[0]), _ptr(down[1]), _ptr(down[2]), _ptr(down[3]), _ptr(out),
                                       _ptr(bad_ids), _stream(X.device)))
    return out, bad_ids


def mfma_probe_sink_floats():
    return int(lib().mfma_probe_sink_floats())


def mfma_probe(kind, waves_per_simd, iters, sink, seed=0, stream_device=None):
    """Calibration launch (see include/ssnvfp4.h): register-resident matrix ops on random
    operands. Returns the launch's floating-point operations; the caller times it."""
    fl = ctypes.c_double(0.0)
    _need(sink, torch.float32, "sink")
    if sink.numel() < mfma_probe_sink_floats():
        raise ValueError(f"sink needs {mfma_probe_sink_floats()} floats")
    _check(lib().mfma_probe(kind, waves_per_simd, iters, seed & 0xFFFFFFFF, _ptr(sink), ctypes.byref(fl),
                            _stream(sink.device)))
    return fl.value
