"""Weight-quantised products Y = X . W_hat^T in float64 (oracle), and the parity bound.

X is row-major [M, K] bf16, W is row-major [N, K] with K the reduction axis, Y is [M, N].
Dense form: W_hat[n, k] = E2M1(code[n, k]) * E4M3(S[n, k // 16]) * s_t ("NVFP4 Without FP4
Hardware", ai-muninn.com, section "Convert BF16 to NVFP4 yourself"). 2:4 form: only the two
kept values of every group of four contribute, at their stored positions ("NVFP4 vs 2:4
sparse", robertz.co, section "What 2:4 actually is": the pruned lanes are skipped, which halves
the multiplies).

Every product x * w_hat is exact in float64 (8 + 6 + 24 significant bits), so the dense
oracle is the plain definition evaluated with a float64 matrix product; its own rounding is
about K * 2^-53 relative to sum |x * w_hat|, far below any tolerance used. The 2:4 oracle sums
the kept terms directly from (vals, meta) by gathering x at the stored positions — it does
not go through decompression, so comparing the two is a real check.

Parity bound for a GPU result computed with float32 accumulation: per output element,
|Y_gpu - Y| <= 2e-3 * sum_k |x_k * w_hat_k|; for a bf16 output, half a bf16 ulp of the
result is added (the unavoidable output rounding).
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_decode, bf16_ulp, e2m1_decode, e4m3_decode
from .quant import BLOCK, dequantize
from .sp24 import positions

REL_TOL = 2e-3


def gemm_dense(x_bits: np.ndarray, codes: np.ndarray, scales: np.ndarray, s_t, rows=None):
    """Y = X . W_hat^T and the bound base B = |X| . |W_hat|^T, both float64 [M, N].

    ``rows`` optionally restricts to a subset of W rows (output columns)."""
    if rows is not None:
        codes, scales = codes[rows], scales[rows]
    x = bf16_decode(x_bits)
    w = dequantize(codes, scales, s_t)
    return x @ w.T, np.abs(x) @ np.abs(w).T


def sp24_kept_terms(vals: np.ndarray, meta: np.ndarray, scales: np.ndarray, s_t):
    """Positions k [N, K/2] and decoded kept weights [N, K/2] (two per group, in order)."""
    vals = np.asarray(vals, dtype=np.uint8)
    N, G = vals.shape
    i0, i1 = positions(meta)
    g = np.arange(G)[None, :]
    k0, k1 = 4 * g + i0, 4 * g + i1
    st = np.float64(np.float32(s_t))
    sc = e4m3_decode(scales)
    n = np.arange(N)[:, None]
    w0 = e2m1_decode(vals & 0xF) * sc[n, k0 // BLOCK] * st
    w1 = e2m1_decode(vals >> 4) * sc[n, k1 // BLOCK] * st
    k = np.stack([k0, k1], axis=2).reshape(N, 2 * G)
    w = np.stack([w0, w1], axis=2).reshape(N, 2 * G)
    return k, w


def gemm_sp24(x_bits: np.ndarray, vals: np.ndarray, meta: np.ndarray, scales: np.ndarray, s_t,
              rows=None, chunk: int = 64):
    """2:4 product from the compressed operand: Y[m, n] = sum over kept (k, w) of x[m, k] * w."""
    if rows is not None:
        vals, meta, scales = vals[rows], meta[rows], scales[rows]
    x = bf16_decode(x_bits)
    k, w = sp24_kept_terms(vals, meta, scales, s_t)
    N = k.shape[0]
    Y = np.empty((x.shape[0], N))
    B = np.empty((x.shape[0], N))
    for n0 in range(0, N, chunk):
        xs = x[:, k[n0:n0 + chunk]]                     # [M, n, K/2] gathered activations
        Y[:, n0:n0 + chunk] = np.einsum("mnj,nj->mn", xs, w[n0:n0 + chunk])
        B[:, n0:n0 + chunk] = np.einsum("mnj,nj->mn", np.abs(xs), np.abs(w[n0:n0 + chunk]))
    return Y, B


def bound(B: np.ndarray, Y: np.ndarray, out: str = "f32") -> np.ndarray:
    """Allowed |Y_gpu - Y| per element."""
    tol = REL_TOL * B
    if out == "bf16":
        tol = tol + 0.5 * bf16_ulp(np.abs(Y) + tol)
    return tol
