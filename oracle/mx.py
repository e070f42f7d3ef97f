"""MXFP4 quantisation and the W4A4 product (oracle): activations quantised as well as weights.

The pages call block-scaled FP4 x FP4 ("NVFP4 W4A4") the performance unlock of FP4 tensor
cores ("Trying to beat the bandwidth", NVIDIA developer forum thread: W4A16 has to dequantise to
BF16 first, W4A4 does not) and note that a W4A4 checkpoint also carries calibrated activation
scales ("NVFP4 Without FP4 Hardware", ai-muninn.com, section "Convert BF16 to NVFP4
yourself"). They define no activation format beyond that. The matrix cores of this build take
FP4 operands with one power-of-two scale per 32 values along K for each operand (OCP
Microscaling, "MX"), not an E4M3 scale per 16, and an E4M3 scale's 3-bit mantissa cannot be
folded into a 4-bit element without rounding. The reading taken here is therefore the OCP MXFP4
format for both operands of the W4A4 variant:

* element: E2M1 nibble (as for NVFP4: magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6; bit 3 = sign);
* scale: one E8M0 byte per 32 consecutive values along K, value 2^(b - 127) (0xFF, NaN, is
  never produced);
* quantisation of a block (the OCP reference rule): e = floor(log2(amax)) - 2, clamped to
  [-127, 127] (2 = exponent of the largest E2M1 magnitude, 6 = 1.5 * 2^2; a block of zeros
  takes e = -127); X = 2^e; code = sign(v) | E2M1 nearest (ties to the even code, saturating at
  6) of |v| / X. With this rule amax / X lies in [4, 8), so values above 6 X saturate to 6 X;
* packing: element k = 2j in the low nibble of byte j, as for the NVFP4 codes; scales
  [R, K/32] row-major.

Every division is by a power of two, so |v| / X is exact and every rounding decision is taken
on the exact value. The product Y = X_hat . W_hat^T has exact terms (2 + 2 significant bits
times a power of two) and is summed in float64 here; the GPU sums in f32, bound by 2e-3 * sum
|x_hat w_hat| as for the other products. How far W4A4 may move a result from the W4A16 product
on the same weights is ``activation_error``: sum_k |x_k - x_hat_k| |w_hat_k| per output.

Pinned by the tests in tests/test_oracle_mx.py (exact rational brute force of the rule, worked
blocks, re-quantisation identity, the E8M0 decode against torch's float8_e8m0fnu, products by
exact sums, one-hot rows and a closed form).
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_decode, e2m1_decode, e2m1_round_magnitude
from .quant import pack_nibbles, unpack_nibbles

MX_BLOCK = 32
E2M1_EMAX = 2          # exponent of the largest E2M1 magnitude (6 = 1.5 * 2^2)
E8M0_BIAS = 127


def e8m0_decode(b: np.ndarray) -> np.ndarray:
    """E8M0 scale byte -> 2^(b - 127) (float64; 0xFF would be NaN)."""
    b = np.asarray(b).astype(np.int64)
    return np.where(b == 0xFF, np.nan, np.ldexp(1.0, b - E8M0_BIAS))


def scale_exponent(amax: np.ndarray) -> np.ndarray:
    """floor(log2(amax)) - 2 clamped to [-127, 127]; -127 for amax == 0."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))      # amax = f * 2^ex, f in [0.5, 1)
    e = np.where(amax > 0, ex - 1 - E2M1_EMAX, -E8M0_BIAS)
    return np.clip(e, -E8M0_BIAS, E8M0_BIAS).astype(np.int64)


def quantize(v: np.ndarray):
    """MXFP4 quantisation of float32 (or float64 holding float32/bf16 values) [R, K], K % 32 == 0.

    Returns (codes uint8 [R, K/2], scales uint8 [R, K/32])."""
    v = np.asarray(v, dtype=np.float64)
    R, K = v.shape
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = v.reshape(R, K // MX_BLOCK, MX_BLOCK)
    mag = np.abs(blocks)
    e = scale_exponent(mag.max(axis=2))
    r = mag / np.ldexp(1.0, e)[:, :, None]               # exact: division by a power of two
    code = e2m1_round_magnitude(r).astype(np.uint8) | (np.signbit(blocks).astype(np.uint8) << 3)
    return pack_nibbles(code.reshape(R, K)), (e + E8M0_BIAS).astype(np.uint8)


def quantize_bf16(x_bits: np.ndarray):
    """MXFP4 quantisation of bf16 activations given as bit patterns [M, K]."""
    return quantize(bf16_decode(x_bits))


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decoded values E2M1(code) * 2^(scale - 127), float64 [R, K] (exact)."""
    nib = unpack_nibbles(codes)
    return e2m1_decode(nib) * np.repeat(e8m0_decode(scales), MX_BLOCK, axis=1)


def gemm_w4a4(xc: np.ndarray, xs: np.ndarray, wc: np.ndarray, ws: np.ndarray, rows=None):
    """Y = X_hat . W_hat^T and the bound base B = |X_hat| . |W_hat|^T (float64 [M, N]) for MXFP4
    activations (xc, xs) and weights (wc, ws); ``rows`` restricts to a subset of weight rows."""
    if rows is not None:
        wc, ws = wc[rows], ws[rows]
    x = dequantize(xc, xs)
    w = dequantize(wc, ws)
    return x @ w.T, np.abs(x) @ np.abs(w).T


def activation_error(x: np.ndarray, xc: np.ndarray, xs: np.ndarray, wc: np.ndarray, ws: np.ndarray) -> np.ndarray:
    """sum_k |x_k - x_hat_k| |w_hat_k| per output [M, N]: the most the activations' quantisation
    can move a product from the one on unquantised activations (same weights)."""
    dx = np.abs(np.asarray(x, dtype=np.float64) - dequantize(xc, xs))
    return dx @ np.abs(dequantize(wc, ws)).T
