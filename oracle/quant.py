"""NVFP4 quantisation and decode (oracle).

Follows "NVFP4 Without FP4 Hardware" (ai-muninn.com), section "Convert BF16 to NVFP4
yourself": every weight becomes a 4-bit E2M1 value, every 16 consecutive values along a row
(the reduction axis K) share one FP8 E4M3 block scale, and the tensor carries one FP32 global
scale; no calibration data is involved. Section "The shared global scale" adds that a group
of tensors may share one global scale taken from the group's largest magnitude, which is the
``tensor_scale_in`` argument here. The numeric recipe (the pages print no code) is the plain
reading that the ranges of the two formats fix:

1. s_t = amax / (6 * 448), rounded to float32 (6 = largest E2M1, 448 = largest E4M3).
2. Block scale S_b = E4M3 nearest (ties to even) of min(amax_b / (6 * s_t), 448), where
   amax_b is the largest |w| of the 16-value block.
3. Code = E2M1 nearest (ties to even, saturating at 6) of |w| / (s_t * S_b), with the sign
   bit of w (so a negative value that rounds to zero keeps the FP4 negative zero, as in the
   section "Bit-exact check against lyf's ModelOpt output"). A block with S_b = 0 stores
   code 0 for all its values.
4. Decoded weight: w_hat = E2M1(code) * E4M3(S_b) * s_t.

Exactness: every rounding decision is taken on a float64 quotient. w has 24 significant bits
and s_t * S_b at most 28, so a quotient that is not exactly a midpoint of the 4-bit (E4M3) or
3-bit (E2M1) grid lies further than half a float64 ulp from every midpoint; rounding the
float64 quotient therefore decides exactly as rounding the exact quotient would. The same holds
for s_t: 2688 = 2^7 * 21, so amax / 2688 is never a float32 midpoint, and float64 division
then conversion to float32 equals the correctly rounded float32 quotient. The tests pin this
against exact rational arithmetic.

Packing: element k = 2j sits in the low nibble of byte j of its row, k = 2j + 1 in the high
nibble (the pages give the sizes, numel/2 code bytes and numel/16 scale bytes, not the order).
"""
from __future__ import annotations

import numpy as np

from .formats import e2m1_decode, e2m1_round_magnitude, e4m3_decode, e4m3_round

BLOCK = 16
TENSOR_SCALE_DIV = 6.0 * 448.0  # 2688


def tensor_scale(w: np.ndarray) -> np.float32:
    """s_t = fl32(amax / 2688) over all elements of w (float32 input)."""
    amax = float(np.max(np.abs(np.asarray(w, dtype=np.float64)))) if np.size(w) else 0.0
    return np.float32(amax / TENSOR_SCALE_DIV)


def pack_nibbles(nib: np.ndarray) -> np.ndarray:
    """[N, K] nibbles -> [N, K/2] bytes, even k in the low nibble."""
    nib = np.asarray(nib, dtype=np.uint8)
    return (nib[:, 0::2] & 0xF) | ((nib[:, 1::2] & 0xF) << 4)


def unpack_nibbles(b: np.ndarray) -> np.ndarray:
    """[N, K/2] bytes -> [N, K] nibbles (uint8)."""
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty((b.shape[0], b.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = b & 0xF
    out[:, 1::2] = b >> 4
    return out


def quantize(w: np.ndarray, tensor_scale_in=None):
    """Quantise float32 W [N, K] (K % 16 == 0) to NVFP4.

    Returns (codes uint8 [N, K/2], scales uint8 [N, K/16], s_t float32). With
    ``tensor_scale_in`` the given global scale is used instead of this tensor's own (a
    scale shared by a group of tensors).
    """
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 16")
    s_t = tensor_scale(w) if tensor_scale_in is None else np.float32(tensor_scale_in)
    st = np.float64(s_t)
    blocks = w.astype(np.float64).reshape(N, K // BLOCK, BLOCK)
    mag = np.abs(blocks)
    amax_b = mag.max(axis=2)
    if st > 0:
        q = amax_b / (6.0 * st)
        S = e4m3_round(q).astype(np.uint8)          # min(q, 448) is applied inside
    else:
        S = np.zeros_like(amax_b, dtype=np.uint8)
    denom = st * e4m3_decode(S)                     # exact product
    valid = denom > 0
    r = np.where(valid[:, :, None], mag / np.where(valid, denom, 1.0)[:, :, None], 0.0)
    mcode = e2m1_round_magnitude(r).astype(np.uint8)
    sign = np.signbit(blocks).astype(np.uint8) << 3
    code = np.where(valid[:, :, None], mcode | sign, 0).astype(np.uint8)
    return pack_nibbles(code.reshape(N, K)), S, s_t


def dequantize(codes: np.ndarray, scales: np.ndarray, s_t) -> np.ndarray:
    """Decoded weights w_hat = E2M1(code) * E4M3(S) * s_t, float64 [N, K] (exact)."""
    nib = unpack_nibbles(codes)
    N, K = nib.shape
    sc = np.repeat(e4m3_decode(scales), BLOCK, axis=1)
    return e2m1_decode(nib) * sc * np.float64(np.float32(s_t))

