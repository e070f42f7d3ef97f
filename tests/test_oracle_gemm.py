"""Pins for the oracle's weight-quantised products: exact rational brute force, one-hot
extraction, a closed form, and 2:4 gather == dense product of the decompressed operand."""
from fractions import Fraction

import numpy as np
import torch

import synth
from oracle import formats, gemm, quant, sp24


def _decode_exact(codes, scales, st):
    """Independent exact decode: E2M1 by literal table, E4M3 by torch, tensor scale as Fraction."""
    e2 = [Fraction(v) for v in [0, 0.5, 1, 1.5, 2, 3, 4, 6]]
    e4 = torch.from_numpy(np.ascontiguousarray(scales)).view(torch.float8_e4m3fn).double().numpy()
    nib = np.empty((codes.shape[0], codes.shape[1] * 2), np.uint8)
    nib[:, 0::2], nib[:, 1::2] = codes & 15, codes >> 4
    N, K = nib.shape
    out = [[None] * K for _ in range(N)]
    for n in range(N):
        for k in range(K):
            c = int(nib[n, k])
            v = e2[c & 7] * Fraction(float(e4[n, k // 16])) * Fraction(float(st))
            out[n][k] = -v if c & 8 else v
    return out


def test_dense_matches_exact_rational_sum():
    M, N, K = 3, 5, 64
    rng = np.random.default_rng(0)
    xb = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    codes, scales, st = quant.quantize(w)
    Y, B = gemm.gemm_dense(xb, codes, scales, st)
    wx = _decode_exact(codes, scales, st)
    x = [[Fraction(float(v)) for v in row] for row in formats.bf16_decode(xb)]
    for m in range(M):
        for n in range(N):
            exact = sum(x[m][k] * wx[n][k] for k in range(K))
            mag = sum(abs(x[m][k] * wx[n][k]) for k in range(K))
            assert abs(Fraction(Y[m, n]) - exact) <= mag * Fraction(K, 2 ** 52)
            assert abs(Fraction(B[m, n]) - mag) <= mag * Fraction(K, 2 ** 52)


def test_one_hot_rows_extract_weights():
    N, K = 7, 48
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    codes, scales, st = quant.quantize(w)
    xb = synth.f32_to_bf16_bits(np.eye(K, dtype=np.float32))
    Y, _ = gemm.gemm_dense(xb, codes, scales, st)
    assert np.array_equal(Y.T, quant.dequantize(codes, scales, st))
    # non-square, non-symmetric: a transposed operand would not even have the right shape
    assert Y.shape == (K, N)


def test_constant_closed_form():
    M, N, K = 2, 3, 64
    codes = np.full((N, K // 2), 0x55, np.uint8)       # every code 5 (value 3.0)
    scales = np.full((N, K // 16), 0x40, np.uint8)     # E4M3 0x40 = 2.0
    st = np.float32(0.125)
    xb = synth.f32_to_bf16_bits(np.ones((M, K), np.float32))
    Y, B = gemm.gemm_dense(xb, codes, scales, st)
    assert np.all(Y == K * 3.0 * 2.0 * 0.125) and np.all(B == Y)
    neg = np.full((N, K // 2), 0xDD, np.uint8)        # code 0xD = -3.0
    Yn, Bn = gemm.gemm_dense(xb, neg, scales, st)
    assert np.all(Yn == -Y) and np.all(Bn == B)


def test_sp24_gather_equals_dense_of_decompressed():
    M, N, K = 9, 33, 256
    xb = synth.activations(M, K, seed=3)
    w = sp24.prune24(synth.weights(N, K, seed=3))
    codes, scales, st = quant.quantize(w)
    vals, meta, bad = sp24.compress(codes)
    assert bad == 0
    Ys, Bs = gemm.gemm_sp24(xb, vals, meta, scales, st)
    Yd, Bd = gemm.gemm_dense(xb, sp24.decompress(vals, meta), scales, st)
    Yc, _ = gemm.gemm_dense(xb, codes, scales, st)
    tol = 1e-12 * Bd + 1e-300
    assert np.all(np.abs(Ys - Yd) <= tol) and np.all(np.abs(Bs - Bd) <= tol)
    assert np.all(np.abs(Yc - Yd) <= tol)          # pruned zeros contribute nothing
    # rows subset
    Yr, _ = gemm.gemm_sp24(xb, vals, meta, scales, st, rows=np.array([3, 17]))
    assert np.all(np.abs(Yr - Ys[:, [3, 17]]) <= tol[:, [3, 17]])


def test_sp24_gather_uses_positions():
    # one row, one group kept at positions (1, 3): only x[1] and x[3] contribute
    vals = np.array([[0x42] + [0] * 7], np.uint8)        # codes 2 (1.0) at i0, 4 (2.0) at i1
    meta = np.array([[0x0D] + [0x44] * 3], np.uint8)     # group 0: i0=1, i1=3; others (0,1)
    scales = np.array([[0x38, 0x38]], np.uint8)          # E4M3 0x38 = 1.0
    x = np.zeros((1, 32), np.float32)
    x[0, :4] = [100.0, 3.0, 100.0, 5.0]
    Y, _ = gemm.gemm_sp24(synth.f32_to_bf16_bits(x), vals, meta, scales, np.float32(1.0))
    assert Y[0, 0] == 3.0 * 1.0 + 5.0 * 2.0


def test_bound_bf16_output_adds_half_ulp():
    B = np.array([[0.0, 1.0]])
    Y = np.array([[1.0, 1.0]])
    b = gemm.bound(B, Y, out="bf16")
    assert b[0, 0] == 0.5 * 2.0 ** -7
    assert b[0, 1] == 2e-3 + 0.5 * 2.0 ** -7
