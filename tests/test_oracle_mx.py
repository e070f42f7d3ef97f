"""Pins for the oracle's MXFP4 quantisation and W4A4 product: the E8M0 decode against torch's
float8_e8m0fnu, worked blocks computed by hand, an exact rational implementation of the block
rule on random blocks, the re-quantisation identity, the element error bound, and products by
exact rational sums, one-hot rows and a closed form."""
from fractions import Fraction

import numpy as np
import torch

import synth
from oracle import formats, mx

GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def test_e8m0_decode_matches_torch():
    b = np.arange(255, dtype=np.uint8)
    want = torch.from_numpy(b).view(torch.float8_e8m0fnu).double().numpy()
    assert np.array_equal(mx.e8m0_decode(b), want)
    assert np.isnan(mx.e8m0_decode(np.array([255]))[0])


def _block(vals):
    v = np.zeros((1, 32), np.float32)
    v[0, :len(vals)] = vals
    return v


def _nibbles(codes):
    n = np.empty(codes.shape[1] * 2, np.uint8)
    n[0::2], n[1::2] = codes[0] & 15, codes[0] >> 4
    return n


def test_worked_blocks():
    # amax 4: floor(log2 4) - 2 = 0, X = 1: 1 -> code 2, 2 -> 4, 3 -> 5, 4 -> 6
    c, s = mx.quantize(_block([1, 0, 2, 0, 3, 0, 4, 0]))
    assert s[0, 0] == 127 and list(_nibbles(c)[:8]) == [2, 0, 4, 0, 5, 0, 6, 0]
    # amax 6 keeps X = 1 (6 -> code 7); amax 7 too, and 7 saturates to 6
    c, s = mx.quantize(_block([6, -7, 0.25, -0.25]))
    assert s[0, 0] == 127 and list(_nibbles(c)[:4]) == [7, 15, 0, 8]     # 0.25 ties to 0; -0.25 -> -0
    # amax 8: X = 2; 8 -> 4 (code 6), 3 -> 1.5 (code 3), 5 -> 2.5 ties to 2 (code 4), 7 -> 3.5 ties to 4 (code 6)
    c, s = mx.quantize(_block([8, 3, 5, 7]))
    assert s[0, 0] == 128 and list(_nibbles(c)[:4]) == [6, 3, 4, 6]
    # all zeros: the smallest scale, codes 0
    c, s = mx.quantize(np.zeros((2, 64), np.float32))
    assert np.all(s == 0) and np.all(c == 0)


def _floor_log2(q: Fraction) -> int:
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    return e


def _rne_grid(r: Fraction) -> int:
    if r >= 6:
        return 7
    for i in range(7):
        lo, hi = GRID[i], GRID[i + 1]
        if r <= hi:
            mid = (lo + hi) / 2
            if r < mid:
                return i
            if r > mid:
                return i + 1
            return i if i % 2 == 0 else i + 1
    return 7


def test_rule_matches_exact_rational_implementation():
    rng = np.random.default_rng(0)
    for trial in range(60):
        v = (rng.standard_normal((3, 64)) * np.exp(rng.uniform(-20, 20))).astype(np.float32)
        if trial % 5 == 0:                       # values on grid midpoints of a power-of-two scale
            v = (rng.integers(-12, 13, (3, 64)) * 0.25 * 2.0 ** rng.integers(-10, 10)).astype(np.float32)
        c, s = mx.quantize(v)
        nib = np.stack([_nibbles(c[i:i + 1]) for i in range(3)])
        for r in range(3):
            for b in range(2):
                blk = [Fraction(float(t)) for t in v[r, 32 * b:32 * b + 32]]
                amax = max(abs(t) for t in blk)
                e = -127 if amax == 0 else max(-127, min(127, _floor_log2(amax) - 2))
                assert s[r, b] == e + 127
                X = Fraction(2) ** e
                for k, t in enumerate(blk):
                    want = _rne_grid(abs(t) / X) | (8 if np.signbit(v[r, 32 * b + k]) else 0)
                    assert nib[r, 32 * b + k] == want


def test_requantising_the_decode_is_the_identity():
    # a quantised block's largest code is 4 or 6 (amax / X lies in [4, 8)), so decoding and
    # quantising again gives the same scale and codes
    rng = np.random.default_rng(1)
    v = (rng.standard_normal((20, 256)) * np.exp(rng.uniform(-5, 5, (20, 1)))).astype(np.float32)
    c, s = mx.quantize(v)
    c2, s2 = mx.quantize(mx.dequantize(c, s).astype(np.float32))
    assert np.array_equal(s, s2)
    # -0 decodes to -0.0 and requantises to 0x8 (np.signbit); +0 stays 0
    assert np.array_equal(c, c2)


def test_element_error_is_within_two_scales_and_half_a_step_below_six():
    rng = np.random.default_rng(2)
    v = (rng.standard_normal((64, 128)) * 3).astype(np.float32)
    c, s = mx.quantize(v)
    X = np.repeat(mx.e8m0_decode(s), 32, axis=1)
    err = np.abs(v - mx.dequantize(c, s))
    assert np.all(err <= 2 * X)
    below = np.abs(v) <= 6 * X
    assert np.all(err[below] <= X[below])            # half the widest step (2X between 4X and 6X)
    assert np.any(err > X)                           # saturation between 6X and 8X does happen


def test_w4a4_product_is_the_exact_rational_sum():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 64)).astype(np.float32)
    w = (rng.standard_normal((4, 64)) * 0.02).astype(np.float32)
    xc, xs = mx.quantize(x)
    wc, ws = mx.quantize(w)
    Y, B = mx.gemm_w4a4(xc, xs, wc, ws)
    xn, wn = np.stack([_nibbles(xc[i:i + 1]) for i in range(3)]), np.stack([_nibbles(wc[i:i + 1]) for i in range(4)])
    val = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]

    def dec(n, sc):
        t = val[n & 7] * Fraction(2) ** (int(sc) - 127)
        return -t if n & 8 else t
    for m in range(3):
        for n in range(4):
            exact = sum(dec(xn[m, k], xs[m, k // 32]) * dec(wn[n, k], ws[n, k // 32]) for k in range(64))
            mag = sum(abs(dec(xn[m, k], xs[m, k // 32]) * dec(wn[n, k], ws[n, k // 32])) for k in range(64))
            assert Y[m, n] == float(exact) and B[m, n] == float(mag)


def test_w4a4_one_hot_and_closed_form():
    K = 128
    w = (np.random.default_rng(4).standard_normal((5, K)) * 0.02).astype(np.float32)
    wc, ws = mx.quantize(w)
    eye = np.eye(K, dtype=np.float32)[[0, 31, 32, 100]]
    xc, xs = mx.quantize(eye)
    Y, _ = mx.gemm_w4a4(xc, xs, wc, ws)
    assert np.array_equal(Y, mx.dequantize(wc, ws)[:, [0, 31, 32, 100]].T)   # unit rows: 1 = 4 * 2^-2 exactly
    # constant operands decode exactly: 1.5 = 6 * 2^-2 and -0.75 = -6 * 2^-3, so Y = -K * 1.125
    ones = np.full((2, K), 1.5, np.float32)
    xc, xs = mx.quantize(ones)
    wc, ws = mx.quantize(np.full((3, K), -0.75, np.float32))
    Y, B = mx.gemm_w4a4(xc, xs, wc, ws)
    assert np.all(Y == -K * 1.5 * 0.75) and np.all(B == K * 1.5 * 0.75)


def test_activation_error_bounds_the_distance_to_the_w4a16_product():
    rng = np.random.default_rng(5)
    x_bits = synth.activations(6, 256, seed=7)
    x = formats.bf16_decode(x_bits)
    w = (rng.standard_normal((9, 256)) * 0.02).astype(np.float32)
    xc, xs = mx.quantize_bf16(x_bits)
    wc, ws = mx.quantize(w)
    Y4, _ = mx.gemm_w4a4(xc, xs, wc, ws)
    Y16 = x @ mx.dequantize(wc, ws).T
    D = mx.activation_error(x, xc, xs, wc, ws)
    assert np.all(np.abs(Y4 - Y16) <= D * (1 + 1e-12)) and np.all(D > 0)
    assert np.max(np.abs(Y4 - Y16) / D) > 0.05       # not vacuous
