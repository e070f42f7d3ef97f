"""Pins for the oracle's NVFP4 quantiser: a worked example, exact rational brute force, the
re-quantisation invariant, the shared-scale property and the pages' byte counts."""
import json
import os
from fractions import Fraction

import numpy as np
import torch

from oracle import accounting, formats, quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_example_bytes():
    # amax = 4 -> s_t = 4/2688; block scale = 4 / (6 s_t) = 448 exactly -> byte 0x7E.
    # r = |w| / (s_t * 448) = 1.5 |w|: 1 -> 1.5 (code 3), 2 -> 3 (code 5), 3 -> 4.5 (nearest 4,
    # code 6), 4 -> 6 (code 7). Packed with the even element in the low nibble.
    w = np.array([[1, 0, 2, 0, 3, 0, 4, 0] + [0] * 8], dtype=np.float32)
    codes, scales, st = quant.quantize(w)
    assert st == np.float32(4.0 / 2688.0)
    assert scales.tolist() == [[0x7E]]
    assert codes.tolist() == [[0x03, 0x05, 0x06, 0x07, 0, 0, 0, 0]]
    # negative values keep their sign bit, and a tiny negative keeps the FP4 negative zero
    w2 = np.array([[-1, 0, 2, -1e-9, 3, 0, -4, 0] + [0] * 8], dtype=np.float32)
    c2, s2, _ = quant.quantize(w2)
    assert c2.tolist() == [[0x0B, 0x85, 0x06, 0x0F, 0, 0, 0, 0]]


def test_zero_tensor():
    codes, scales, st = quant.quantize(np.zeros((2, 32), np.float32))
    assert st == 0 and not codes.any() and not scales.any()


def _f32_nearest(q: Fraction) -> np.float32:
    """Correctly rounded float32 of an exact rational (brute force over neighbours)."""
    c = np.float32(float(q))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    best = min(cands, key=lambda v: (abs(Fraction(float(v)) - q),
                                     int(np.array(v, np.float32).view(np.uint32)) & 1))
    return np.float32(best)


def _nearest(q: Fraction, grid):
    best = None
    for i, g in enumerate(grid):
        d = abs(q - g)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


def _quantize_exact(w: np.ndarray, st=None):
    """Independent exact-rational quantiser (Fractions, brute-force nearest)."""
    e2 = [Fraction(v) for v in [0, 0.5, 1, 1.5, 2, 3, 4, 6]]
    e4 = [Fraction(float(v)) for v in torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).double()]
    N, K = w.shape
    if st is None:
        st = _f32_nearest(max(abs(Fraction(float(v))) for v in w.ravel()) / 2688)
    S = np.zeros((N, K // 16), np.uint8)
    code = np.zeros((N, K), np.uint8)
    stf = Fraction(float(st))
    for n in range(N):
        for b in range(K // 16):
            blk = [Fraction(float(v)) for v in w[n, 16 * b:16 * b + 16]]
            if stf == 0:
                continue
            q = min(max(abs(v) for v in blk) / (6 * stf), Fraction(448))
            S[n, b] = _nearest(q, e4)
            d = stf * e4[S[n, b]]
            if d == 0:
                continue
            for i, v in enumerate(blk):
                c = _nearest(min(abs(v) / d, Fraction(6)), e2)
                if np.signbit(w[n, 16 * b + i]):
                    c |= 8
                code[n, 16 * b + i] = c
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, S, st


def test_quantize_matches_exact_rational_brute_force():
    rng = np.random.default_rng(5)
    for trial in range(6):
        w = (rng.standard_normal((3, 32)) * 0.02).astype(np.float32)
        if trial % 2:
            w[:, ::5] = 0.0                      # exact zeros and -0.0
            w[0, 1] = -0.0
        c, s, st = quant.quantize(w)
        ce, se, ste = _quantize_exact(w)
        assert st == ste
        assert np.array_equal(s, se)
        assert np.array_equal(c, ce)


def test_quantize_exact_on_ties():
    # Values placed exactly on E2M1 midpoints relative to the block scale: with amax = 6 * 448 * s
    # the block scale is 448 and r = |w| / (448 s); choose s = 1/2688 so that 6*448*s = 1.
    st = np.float32(1.0 / 2688.0)
    unit = np.float64(st) * 448.0
    r = np.array([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.2, 0.3, 2.9, 3.1, 4.9, 5.1, 1.0, 0.5])
    w = (r * unit).astype(np.float32)[None, :]
    c, s, _ = quant.quantize(w, tensor_scale_in=st)
    ce, se, _ = _quantize_exact(w, st)
    assert np.array_equal(c, ce) and np.array_equal(s, se)


def test_tensor_scale_is_correctly_rounded():
    rng = np.random.default_rng(9)
    for v in rng.standard_normal(300).astype(np.float32):
        a = abs(Fraction(float(v)))
        assert quant.tensor_scale(np.array([v])) == _f32_nearest(a / 2688)


def test_requantize_from_bf16_decode_is_bit_exact():
    # Decode to bf16 keeping the FP4 negative zero, quantise again with the same global scale:
    # codes and block scales come back identical (blocks whose scale is a normal E4M3 value).
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((20, 128)) * 0.02).astype(np.float32)
    w[rng.random(w.shape) < 0.05] = -1e-12      # tiny negatives -> code 0x8
    c, s, st = quant.quantize(w)
    assert (s >= 0x08).all()
    wd = formats.bf16_round(quant.dequantize(c, s, st)).astype(np.float32)
    c2, s2, _ = quant.quantize(wd, tensor_scale_in=st)
    assert np.array_equal(s, s2) and np.array_equal(c, c2)


def test_shared_global_scale():
    # A group of tensors sharing one scale from the group's amax equals quantising the stacked group.
    rng = np.random.default_rng(2)
    a = (rng.standard_normal((4, 64)) * 0.02).astype(np.float32)
    b = (rng.standard_normal((4, 64)) * 0.001).astype(np.float32)
    cg, sg, stg = quant.quantize(np.concatenate([a, b]))
    ca, sa, _ = quant.quantize(a, tensor_scale_in=stg)
    cb, sb, _ = quant.quantize(b, tensor_scale_in=stg)
    assert np.array_equal(cg, np.concatenate([ca, cb])) and np.array_equal(sg, np.concatenate([sa, sb]))
    # with its own (smaller) scale, the small tensor quantises differently
    cb_own, _, stb = quant.quantize(b)
    assert stb < stg and not np.array_equal(cb_own, cb)


def test_byte_counts_match_pages_table():
    with open(os.path.join(GOLDEN, "bitexact_bytes.json")) as f:
        g = json.load(f)
    for t in g["tensors"]:
        numel = t["packed"] * 2
        b = accounting.dense_bytes(numel // 5120, 5120) if numel % 5120 == 0 else accounting.dense_bytes(numel, 1)
        assert b["codes"] == t["packed"]
        assert b["scales"] == t["block_scales"]
        assert b["tensor_scale"] == t["global_scale"]
    # and the quantiser emits exactly these sizes
    c, s, st = quant.quantize(np.ones((8, 96), np.float32))
    assert c.nbytes == 8 * 96 // 2 and s.nbytes == 8 * 96 // 16 and np.float32(st).nbytes == 4
