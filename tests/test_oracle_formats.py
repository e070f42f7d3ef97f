"""Pins for the oracle's number formats (E2M1, E4M3, bf16) against library routines and
exhaustive exact arithmetic."""
from fractions import Fraction

import numpy as np
import torch

from oracle import formats as F


def test_e2m1_table_matches_e4m3_reencoding_via_torch():
    # An E2M1 code (s, e, m) with e >= 1 is the value 2^(e-1) * (1 + m/2); the same value in E4M3
    # (bias 7) has exponent field e + 6 and mantissa m << 2. Decode that byte with torch's
    # float8_e4m3fn (an independent implementation of OCP E4M3) and compare.
    for code in range(16):
        s, e, m = code >> 3, (code >> 1) & 3, code & 1
        if e == 0:
            want = (-1.0 if s else 1.0) * (0.5 if m else 0.0)
        else:
            byte = (s << 7) | ((e + 6) << 3) | (m << 2)
            want = float(torch.tensor([byte], dtype=torch.uint8).view(torch.float8_e4m3fn).float()[0])
        got = F.e2m1_decode(np.array([code]))[0]
        assert got == want and np.signbit(got) == np.signbit(want), code
    assert F.E2M1_TABLE[:8].tolist() == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert np.signbit(F.E2M1_TABLE[8])          # code 0x8 is the FP4 negative zero


def test_e4m3_decode_matches_torch_for_all_bytes():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = F.e4m3_decode(np.arange(256))
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | ((ref == got) & (np.signbit(ref) == np.signbit(got))))
    assert F.E4M3_TABLE[0x7E] == 448.0 and np.isnan(F.E4M3_TABLE[0x7F])
    assert F.E4M3_TABLE[0x01] == 2.0 ** -9 and F.E4M3_TABLE[0x08] == 2.0 ** -6


def test_e4m3_round_matches_torch_cast():
    rng = np.random.default_rng(7)
    # random magnitudes over the whole range, plus every exact midpoint and every grid value
    q = np.concatenate([
        np.exp(rng.uniform(np.log(2.0 ** -11), np.log(448.0), 20000)).astype(np.float32),
        ((F.E4M3_TABLE[:126] + F.E4M3_TABLE[1:127]) / 2).astype(np.float32),
        F.E4M3_TABLE[:127].astype(np.float32),
    ])
    ref = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_round(q.astype(np.float64))
    assert np.array_equal(got, ref)


def test_e4m3_round_saturates():
    assert F.e4m3_round(np.array([448.0, 460.0, 1e6]))[0] == 0x7E
    assert np.all(F.e4m3_round(np.array([460.0, 1e6])) == 0x7E)
    assert F.e4m3_round(np.array([2.0 ** -10]))[0] == 0          # tie between 0 and 2^-9 -> even (0)
    assert F.e4m3_round(np.array([3 * 2.0 ** -10]))[0] == 2      # tie between 1 and 2 (x 2^-9) -> 2


def _nearest_exact(q: Fraction, grid):
    """Brute force: nearest grid value, ties to the even index (grid given as Fractions)."""
    best = None
    for i, g in enumerate(grid):
        d = abs(q - g)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


def test_e2m1_round_tie_table_and_brute_force():
    mids = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for r, code in mids.items():
        assert F.e2m1_round_magnitude(np.array([r]))[0] == code, r
    assert F.e2m1_round_magnitude(np.array([6.0, 7.0, 100.0])).tolist() == [7, 7, 7]
    grid = [Fraction(v) for v in F.E2M1_TABLE[:8]]
    rng = np.random.default_rng(3)
    for _ in range(3000):
        num, den = int(rng.integers(0, 1 << 20)), int(rng.integers(1, 1 << 18))
        q = Fraction(num, den)
        if q > 6:
            continue
        assert F.e2m1_round_magnitude(np.array([float(q)]))[0] == _nearest_exact(q, grid)


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(5000) * 10.0 ** rng.integers(-30, 30, 5000),
                        [0.0, -0.0, 1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 3e38]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    got = F.bf16_round(x.astype(np.float64))
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))


def test_bf16_ulp():
    assert F.bf16_ulp(np.array([1.0]))[0] == 2.0 ** -7
    assert F.bf16_ulp(np.array([3.0]))[0] == 2.0 ** -6
    assert F.bf16_ulp(np.array([0.0]))[0] == 2.0 ** -133
