"""Number formats used by NVFP4 weights: E2M1 values, E4M3 block scales, bf16 activations.

The NVFP4 triplet (4-bit E2M1 values, one FP8 E4M3 scale per 16 values, one FP32 tensor
scale) is named in "NVFP4 Without FP4 Hardware" (ai-muninn.com), section "Convert BF16 to
NVFP4 yourself", and in "NVFP4 vs 2:4 sparse" (robertz.co), section "The byte saving is
about a quarter, not a half" (4 value bits plus an 8-bit scale per 16 = 4.5 bits). The pages
name the formats without printing code tables; the readings here are the OCP ones, which
are the only ones consistent with a largest E2M1 magnitude of 6 and a largest E4M3 value of
448 (the tensor scale is amax / (6 * 448)):

* E2M1 nibble ``s e1 e0 m`` (bit 3 = sign), exponent bias 1, no Inf/NaN. Exponent field 0 is
  subnormal (m * 0.5). Magnitudes by code 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6. Code 8 is -0.
* E4M3 byte ``s eeee mmm``, exponent bias 7, exponent field 0 subnormal (m * 2^-9),
  0x7F / 0xFF are NaN (no Inf), largest finite value 0x7E = 448.

Rounding to either grid is round-to-nearest with ties to the even code, decided on the
exact value passed in. Parity: pinned by exhaustive tables and by library routines (see
the tests); nothing here is parity unpinned.
"""
from __future__ import annotations

import numpy as np


def _e2m1_value(code: int) -> float:
    s = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    mag = m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return s * mag


def _e4m3_value(byte: int) -> float:
    s = -1.0 if byte & 0x80 else 1.0
    e = (byte >> 3) & 0xF
    m = byte & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    mag = m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return s * mag


# decode tables built from the bit fields
E2M1_TABLE = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3_TABLE = np.array([_e4m3_value(b) for b in range(256)], dtype=np.float64)
E2M1_MAX = 6.0
E4M3_MAX = 448.0

# non-negative grids, indexed by code (codes are monotone in value on the positive half)
_E2M1_GRID = E2M1_TABLE[:8].copy()
_E4M3_GRID = E4M3_TABLE[:127].copy()


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """E2M1 nibble (0..15, any integer dtype) -> float64 (code 8 gives -0.0)."""
    return E2M1_TABLE[np.asarray(codes).astype(np.intp) & 0xF]


def e4m3_decode(b: np.ndarray) -> np.ndarray:
    """E4M3 byte -> float64."""
    return E4M3_TABLE[np.asarray(b).astype(np.intp) & 0xFF]


def _round_to_grid(q: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the grid value nearest to q (q >= 0, exact float64), ties to the even index,
    values beyond the last grid point saturate to it."""
    q = np.asarray(q, dtype=np.float64)
    if np.any(q < 0) or np.any(np.isnan(q)):
        raise ValueError("round_to_grid expects non-negative finite inputs")
    n = len(grid)
    hi = np.clip(np.searchsorted(grid, q, side="left"), 0, n - 1)
    lo = np.clip(hi - 1, 0, n - 1)
    mid = (grid[lo] + grid[hi]) / 2.0  # exact: adjacent grid values share a few bits
    pick = np.where(q > mid, hi, np.where(q < mid, lo, np.where(lo % 2 == 0, lo, hi)))
    return pick.astype(np.int64)


def e2m1_round_magnitude(r: np.ndarray) -> np.ndarray:
    """Nearest E2M1 magnitude code (0..7) to r >= 0, ties to even code, saturating at 6."""
    return _round_to_grid(r, _E2M1_GRID)


def e4m3_round(q: np.ndarray) -> np.ndarray:
    """Nearest non-negative E4M3 byte (0x00..0x7E) to q >= 0, ties to even, saturating at 448."""
    return _round_to_grid(np.minimum(np.asarray(q, dtype=np.float64), E4M3_MAX), _E4M3_GRID)


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def bf16_round(y: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (8 significant bits, ties to even);
    returns float64 holding the rounded values. Overflow gives +-inf."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    out = np.zeros_like(a)
    nz = a > 0
    _, ex = np.frexp(a[nz])               # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -126)          # unbiased exponent, clamped to the subnormal floor
    quantum = np.ldexp(1.0, e - 7)
    out[nz] = np.rint(a[nz] / quantum) * quantum   # rint = round half to even
    out[out > 3.3895313892515355e38] = np.inf
    return np.copysign(out, y)


def bf16_ulp(y: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |y| (float64)."""
    a = np.abs(np.asarray(y, dtype=np.float64))
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.where(a > 0, np.maximum(ex - 1, -126), -126)
    return np.ldexp(1.0, e - 7)
