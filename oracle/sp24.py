"""2:4 structured sparsity along the reduction dimension K (oracle).

The rule: consecutive, non-overlapping groups of four entries along K; a group is eligible
when at least two of its four entries are zero ("Sparse GPU FLOPS Need the Right Zeros in the
Right Places", leviathansystems.co, section "The operation determines which four entries
belong together"; "Myth: 2:4 sparsity doubles your inference throughput", spheron.network,
section "What 2:4 Sparsity Actually Prunes and How the Hardware Exploits It"). The test is made
per group, never as a global zero fraction (same leviathansystems.co page, section "Two
half-zero vectors produce different pattern answers").

Compressed form: the two kept values of each group plus a 2-bit position (0..3) for each
("NVFP4 vs 2:4 sparse", robertz.co, section "What 2:4 actually is" and its figure, where the
group w0 0 0 w3 is stored as w0 w3 with positions 0 and 3). Byte layout (the pages fix the
content, not the bit order):

* vals  [N, K/4]: byte g = code[4g + i0] | code[4g + i1] << 4, with i0 < i1 — so ``vals`` is
  itself an NVFP4 code array of width K/2 (two nibbles per byte, lower position first).
* meta  [N, K/8]: nib(g) = i0 | i1 << 2; byte j = nib(2j) | nib(2j + 1) << 4, so one
  little-endian 32-bit word holds the positions of 8 consecutive groups.
* scales stay [N, K/16] in the original K (prune, then quantise, then compress).

Readings where the pages are silent: a code counts as zero when its magnitude bits are 0, so
the FP4 negative zero (0x8) is a zero; with more than two zeros the kept positions are the
nonzero ones first, then the lowest-index zeros, listed in ascending order (this reproduces the
figure's positions 0 and 3 for w0 0 0 w3); kept codes are stored verbatim (a kept 0x8 stays
0x8); a failing group (fewer than two zeros) is written as vals 0x00 with positions (0, 1) and
counted, so that even a failing call produces well-defined bytes.

Magnitude pruning (keep the two largest |w| of each group, ties to the lower index, others set
to +0.0) is how the synthetic sparse weights are made; it is applied to the float32 weights
before quantisation.
"""
from __future__ import annotations

import numpy as np

from .quant import pack_nibbles, unpack_nibbles

GROUP = 4


def prune24(w: np.ndarray) -> np.ndarray:
    """Keep the 2 largest |w| in every group of 4 along K (ties: lower index wins), zero the rest."""
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    if K % GROUP:
        raise ValueError("K must be a multiple of 4")
    g = w.reshape(N, K // GROUP, GROUP)
    order = np.argsort(-np.abs(g), axis=2, kind="stable")  # stable: equal |w| keeps lower index first
    keep = np.zeros(g.shape, dtype=bool)
    np.put_along_axis(keep, order[:, :, :2], True, axis=2)
    return np.where(keep, g, np.float32(0.0)).reshape(N, K).astype(np.float32)


def _zero_mask(codes: np.ndarray) -> np.ndarray:
    nib = unpack_nibbles(codes)
    N, K = nib.shape
    return ((nib & 0x7) == 0).reshape(N, K // GROUP, GROUP), nib.reshape(N, K // GROUP, GROUP)


def check(codes: np.ndarray):
    """Per-group 2:4 check of NVFP4 codes [N, K/2].

    Returns (bad_groups, first_bad) where first_bad is the smallest flat group index
    n * (K/4) + g of a failing group, or -1 when every group passes.
    """
    zero, _ = _zero_mask(codes)
    bad = zero.sum(axis=2) < 2
    flat = np.flatnonzero(bad.reshape(-1))
    return int(bad.sum()), int(flat[0]) if flat.size else -1


def _select(zero: np.ndarray):
    """Kept positions (i0 < i1) per group and the failure mask."""
    idx = np.arange(GROUP)
    key = zero.astype(np.int64) * GROUP + idx          # nonzero positions first, then zeros, by index
    order = np.argsort(key, axis=2, kind="stable")
    two = np.sort(order[:, :, :2], axis=2)
    fail = zero.sum(axis=2) < 2
    i0 = np.where(fail, 0, two[:, :, 0])
    i1 = np.where(fail, 1, two[:, :, 1])
    return i0, i1, fail


def compress(codes: np.ndarray):
    """Compress NVFP4 codes [N, K/2] (K % 8 == 0) to (vals [N, K/4], meta [N, K/8], bad_groups)."""
    zero, nib = _zero_mask(codes)
    N, G, _ = nib.shape
    if G % 2:
        raise ValueError("K must be a multiple of 8")
    i0, i1, fail = _select(zero)
    c0 = np.take_along_axis(nib, i0[:, :, None], axis=2)[:, :, 0]
    c1 = np.take_along_axis(nib, i1[:, :, None], axis=2)[:, :, 0]
    vals = np.where(fail, 0, c0 | (c1 << 4)).astype(np.uint8)
    pos = (i0 | (i1 << 2)).astype(np.uint8)
    meta = pack_nibbles(pos)
    return vals, meta, int(fail.sum())


def positions(meta: np.ndarray):
    """meta [N, K/8] -> (i0, i1) int arrays [N, K/4]."""
    pos = unpack_nibbles(meta)
    return (pos & 0x3).astype(np.int64), (pos >> 2).astype(np.int64)


def decompress(vals: np.ndarray, meta: np.ndarray) -> np.ndarray:
    """(vals [N, K/4], meta [N, K/8]) -> dense codes [N, K/2]; unselected positions get code 0."""
    vals = np.asarray(vals, dtype=np.uint8)
    N, G = vals.shape
    i0, i1 = positions(meta)
    nib = np.zeros((N, G, GROUP), dtype=np.uint8)
    np.put_along_axis(nib, i0[:, :, None], (vals & 0xF)[:, :, None], axis=2)
    np.put_along_axis(nib, i1[:, :, None], (vals >> 4)[:, :, None], axis=2)
    return pack_nibbles(nib.reshape(N, G * GROUP))
